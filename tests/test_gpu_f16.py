"""GPU parity of the fp16 element type against the fp64 oracle, over every
kernel family: the generic forward (short length bounds, every head dim), the
LDS-DMA forwards on sequence-aligned tiles (long bounds), local attention, the
first-token forward (given rows and gathered rows), the backward (swizzled and
plain tiles), the first-token backward, the fused-QKV calls (bit-exact against
separate tensors), pack/unpack (bit-exact) and the captured bucket forward.

fp16 is held to the bf16 bar of tests/gpu_util.py (16-bit inputs, fp32
accumulation); reference gradients are evaluated at the oracle's output rounded
to fp16, the output the forward contract delivers."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, check_lse, check_out, from_dev, say, to_dev, to_f64
from tests.test_gpu_bwd import check_grad

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")
graphs = pytest.importorskip("padding_free_packed_amd.graphs")

F16 = W.FP16
EDGE = [1, 127, 128, 129, 5, 256, 257, 3, 300, 64, 65, 1, 1, 2, 31, 32, 33, 16, 15, 17, 200]


def _bits(t):
    return t.view(torch.int16)


def _fwd(w, window=None):
    cu_ref, _, N = oracle.layout(w.lengths, w.max_seq_len)
    cu = torch.from_numpy(cu_ref).to(DEV)
    q, k, v = (to_dev(x, F16) for x in (w.q, w.k, w.v))
    assert q.dtype == torch.float16
    ws = pe.workspace(pe.pe_attn_workspace_size(w.num_seqs, N, w.num_heads, w.head_dim, pe.PE_FP16, True), DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((w.num_heads, N), float("nan"), device=DEV)
    if window is None:
        pe.pe_varlen_attn_fwd(q, k, v, cu, w.num_seqs, N, w.max_seq_len, w.scale, out, lse, ws)
    else:
        pe.pe_varlen_attn_fwd_local(q, k, v, cu, w.num_seqs, N, w.max_seq_len, w.scale, window, out, lse, ws)
    return cu_ref, cu, (q, k, v), out, lse, ws


@pytest.mark.parametrize("d,S", [(8, 64), (16, 64), (32, 64), (64, 64), (128, 64), (32, 300), (64, 300),
                                 (128, 300), (16, 300), (24, 300), (40, 64), (96, 300), (120, 300)])
def test_forward(d, S):
    w = W.custom(300 + d + S, np.minimum(EDGE, S), S, 2, d, F16)
    say(f"[f16 fwd] d={d} S={S} N={w.total_tokens}")
    cu_ref, _, _, out, lse, _ = _fwd(w)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(*(W.to_f64(x, F16) for x in (w.q, w.k, w.v)), cu_ref, w.scale)
    check_out(to_f64(out), o_ref, F16, "f16 out")
    check_lse(to_f64(lse), l_ref, F16, "f16 lse")


def test_forward_long_sequences_and_large_scores():
    """Long sequences through the sequence-aligned tile kernel, with scores far above the
    rescale headroom (scale 1): the running maximum moves many times."""
    L = np.array([3000, 1, 2047, 640], dtype=np.int32)
    w = W.custom(41, L, 4096, 4, 64, F16, scale=1.0)
    say(f"[f16 fwd] long, scale 1: N={w.total_tokens}")
    cu_ref, _, _, out, lse, _ = _fwd(w)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(*(W.to_f64(x, F16) for x in (w.q, w.k, w.v)), cu_ref, w.scale)
    check_out(to_f64(out), o_ref, F16, "f16 long out")
    check_lse(to_f64(lse), l_ref, F16, "f16 long lse")


@pytest.mark.parametrize("window", [None, 100])
@pytest.mark.parametrize("d", [32, 64])
def test_forward_probability_near_fp16_max(d, window):
    """A key block after the first whose one large score sits just under 16
    (log2 units) above the first block's maximum, the rest of its scores far
    below: its unnormalised probability, about 65529, is finite in fp32 but
    rounds to infinity in fp16 (largest finite value 65504), so the forward
    must take a new reference before that block's probabilities enter the
    fp16 product. Query rows are e0; keys 0..31 are zero (scores 0), key 32
    is e0 (score 1), every later key is -8 e0; scale * log2(e) = 15.99985."""
    L, H = 200, 2
    w = W.custom(330 + d, np.array([L], dtype=np.int32), L, H, d, F16, scale=11.090250968933105)
    c = float(np.float32(w.scale * 1.4426950408889634))
    assert 65520.0 < 2.0 ** c < 65536.0  # rounds to fp16 infinity (halfway above 65504 is 65520)
    q = np.zeros((L, H, d), np.float32)
    q[:, :, 0] = 1.0
    k = np.zeros((L, H, d), np.float32)
    k[32, :, 0] = 1.0
    k[33:, :, 0] = -8.0
    w.q, w.k = (x.astype(np.float16).view(np.uint16) for x in (q, k))
    say(f"[f16 fwd] p near the fp16 maximum: d={d} L={L} window={window}")
    cu_ref, _, _, out, lse, _ = _fwd(w, window)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(*(W.to_f64(x, F16) for x in (w.q, w.k, w.v)), cu_ref, w.scale, window=window)
    check_out(to_f64(out), o_ref, F16, "f16 out, p near 65504")
    check_lse(to_f64(lse), l_ref, F16, "f16 lse, p near 65504")


@pytest.mark.parametrize("d,S,window", [(64, 300, 20), (32, 300, 40), (128, 300, 0), (16, 64, 5), (32, 48, 7),
                                         (64, 64, 0)])
def test_local_forward_and_backward(d, S, window):
    w = W.custom(310 + d, np.minimum(EDGE, S), S, 2, d, F16, with_grad=True)
    say(f"[f16 local] d={d} S={S} window={window}")
    cu_ref, cu, (q, k, v), out, lse, ws = _fwd(w, window)
    do = to_dev(w.dout, F16)
    N = w.total_tokens
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    pe.pe_varlen_attn_bwd_local(do, q, k, v, out, lse, cu, w.num_seqs, N, S, w.scale, window, dq, dk, dv, ws)
    torch.cuda.synchronize()
    qd, kd, vd, dod = (W.to_f64(x, F16) for x in (w.q, w.k, w.v, w.dout))
    o_ref, l_ref = oracle.attention(qd, kd, vd, cu_ref, w.scale, window=window)
    check_out(to_f64(out), o_ref, F16, "f16 local out")
    check_lse(to_f64(lse), l_ref, F16, "f16 local lse")
    given = W.to_f64(W.to_bits(o_ref.astype(np.float32), F16), F16)
    ref = oracle.attention_backward(dod, qd, kd, vd, cu_ref, w.scale, out=given, window=window)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grad(to_f64(g), r, F16, f"f16 local {name}")


@pytest.mark.parametrize("d,S", [(16, 64), (64, 64), (64, 300), (128, 300), (8, 40), (24, 300), (72, 64), (120, 300)])
def test_backward(d, S):
    w = W.custom(320 + d + S, np.minimum(EDGE, S), S, 2, d, F16, with_grad=True)
    say(f"[f16 bwd] d={d} S={S}")
    cu_ref, cu, (q, k, v), out, lse, ws = _fwd(w)
    do = to_dev(w.dout, F16)
    N = w.total_tokens
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    pe.pe_varlen_attn_bwd(do, q, k, v, out, lse, cu, w.num_seqs, N, S, w.scale, dq, dk, dv, ws)
    torch.cuda.synchronize()
    qd, kd, vd, dod = (W.to_f64(x, F16) for x in (w.q, w.k, w.v, w.dout))
    o_ref, _ = oracle.attention(qd, kd, vd, cu_ref, w.scale)
    given = W.to_f64(W.to_bits(o_ref.astype(np.float32), F16), F16)
    ref = oracle.attention_backward(dod, qd, kd, vd, cu_ref, w.scale, out=given)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grad(to_f64(g), r, F16, f"f16 {name}")


@pytest.mark.parametrize("d", [8, 64, 128])
def test_first_token_forward_and_backward(d):
    S = 300
    w = W.custom(330 + d, np.minimum(EDGE, S), S, 3, d, F16, with_grad=True)
    say(f"[f16 first] d={d}")
    cu_ref, _, N = oracle.layout(w.lengths, S)
    cu = torch.from_numpy(cu_ref).to(DEV)
    q, k, v, do = (to_dev(x, F16) for x in (w.q, w.k, w.v, w.dout))
    B, H = w.num_seqs, w.num_heads
    first = torch.from_numpy(cu_ref[:-1].astype(np.int64)).to(DEV)
    qf, dof = q[first].contiguous(), do[first].contiguous()
    of, lf = torch.full_like(qf, float("nan")), torch.full((H, B), float("nan"), device=DEV)
    pe.pe_varlen_attn_fwd_first_token(qf, k, v, cu, B, N, S, w.scale, of, lf)
    og, lg = torch.full_like(qf, float("nan")), torch.full((H, B), float("nan"), device=DEV)
    pe.pe_varlen_attn_fwd_first_row(q, k, v, cu, B, N, S, w.scale, og, lg)
    dqf, dk, dv = torch.full_like(qf, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    pe.pe_varlen_attn_bwd_first_token(dof, qf, k, v, of, lf, cu, B, N, S, w.scale, dqf, dk, dv)
    torch.cuda.synchronize()
    assert torch.equal(_bits(of), _bits(og)) and torch.equal(lf, lg)
    qd, kd, vd, dod = (W.to_f64(x, F16) for x in (w.q, w.k, w.v, w.dout))
    o_ref, l_ref = oracle.attention_first_token(qd[cu_ref[:-1]], kd, vd, cu_ref, w.scale)
    check_out(to_f64(of), o_ref, F16, "f16 first out")
    check_lse(to_f64(lf), l_ref, F16, "f16 first lse")
    given = W.to_f64(W.to_bits(o_ref.astype(np.float32), F16), F16)
    ref = oracle.attention_first_token_backward(dod[cu_ref[:-1]], qd[cu_ref[:-1]], kd, vd, cu_ref, w.scale,
                                                out_first=given)
    for name, g, r in zip(("dq_first", "dk", "dv"), (dqf, dk, dv), ref):
        check_grad(to_f64(g), r, F16, f"f16 first {name}")


@pytest.mark.parametrize("d,S", [(64, 300), (64, 64), (128, 300)])
def test_fused_qkv_matches_separate_tensors(d, S):
    w = W.custom(340 + d + S, np.minimum(EDGE, S), S, 2, d, F16, with_grad=True)
    say(f"[f16 qkv] d={d} S={S}")
    cu_ref, cu, (q, k, v), out, lse, ws = _fwd(w)
    do = to_dev(w.dout, F16)
    N, B = w.total_tokens, w.num_seqs
    g = [torch.empty_like(q) for _ in range(3)]
    pe.pe_varlen_attn_bwd(do, q, k, v, out, lse, cu, B, N, S, w.scale, *g, ws)
    qkv = torch.stack([q, k, v], dim=1).contiguous()
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    pe.pe_varlen_attn_fwd_qkv(qkv, cu, B, N, S, w.scale, -1, out2, lse2, ws)
    dqkv = torch.full_like(qkv, float("nan"))
    pe.pe_varlen_attn_bwd_qkv(do, qkv, out2, lse2, cu, B, N, S, w.scale, -1, dqkv, ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(out2)) and torch.equal(lse, lse2)
    for i in range(3):
        assert torch.equal(_bits(dqkv[:, i].contiguous()), _bits(g[i])), i


def test_pack_unpack_bit_exact():
    w = W.custom(350, W.random_lengths(351, 700, 1, 48), 48, 12, 64, F16)
    B, S, D = w.num_seqs, w.max_seq_len, w.row_elems
    rng = np.random.default_rng(352)
    grid_np = W.to_bits(rng.standard_normal((B, S, D), dtype=np.float32), F16)
    grid_np[np.arange(S)[None, :] >= w.lengths[:, None]] = W.FP16_NAN
    cu_ref, flat_ref, N = oracle.layout(w.lengths, S)
    grid = to_dev(grid_np, F16)
    cu, flat, packed, n = pe.pack(torch.from_numpy(w.lengths).to(DEV), S, grid)
    out = torch.full_like(grid, float("nan"))
    pe.pe_unpack(packed, cu, B, S, n, out)
    torch.cuda.synchronize()
    assert n == N
    np.testing.assert_array_equal(from_dev(packed), oracle.pack(grid_np, flat_ref))
    np.testing.assert_array_equal(from_dev(out), oracle.unpack(oracle.pack(grid_np, flat_ref), cu_ref, S))


def test_bucket_graph():
    slots, S, H, d = 64, 48, 12, 64
    scale = 0.125
    bucket = graphs.ForwardBucket(slots, S, H, d, torch.float16, scale, -1, with_lse=True, device=DEV)
    rng = np.random.default_rng(353)
    try:
        for B in (64, 20):
            L = rng.integers(8, S + 1, size=B).astype(np.int32)
            xq = W.to_bits(rng.standard_normal((B, S, 3, H, d), dtype=np.float32), F16)
            say(f"[f16 graph] B={B}")
            got = bucket.run(torch.from_numpy(L).to(DEV), to_dev(xq, F16))
            torch.cuda.synchronize()
            cu_ref = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
            assert bucket.status.tolist() == [int(bucket.lengths.sum()), pe.PACK_OK]
            rows = [W.to_f64(np.concatenate([xq[b, :L[b], j] for b in range(B)]), F16) for j in range(3)]
            o_ref, l_ref = oracle.attention(*rows, cu_ref, scale)
            check_out(to_f64(torch.cat([got[b, :L[b]] for b in range(B)])), o_ref, F16, "f16 graph out")
            check_lse(to_f64(bucket.lse[:, :int(cu_ref[-1])]), l_ref, F16, "f16 graph lse")
    finally:
        bucket.close()
