"""GPU parity of the first-token extras: pe_varlen_attn_fwd_first_row (query
gather fused into the kernel) and pe_varlen_attn_bwd_first_token (the readout's
backward) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, check_out, from_dev, say, to_dev, to_f64
from tests.test_gpu_bwd import check_grad

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")

EDGE = [1, 127, 128, 129, 5, 256, 257, 3, 300, 64, 65, 1, 1, 2, 31, 32, 33, 16, 15, 17, 200]


def first_fwd_bwd(w: W.Workload, seqs_dout):
    """GPU first-token forward (fused gather) and backward; dout_first = dout rows cu[:-1]."""
    cu_ref, _, N = oracle.layout(w.lengths, w.max_seq_len)
    cu = torch.from_numpy(cu_ref).to(DEV)
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    B, H, d = w.num_seqs, w.num_heads, w.head_dim
    first = torch.from_numpy(cu_ref[:-1].astype(np.int64)).to(DEV)
    out_f = torch.full((B, H, d), float("nan"), device=DEV).to(q.dtype)
    lse_f = torch.full((H, B), float("nan"), device=DEV)
    pe.pe_varlen_attn_fwd_first_row(q, k, v, cu, B, N, w.max_seq_len, w.scale, out_f, lse_f)
    dof = to_dev(seqs_dout, w.dtype)
    qf = q[first].contiguous()
    dqf = torch.full_like(qf, float("nan"))
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    pe.pe_varlen_attn_bwd_first_token(dof, qf, k, v, out_f, lse_f, cu, B, N, w.max_seq_len, w.scale, dqf, dk, dv)
    torch.cuda.synchronize()
    return cu_ref, q, k, v, cu, qf, out_f, lse_f, dqf, dk, dv


def check_first_bwd(w: W.Workload, label: str):
    say(f"[first bwd] {label}: B={w.num_seqs} N={w.total_tokens} H={w.num_heads} d={w.head_dim} {w.dtype}")
    cu_ref, _, N = oracle.layout(w.lengths, w.max_seq_len)
    dof_bits = w.dout[cu_ref[:-1]]
    cu_ref, q, k, v, cu, qf, out_f, lse_f, dqf, dk, dv = first_fwd_bwd(w, dof_bits)
    qd, kd, vd = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v))
    qf64, dof64 = qd[cu_ref[:-1]], W.to_f64(dof_bits, w.dtype)
    o_ref, l_ref = oracle.attention_first_token(qf64, kd, vd, cu_ref, w.scale)
    out_given = o_ref
    if w.dtype == W.BF16:  # the output the forward contract delivers: the exact one rounded to bf16
        out_given = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_ref.astype(np.float32))).astype(np.float64)
    ref = oracle.attention_first_token_backward(dof64, qf64, kd, vd, cu_ref, w.scale, out_first=out_given,
                                                lse_first=l_ref)
    for name, g, r in zip(("dq_first", "dk", "dv"), (dqf, dk, dv), ref):
        check_grad(to_f64(g), r, w.dtype, f"{label} {name}")


@pytest.mark.parametrize("dtype", [W.FP32, W.BF16])
@pytest.mark.parametrize("d", list(range(8, 129, 8)))
def test_first_token_backward_edge_lengths(dtype, d):
    check_first_bwd(W.custom(80 + d, EDGE, 300, 3, d, dtype, with_grad=True), f"edge d={d}")


def test_first_token_backward_many_heads():
    # 24 heads x 128: more than one head group per sequence
    check_first_bwd(W.custom(81, EDGE[:10], 300, 24, 128, W.BF16, with_grad=True), "24 heads")


def test_first_row_equals_gathered_first_token_bitwise():
    w = W.custom(82, EDGE, 300, 3, 64, W.BF16)
    cu_ref, _, N = oracle.layout(w.lengths, w.max_seq_len)
    cu = torch.from_numpy(cu_ref).to(DEV)
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    B = w.num_seqs
    qf = q[torch.from_numpy(cu_ref[:-1].astype(np.int64)).to(DEV)].contiguous()
    o1, o2 = torch.empty_like(qf), torch.empty_like(qf)
    l1, l2 = torch.empty(3, B, device=DEV), torch.empty(3, B, device=DEV)
    pe.pe_varlen_attn_fwd_first_token(qf, k, v, cu, B, N, w.max_seq_len, w.scale, o1, l1)
    pe.pe_varlen_attn_fwd_first_row(q, k, v, cu, B, N, w.max_seq_len, w.scale, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_graph_transformer_first_token_backward_sampled():
    w = W.graph_transformer(grid=False, with_grad=True)
    say(f"[first bwd] graph-transformer full size: B={w.num_seqs} N={w.total_tokens}")
    cu_ref, _, N = oracle.layout(w.lengths, w.max_seq_len)
    dof_bits = w.dout[cu_ref[:-1]]
    cu_ref, q, k, v, cu, qf, out_f, lse_f, dqf, dk, dv = first_fwd_bwd(w, dof_bits)
    seqs = sorted(set(range(0, w.num_seqs, 97)) | {w.num_seqs - 1})
    gdk, gdv, gdq = from_dev(dk), from_dev(dv), from_dev(dqf)
    assert not np.isnan(gdk).any() and not np.isnan(gdv).any() and not np.isnan(gdq).any()
    qd, kd, vd = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v))
    for b in seqs:
        c0, c1 = int(cu_ref[b]), int(cu_ref[b + 1])
        cu_b = np.array([0, c1 - c0], dtype=np.int32)
        qb, kb, vb = qd[c0:c0 + 1], kd[c0:c1], vd[c0:c1]
        dob = W.to_f64(dof_bits[b:b + 1], w.dtype)
        ref = oracle.attention_first_token_backward(dob, qb, kb, vb, cu_b, w.scale)
        check_grad(gdq[b:b + 1].astype(np.float64), ref[0], w.dtype, f"gt seq {b} dq_first")
        check_grad(gdk[c0:c1].astype(np.float64), ref[1], w.dtype, f"gt seq {b} dk")
        check_grad(gdv[c0:c1].astype(np.float64), ref[2], w.dtype, f"gt seq {b} dv")


def test_mixed_training_first_token_backward_sampled():
    """Full-size mixed batch (bf16, 16 heads, documents up to 8192 tokens): the length
    bound gives each block 32 key slots, so a long document is spread over many slots.
    The longest documents and a spread of others are checked against the oracle."""
    w = W.mixed_training()
    say(f"[first bwd] mixed-training full size: B={w.num_seqs} N={w.total_tokens}")
    cu_ref, _, N = oracle.layout(w.lengths, w.max_seq_len)
    dof_bits = w.dout[cu_ref[:-1]]
    cu_ref, q, k, v, cu, qf, out_f, lse_f, dqf, dk, dv = first_fwd_bwd(w, dof_bits)
    L = np.diff(cu_ref)
    seqs = sorted(set(np.argsort(L)[-4:].tolist()) | set(range(0, w.num_seqs, 211)))
    gdk, gdv, gdq = to_f64(dk), to_f64(dv), to_f64(dqf)
    qd, kd, vd = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v))
    for b in seqs:
        c0, c1 = int(cu_ref[b]), int(cu_ref[b + 1])
        cu_b = np.array([0, c1 - c0], dtype=np.int32)
        qb, kb, vb = qd[c0:c0 + 1], kd[c0:c1], vd[c0:c1]
        dob = W.to_f64(dof_bits[b:b + 1], w.dtype)
        o_ref, l_ref = oracle.attention_first_token(qb, kb, vb, cu_b, w.scale)
        given = W.to_f64(W.to_bits(o_ref.astype(np.float32), w.dtype), w.dtype)
        check_out(to_f64(out_f)[b:b + 1], o_ref, w.dtype, f"mt seq {b} out_first")
        ref = oracle.attention_first_token_backward(dob, qb, kb, vb, cu_b, w.scale, out_first=given, lse_first=l_ref)
        check_grad(gdq[b:b + 1], ref[0], w.dtype, f"mt seq {b} dq_first")
        check_grad(gdk[c0:c1], ref[1], w.dtype, f"mt seq {b} dk")
        check_grad(gdv[c0:c1], ref[2], w.dtype, f"mt seq {b} dv")
