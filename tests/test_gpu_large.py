"""Packed tensors of more than 2^31 elements: pack, forward, first-token forward
and backward, backward and unpack on one buffer whose element offsets pass
2^31, so any offset formed in 32 bits would land on the wrong row.

Only three sequences carry random data (the first, the one holding element
2^31 of a row-major [N, H*d] tensor, and the last); they are checked against
the fp64 oracle run on each sequence alone. Every other sequence is all zeros,
which fixes its results in closed form at any size: the scores are 0, so each
row's log-sum-exp is ln(L) of its sequence and its output is 0; with dO = 0
every gradient row is exactly 0. Pack and unpack are checked bit for bit
against the oracle's flat_index over the whole buffer."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, check_lse, check_out, say, to_f64
from tests.test_gpu_bwd import check_grad

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")

TORCH = {W.FP32: torch.float32, W.BF16: torch.bfloat16}
# (heads, head_dim, sequences): rows of 1024 bf16 or 512 fp32 elements, lengths 900..1100
CASES = {W.BF16: (16, 64, 2200), W.FP32: (8, 64, 4400)}


def _values(rng, shape, dtype):
    """Seeded N(0, 1) values, already representable in the element type (float32 array)."""
    x = rng.standard_normal(shape).astype(np.float32)
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)) if dtype == W.BF16 else x


def _row_max(t: torch.Tensor) -> torch.Tensor:
    """max |x| per row (NaN propagates), without a full-size temporary."""
    return torch.linalg.vector_norm(t.view(t.shape[0], -1), ord=float("inf"), dim=1)


def _dev(x: np.ndarray, dtype):
    return torch.from_numpy(x).to(DEV).to(TORCH[dtype])


@pytest.mark.parametrize("dtype", [W.BF16, W.FP32])
def test_tensors_past_two_to_the_31_elements(dtype):
    H, d, B = CASES[dtype]
    ld = H * d
    rng = np.random.default_rng(90 + ld)
    lengths = rng.integers(900, 1101, size=B).astype(np.int32)
    S = int(lengths.max())
    cu_ref, flat_ref, N = oracle.layout(lengths, S)
    assert N * ld > 2 ** 31
    row_x = 2 ** 31 // ld
    checked = [0, int(np.searchsorted(cu_ref, row_x, side="right")) - 1, B - 1]
    say(f"[large] {dtype}: B={B} N={N} H={H} d={d}, {N * ld / 2 ** 31:.2f} x 2^31 elements, seqs {checked}")
    scale = 1.0 / np.sqrt(d)
    dt = TORCH[dtype]

    # inputs: zeros except the checked sequences; Q goes through pe_pack from a padded grid
    data = {}
    for b in checked:
        L = int(lengths[b])
        data[b] = {n: _values(rng, (L, H, d), dtype) for n in ("q", "k", "v", "do")}
    grid = torch.zeros(B, S, ld, dtype=dt, device=DEV)
    k, v, do = (torch.zeros(N, H, d, dtype=dt, device=DEV) for _ in range(3))
    for b in checked:
        c0, c1 = int(cu_ref[b]), int(cu_ref[b + 1])
        grid[b, : c1 - c0] = _dev(data[b]["q"].reshape(c1 - c0, ld), dtype)
        k[c0:c1], v[c0:c1], do[c0:c1] = (_dev(data[b][n], dtype) for n in ("k", "v", "do"))

    # pack: cu_seqlens and flat_index exact, packed rows bit-exact copies of the grid rows
    lens = torch.from_numpy(lengths).to(DEV)
    ws = pe.workspace(pe.pe_pack_workspace_size(B, S, ld, pe.PE_BF16 if dtype == W.BF16 else pe.PE_FP32), DEV)
    cu = torch.empty(B + 1, dtype=torch.int32, device=DEV)
    flat = torch.empty(N, dtype=torch.int64, device=DEV)
    q = torch.empty(N, H, d, dtype=dt, device=DEV)
    assert pe.pe_pack(lens, S, grid, cu, flat, q, N, ws) == N
    torch.cuda.synchronize()
    assert np.array_equal(cu.cpu().numpy(), cu_ref)
    assert np.array_equal(flat.cpu().numpy(), flat_ref)
    assert torch.equal(q.view(N, ld).view(torch.int16 if dtype == W.BF16 else torch.int32),
                       grid.view(B * S, ld)[flat].view(torch.int16 if dtype == W.BF16 else torch.int32))
    del grid
    torch.cuda.empty_cache()

    # forward
    code = pe.PE_BF16 if dtype == W.BF16 else pe.PE_FP32
    aws = pe.workspace(pe.pe_attn_workspace_size(B, N, H, d, code, True), DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((H, N), float("nan"), device=DEV)
    pe.pe_varlen_attn_fwd(q, k, v, cu, B, N, S, scale, out, lse, aws)
    # first-token forward on the first rows
    q_first = q[torch.from_numpy(cu_ref[:-1].astype(np.int64)).to(DEV)].contiguous()
    out_f = torch.full_like(q_first, float("nan"))
    lse_f = torch.full((H, B), float("nan"), device=DEV)
    pe.pe_varlen_attn_fwd_first_token(q_first, k, v, cu, B, N, S, scale, out_f, lse_f)
    # backward
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    pe.pe_varlen_attn_bwd(do, q, k, v, out, lse, cu, B, N, S, scale, dq, dk, dv, aws)
    torch.cuda.synchronize()

    mine = torch.zeros(N, dtype=torch.bool, device=DEV)
    for b in checked:
        mine[int(cu_ref[b]):int(cu_ref[b + 1])] = True
    seq_len = torch.from_numpy(np.repeat(lengths, lengths).astype(np.float64)).to(DEV)
    # zero sequences in closed form
    rest = ~mine
    for name, t in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert (_row_max(t)[rest] == 0).all(), f"{name}: a zero sequence has a nonzero row"
    lse_err = (lse[:, rest].double() - torch.log(seq_len[rest])[None, :]).abs().max().item()
    assert lse_err <= 1e-5 * np.log(1101.0), f"lse of zero sequences off by {lse_err:.3e}"
    fz = torch.from_numpy(np.setdiff1d(np.arange(B), checked)).to(DEV)
    assert (_row_max(out_f)[fz] == 0).all()
    assert ((lse_f[:, fz].double() - torch.log(torch.from_numpy(lengths.astype(np.float64)).to(DEV)[fz])[None, :])
            .abs().max().item() <= 1e-5 * np.log(1101.0))

    # checked sequences against the oracle
    for b in checked:
        c0, c1 = int(cu_ref[b]), int(cu_ref[b + 1])
        L = c1 - c0
        q64, k64, v64, do64 = (data[b][n].astype(np.float64) for n in ("q", "k", "v", "do"))
        cu1 = np.array([0, L], dtype=np.int32)
        o_ref, l_ref = oracle.attention(q64, k64, v64, cu1, scale)
        check_out(to_f64(out[c0:c1].cpu()), o_ref, dtype, f"seq {b} out")
        check_lse(lse[:, c0:c1].cpu().numpy().astype(np.float64), l_ref, dtype, f"seq {b} lse")
        check_out(to_f64(out_f[b:b + 1].cpu()), o_ref[:1], dtype, f"seq {b} first-token out")
        check_lse(lse_f[:, b:b + 1].cpu().numpy().astype(np.float64), l_ref[:, :1], dtype, f"seq {b} first-token lse")
        out_given = None
        if dtype == W.BF16:
            out_given = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_ref.astype(np.float32))).astype(np.float64)
        ref = oracle.attention_backward(do64, q64, k64, v64, cu1, scale, out=out_given)
        for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            check_grad(to_f64(g[c0:c1].cpu()), r, dtype, f"seq {b} {name}")
    del dq, dk, dv, do

    # first-token backward: dO on the first rows of the checked sequences only
    do_f = torch.zeros_like(q_first)
    for b in checked:
        do_f[b] = _dev(data[b]["do"][:1].reshape(H, d), dtype)
    dq_f = torch.full_like(q_first, float("nan"))
    dk, dv = (torch.full_like(q, float("nan")) for _ in range(2))
    pe.pe_varlen_attn_bwd_first_token(do_f, q_first, k, v, out_f, lse_f, cu, B, N, S, scale, dq_f, dk, dv)
    torch.cuda.synchronize()
    assert (_row_max(dk)[rest] == 0).all() and (_row_max(dv)[rest] == 0).all() and (_row_max(dq_f)[fz] == 0).all()
    for b in checked:
        c0, c1 = int(cu_ref[b]), int(cu_ref[b + 1])
        L = c1 - c0
        q64, k64, v64, do64 = (data[b][n].astype(np.float64) for n in ("q", "k", "v", "do"))
        cu1 = np.array([0, L], dtype=np.int32)
        o_ref, l_ref = oracle.attention_first_token(q64[:1], k64, v64, cu1, scale)
        if dtype == W.BF16:  # the output the forward contract delivers: the exact one rounded to bf16
            o_ref = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_ref.astype(np.float32))).astype(np.float64)
        rq, rk, rv = oracle.attention_first_token_backward(do64[:1], q64[:1], k64, v64, cu1, scale,
                                                           out_first=o_ref, lse_first=l_ref)
        check_grad(to_f64(dq_f[b:b + 1].cpu()), rq, dtype, f"seq {b} first-token dq")
        check_grad(to_f64(dk[c0:c1].cpu()), rk, dtype, f"seq {b} first-token dk")
        check_grad(to_f64(dv[c0:c1].cpu()), rv, dtype, f"seq {b} first-token dv")
    del dk, dv
    torch.cuda.empty_cache()

    # unpack: real rows bit-exact at flat_index, padding rows +0.0
    grid_out = torch.full((B, S, ld), float("nan"), dtype=dt, device=DEV)
    pe.pe_unpack(out, cu, B, S, N, grid_out)
    torch.cuda.synchronize()
    iv = torch.int16 if dtype == W.BF16 else torch.int32
    want = torch.zeros(B * S, ld, dtype=iv, device=DEV)
    want[flat] = out.view(N, ld).view(iv)
    assert torch.equal(grid_out.view(B * S, ld).view(iv), want)
