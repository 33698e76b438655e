"""GPU parity of pe_varlen_attn_bwd against the fp64 oracle.

The GPU backward takes the GPU forward's output and log-sum-exp, as a training
step does; the oracle recomputes everything in float64 from the same inputs.
Gradients use the tolerances of tests/gpu_util.py, except that bf16 gradients
may also differ by the rounding of the bf16 output itself (2^-8 of the value),
see check_grad."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, check_out, from_dev, min_cosine, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")


def check_grad(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    if dtype == W.FP32:
        return check_out(gpu, ref, dtype, what)
    # bf16: |err| <= 2e-2 + 2^-8 |ref| (the output rounding to bf16 alone reaches 2^-8 |ref|),
    # and per-token cosine >= 0.999
    assert np.isfinite(gpu).all(), f"{what}: non-finite"
    err = np.abs(gpu - ref)
    bound = 2e-2 + np.abs(ref) / 256.0
    assert (err <= bound).all(), f"{what}: max excess {(err - bound).max():.3e}, max err {err.max():.3e}"
    cos, i, nrm, e = min_cosine(gpu.reshape(gpu.shape[0], -1), ref.reshape(ref.shape[0], -1), where=True)
    assert cos >= 0.999, f"{what}: min per-token cosine {cos:.6f} at row {i} (ref norm {nrm:.4g}, max err {e:.3g})"
    return float(err.max())


def gpu_fwd_bwd(w: W.Workload, full_workspace: bool = True):
    """Forward then backward on the GPU. full_workspace: the workspace of pe_attn_bwd_workspace_size
    (fp32 at d 32/64: dS handed from the dK/dV pass to the dQ pass), else the smaller one of
    pe_attn_workspace_size (dQ recomputes S and dP)."""
    cu_ref, _, N = oracle.layout(w.lengths, w.max_seq_len)
    cu = torch.from_numpy(cu_ref).to(DEV)
    q, k, v, do = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v, w.dout))
    code = pe.PE_BF16 if w.dtype == W.BF16 else pe.PE_FP32
    size = (pe.pe_attn_bwd_workspace_size(w.num_seqs, N, w.max_seq_len, w.num_heads, w.head_dim, code)
            if full_workspace else pe.pe_attn_workspace_size(w.num_seqs, N, w.num_heads, w.head_dim, code, True))
    ws = pe.workspace(size, DEV)
    out = torch.empty_like(q)
    lse = torch.empty(w.num_heads, N, device=DEV)
    pe.pe_varlen_attn_fwd(q, k, v, cu, w.num_seqs, N, w.max_seq_len, w.scale, out, lse, ws)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    pe.pe_varlen_attn_bwd(do, q, k, v, out, lse, cu, w.num_seqs, N, w.max_seq_len, w.scale, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return cu_ref, dq, dk, dv


def check_bwd(w: W.Workload, label: str, seqs=None, full_workspace: bool = True):
    """The backward op takes the forward's output as an input (its D term is
    <dO, out>). For bf16 the reference is therefore evaluated at the output the
    forward contract delivers: the oracle's own output rounded to bf16 (nearest
    even). fp32 compares against the exact gradient."""
    say(f"[bwd] {label}: B={w.num_seqs} N={w.total_tokens} H={w.num_heads} d={w.head_dim} {w.dtype}")
    cu_ref, dq, dk, dv = gpu_fwd_bwd(w, full_workspace)
    q, k, v, do = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v, w.dout))
    if seqs is None:
        rows = np.arange(int(cu_ref[-1]))
    else:
        rows = np.concatenate([np.arange(cu_ref[b], cu_ref[b + 1]) for b in seqs])
    out_given = None
    if w.dtype == W.BF16:
        o_rows, _ = oracle.attention_rows(q, k, v, cu_ref, w.scale, rows)
        out_given = np.zeros_like(q)
        out_given[rows] = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_rows.astype(np.float32))).astype(np.float64)
    ref = oracle.attention_backward(do, q, k, v, cu_ref, w.scale, seqs, out=out_given)
    for name, gtens, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grad(to_f64(gtens)[rows], r[rows], w.dtype, f"{label} {name}")
    return cu_ref, dq, dk, dv


def test_tiny():
    check_bwd(W.tiny(), "tiny")


def test_gigl_example():
    check_bwd(W.custom(5, [3, 1, 2], 3, 2, 8, W.FP32, with_grad=True), "gigl example")


EDGE = [1, 127, 128, 129, 5, 256, 257, 3, 300, 64, 65, 1, 1, 2, 31, 32, 33, 16, 15, 17, 200]


@pytest.mark.parametrize("dtype", [W.FP32, W.BF16])
@pytest.mark.parametrize("d", list(range(8, 129, 8)))
def test_edge_lengths(dtype, d):
    check_bwd(W.custom(60 + d, EDGE, 300, 3, d, dtype, with_grad=True), f"edge lengths d={d}")


@pytest.mark.parametrize("d,S", [(32, 256), (64, 256), (64, 64), (32, 40)])
def test_fp32_ds_handoff_edge_lengths(d, S):
    """fp32 global attention with the workspace of pe_attn_bwd_workspace_size (length bounds up
    to 256): the dK/dV pass stores every 32x32 dS block and the dQ pass reads them back; lengths
    at the bound, of one token and around 32-row blocks."""
    L = np.minimum(np.array(EDGE + [S, S - 1, 33, 97], dtype=np.int32), S)
    check_bwd(W.custom(90 + d + S, L, S, 3, d, W.FP32, with_grad=True), f"dS hand-off d={d} S={S}")


@pytest.mark.parametrize("d", [32, 64])
def test_fp32_recompute_path(d):
    """fp32 with the smaller workspace: dQ recomputes S and dP instead of reading the dS blocks
    of the dK/dV pass; the same oracle bar, and the two paths agree to fp32 rounding."""
    w = W.custom(80 + d, np.minimum(EDGE, 256), 256, 3, d, W.FP32, with_grad=True)
    check_bwd(w, f"edge lengths d={d}, recompute path", full_workspace=False)
    a = gpu_fwd_bwd(w, True)[1:]
    b = gpu_fwd_bwd(w, False)[1:]
    for x, y in zip(a, b):
        err = (x - y).abs().max().item()
        assert err <= 1e-5 * max(1.0, y.abs().max().item()), f"paths differ by {err:.3e}"


@pytest.mark.parametrize("S", [32, 64])
@pytest.mark.parametrize("d", [32, 64])
def test_short_single_pass(S, d):
    """A length bound of at most 64: one wave per (sequence, head) forms dQ, dK and dV in one pass.
    Lengths at the block edges (1, 31, 32, 33, 63, 64) and random ones, three heads."""
    L = np.concatenate([[1, 2, 31, 32, 33, 63, 64, 17], W.random_lengths(81 + d, 200, 1, 64)])
    L = np.minimum(L, S).astype(np.int32)
    check_bwd(W.custom(80 + d + S, L, S, 3, d, W.BF16, with_grad=True), f"short single pass S={S} d={d}")


@pytest.mark.parametrize("dtype", [W.FP32, W.BF16])
def test_ragged_mixed(dtype):
    rng = np.random.default_rng(71)
    L = np.concatenate([rng.integers(16, 49, size=120), [1500, 777, 2100], rng.integers(100, 400, size=5)])
    L = rng.permutation(L).astype(np.int32)
    check_bwd(W.custom(72, L, 2100, 4, 64, dtype, with_grad=True), "ragged mixed")


def test_single_token_sequences():
    # a length-1 sequence has P = 1, so dQ = dK = 0 and dV = dO
    w = W.custom(73, [1, 4, 1, 1], 4, 2, 64, W.FP32, with_grad=True)
    cu_ref, dq, dk, dv = gpu_fwd_bwd(w)
    for r in (0, 5, 6):
        assert np.abs(from_dev(dq)[r]).max() <= 1e-6
        assert np.abs(from_dev(dk)[r]).max() <= 1e-6
        np.testing.assert_allclose(from_dev(dv)[r], w.dout[r], atol=1e-6)
    check_bwd(w, "length-one sequences")


def test_deterministic_and_isolated():
    L = np.array([50, 130, 7, 260, 90, 1, 128], dtype=np.int32)
    w = W.custom(74, L, 260, 2, 64, W.BF16, with_grad=True)
    a = gpu_fwd_bwd(w)[1:]
    b = gpu_fwd_bwd(w)[1:]
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    cu64 = np.concatenate([[0], np.cumsum(L)])
    bsel = 3
    for x in (w.q, w.k, w.v, w.dout):
        x[cu64[bsel]:cu64[bsel + 1]] = W.f32_to_bf16_bits(
            5 * np.random.default_rng(2).standard_normal(x[cu64[bsel]:cu64[bsel + 1]].shape, dtype=np.float32))
    c = gpu_fwd_bwd(w)[1:]
    other = np.r_[0:cu64[bsel], cu64[bsel + 1]:cu64[-1]]
    for x, y in zip(a, c):
        assert np.array_equal(from_dev(x)[other], from_dev(y)[other])


def test_mixed_training_full_size():
    w = W.mixed_training()
    L = w.lengths
    order = np.argsort(L)
    seqs = sorted({int(order[0]), int(order[1]), int(order[len(L) // 2]), int(order[-1]), int(order[-2]),
                   int(order[-40]), 0, len(L) - 1})
    check_bwd(w, "mixed-training full size", seqs=seqs)


def test_graph_transformer_full_size():
    w = W.graph_transformer(grid=False, with_grad=True)
    L = w.lengths
    order = np.argsort(L)
    seqs = sorted({int(order[0]), int(order[-1]), int(order[len(L) // 2]), 0, 1, len(L) - 1} |
                  set(int(x) for x in np.random.default_rng(5).integers(0, len(L), size=24)))
    check_bwd(w, "graph-transformer full size", seqs=seqs)


@pytest.mark.parametrize("dtype", [W.FP32, W.BF16])
def test_very_long_sequence(dtype):
    """A 40000-token document (313 query tiles and 1250 key blocks of its own)
    among shorter sequences. The forward is checked at sampled rows, the
    backward in full on the other sequences and, on the long document, through
    two sums that hold at any length: each row of P sums to 1, so the dV rows
    sum to the dO rows; each row of dS sums to 0 (D is <dO, O> with O = P V), so
    the dK rows sum to 0."""
    from tests.test_gpu_fwd import check_sampled

    w = W.custom(95, [40000, 3, 1, 6000, 777], 40000, 2, 64, dtype, with_grad=True)
    label = f"40000-token document {dtype}"
    check_sampled(w, label)
    cu_ref, dq, dk, dv = check_bwd(w, label, seqs=[1, 2, 3, 4])
    c0, c1 = int(cu_ref[0]), int(cu_ref[1])
    do = W.to_f64(w.dout, w.dtype)[c0:c1]
    gdv, gdk = to_f64(dv)[c0:c1], to_f64(dk)[c0:c1]
    assert np.isfinite(gdv).all() and np.isfinite(gdk).all() and np.isfinite(to_f64(dq)[c0:c1]).all()
    # bf16: P enters the dV product rounded to bf16 (2^-9 of each weight) and dV is stored in bf16
    rel = 2.0 ** -8 if dtype == W.BF16 else 1e-5
    err_v = np.abs(gdv.sum(axis=0) - do.sum(axis=0))
    assert (err_v <= rel * (np.abs(gdv).sum(axis=0) + np.abs(do).sum(axis=0))).all(), \
        f"sum of dV rows vs sum of dO rows: max |delta| {err_v.max():.3e}"
    if dtype == W.FP32:
        err_k = np.abs(gdk.sum(axis=0))
        assert (err_k <= 1e-4 * np.abs(gdk).sum(axis=0)).all(), f"sum of dK rows: max {err_k.max():.3e}"
