"""GPU parity of the local (sliding-window) calls pe_varlen_attn_fwd_local and
pe_varlen_attn_bwd_local against the fp64 oracle's windowed attention, on every
kernel family (fp32 one-wave kernels, generic kernels, bf16 LDS-DMA kernels)."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, check_lse, check_out, from_dev, sample_rows, say, to_dev, to_f64
from tests.test_gpu_bwd import check_grad

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")

EDGE = [1, 127, 128, 129, 5, 256, 257, 3, 300, 64, 65, 1, 1, 2, 31, 32, 33, 16, 15, 17, 200]


def _code(w):
    return pe.PE_BF16 if w.dtype == W.BF16 else pe.PE_FP32


def gpu_local(w: W.Workload, window: int, with_bwd=False):
    cu_ref, _, N = oracle.layout(w.lengths, w.max_seq_len)
    cu = torch.from_numpy(cu_ref).to(DEV)
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    ws = pe.workspace(pe.pe_attn_workspace_size(w.num_seqs, N, w.num_heads, w.head_dim, _code(w), with_bwd), DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((w.num_heads, N), float("nan"), device=DEV)
    pe.pe_varlen_attn_fwd_local(q, k, v, cu, w.num_seqs, N, w.max_seq_len, w.scale, window, out, lse, ws)
    grads = None
    if with_bwd:
        do = to_dev(w.dout, w.dtype)
        grads = tuple(torch.full_like(q, float("nan")) for _ in range(3))
        pe.pe_varlen_attn_bwd_local(do, q, k, v, out, lse, cu, w.num_seqs, N, w.max_seq_len, w.scale, window,
                                    *grads, ws)
    torch.cuda.synchronize()
    return cu_ref, out, lse, grads


def check_local(w: W.Workload, window: int, label: str):
    say(f"[local fwd] {label} w={window}: B={w.num_seqs} N={w.total_tokens} d={w.head_dim} {w.dtype}")
    cu_ref, out, lse, _ = gpu_local(w, window)
    q, k, v = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v))
    o_ref, l_ref = oracle.attention(q, k, v, cu_ref, w.scale, window=window)
    check_out(to_f64(out), o_ref, w.dtype, f"{label} out")
    check_lse(to_f64(lse), l_ref, w.dtype, f"{label} lse")


@pytest.mark.parametrize("dtype", [W.FP32, W.BF16])
@pytest.mark.parametrize("d", [8, 32, 64, 128])
@pytest.mark.parametrize("window", [0, 1, 32, 100])
def test_local_forward_edge_lengths(dtype, d, window):
    # max_seq_len 300: bf16 d 32/64/128 take the LDS-DMA kernels, fp32 d 32/64 the one-wave kernels
    check_local(W.custom(60 + d, EDGE, 300, 2, d, dtype), window, f"edge d={d}")


@pytest.mark.parametrize("dtype", [W.FP32, W.BF16])
@pytest.mark.parametrize("window", [3, 31, 64])
@pytest.mark.parametrize("d", [32, 64])
def test_local_forward_short_bound(dtype, window, d):
    # length bound 48: 16-bit d 32/64 take the one-wave-per-sequence kernel (band mask per score)
    L = W.random_lengths(61, 300, 1, 48)
    check_local(W.custom(62 + d, L, 48, 3, d, dtype), window, f"short bound d={d}")


def test_local_wide_window_equals_global_bitwise():
    w = W.custom(63, EDGE, 300, 2, 64, W.BF16)
    cu_ref, out_l, lse_l, _ = gpu_local(w, 299)
    cu = torch.from_numpy(cu_ref).to(DEV)
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    N = int(cu_ref[-1])
    ws = pe.workspace(pe.pe_attn_workspace_size(w.num_seqs, N, 2, 64, pe.PE_BF16, False), DEV)
    out = torch.empty_like(q)
    lse = torch.empty(2, N, device=DEV)
    pe.pe_varlen_attn_fwd(q, k, v, cu, w.num_seqs, N, w.max_seq_len, w.scale, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_l.view(torch.int16))
    assert torch.equal(lse, lse_l)


def test_local_wide_window_backward_equals_global_bitwise():
    """A window wider than every sequence: the local backward streams and computes exactly what
    the global one does, so the gradients agree bit for bit."""
    w = W.custom(65, EDGE, 300, 2, 64, W.BF16, with_grad=True)
    cu_ref, out, lse, grads_l = gpu_local(w, 299, with_bwd=True)
    cu = torch.from_numpy(cu_ref).to(DEV)
    q, k, v, do = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v, w.dout))
    N = int(cu_ref[-1])
    ws = pe.workspace(pe.pe_attn_workspace_size(w.num_seqs, N, 2, 64, pe.PE_BF16, True), DEV)
    grads = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    pe.pe_varlen_attn_bwd(do, q, k, v, out, lse, cu, w.num_seqs, N, w.max_seq_len, w.scale, *grads, ws)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), grads, grads_l):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


def test_local_long_document_sampled():
    # the long-document lengths (first 200 sequences), window 32, sampled rows
    full = W.long_document()
    L = full.lengths[:200]
    w = W.custom(64, L, 8192, 4, 64, W.BF16)
    say(f"[local fwd] long documents w=32: N={w.total_tokens}")
    cu_ref, out, lse, _ = gpu_local(w, 32)
    rows = sample_rows(cu_ref, 128, 200, seed=3)
    q, k, v = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v))
    o_ref, l_ref = oracle.attention_rows(q, k, v, cu_ref, w.scale, rows, window=32)
    check_out(W.to_f64(from_dev(out)[rows], w.dtype), o_ref, w.dtype, "long local out")
    check_lse(from_dev(lse)[:, rows].astype(np.float64), l_ref, w.dtype, "long local lse")


def check_local_bwd(w: W.Workload, window: int, label: str):
    say(f"[local bwd] {label} w={window}: B={w.num_seqs} N={w.total_tokens} d={w.head_dim} {w.dtype}")
    cu_ref, out, lse, grads = gpu_local(w, window, with_bwd=True)
    q, k, v, do = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v, w.dout))
    out_given = None
    if w.dtype == W.BF16:
        o_ref, _ = oracle.attention(q, k, v, cu_ref, w.scale, window=window)
        out_given = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_ref.astype(np.float32))).astype(np.float64)
    ref = oracle.attention_backward(do, q, k, v, cu_ref, w.scale, out=out_given, window=window)
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        check_grad(to_f64(g), r, w.dtype, f"{label} {name}")


@pytest.mark.parametrize("dtype", [W.FP32, W.BF16])
@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("window", [0, 5, 40])
def test_local_backward_edge_lengths(dtype, d, window):
    check_local_bwd(W.custom(70 + d, EDGE, 300, 2, d, dtype, with_grad=True), window, f"edge d={d}")


@pytest.mark.parametrize("window", [0, 3, 31])
@pytest.mark.parametrize("d", [32, 64])
def test_local_backward_short_bound(window, d):
    # length bound 48: the 16-bit single-pass kernel (one wave per sequence and head, band mask per score)
    L = W.random_lengths(66, 200, 1, 48)
    check_local_bwd(W.custom(67 + d, L, 48, 3, d, W.BF16, with_grad=True), window, f"short bound d={d}")


def test_local_backward_generic_head_dims():
    check_local_bwd(W.custom(71, EDGE[:12], 300, 2, 16, W.FP32, with_grad=True), 7, "fp32 d=16")
    check_local_bwd(W.custom(72, EDGE[:12], 300, 2, 128, W.BF16, with_grad=True), 7, "bf16 d=128")


@pytest.mark.parametrize("dtype", [W.FP32, W.BF16])
def test_local_backward_long_sequences(dtype):
    # an 8192-token document among shorter ones: the banded tiles run across many key blocks
    L = [2188, 17, 8192, 368, 1, 16, 1000, 129]
    check_local_bwd(W.custom(73, L, 8192, 2, 64, dtype, with_grad=True), 32, "long sequences d=64")
