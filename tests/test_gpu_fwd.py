"""GPU parity of pe_varlen_attn_fwd and pe_varlen_attn_fwd_first_token against
the fp64 oracle: small ragged cases element by element, the standing workloads
at full size on sampled rows, and properties (isolation, determinism, write
coverage) that hold at any size."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, check_lse, check_out, from_dev, sample_rows, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")

TILE = 128


def gpu_forward(w: W.Workload, with_lse=True, poison=True):
    cu_ref, _, N = oracle.layout(w.lengths, w.max_seq_len)
    cu = torch.from_numpy(cu_ref).to(DEV)
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    out = torch.full_like(q, float("nan")) if poison else torch.empty_like(q)
    lse = torch.full((w.num_heads, N), float("nan"), device=DEV) if with_lse else None
    ws = pe.workspace(pe.pe_attn_workspace_size(w.num_seqs, N, w.num_heads, w.head_dim,
                                                pe.PE_BF16 if w.dtype == W.BF16 else pe.PE_FP32, False), DEV)
    pe.pe_varlen_attn_fwd(q, k, v, cu, w.num_seqs, N, w.max_seq_len, w.scale, out, lse, ws)
    torch.cuda.synchronize()
    return cu_ref, q, k, v, cu, out, lse


def gpu_first(w: W.Workload, q, k, v, cu, cu_ref):
    qf = q[torch.from_numpy(cu_ref[:-1].astype(np.int64)).to(DEV)].contiguous()
    of = torch.full_like(qf, float("nan"))
    lf = torch.full((w.num_heads, w.num_seqs), float("nan"), device=DEV)
    pe.pe_varlen_attn_fwd_first_token(qf, k, v, cu, w.num_seqs, int(cu_ref[-1]), w.max_seq_len, w.scale, of, lf)
    torch.cuda.synchronize()
    return of, lf


def check_full(w: W.Workload, label: str):
    say(f"[fwd] {label}: B={w.num_seqs} N={w.total_tokens} H={w.num_heads} d={w.head_dim} {w.dtype}")
    cu_ref, q, k, v, cu, out, lse = gpu_forward(w)
    qf64, kf64, vf64 = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v))
    o_ref, l_ref = oracle.attention(qf64, kf64, vf64, cu_ref, w.scale)
    check_out(to_f64(out), o_ref, w.dtype)
    check_lse(to_f64(lse), l_ref, w.dtype)
    say(f"[first] {label}")
    of, lf = gpu_first(w, q, k, v, cu, cu_ref)
    of_ref, lf_ref = oracle.attention_first_token(qf64[cu_ref[:-1]], kf64, vf64, cu_ref, w.scale)
    check_out(to_f64(of), of_ref, w.dtype, "first-token out")
    check_lse(to_f64(lf), lf_ref, w.dtype, "first-token lse")


def test_tiny():
    check_full(W.tiny(with_grad=False), "tiny")


def test_gigl_example():
    check_full(W.custom(5, [3, 1, 2], 3, 2, 8, W.FP32), "gigl example")


EDGE = [1, 127, 128, 129, 5, 256, 257, 3, 300, 64, 65, 1, 1, 2, 31, 32, 33, 16, 15, 17, 200]


@pytest.mark.parametrize("dtype", [W.FP32, W.BF16])
@pytest.mark.parametrize("d", list(range(8, 129, 8)))
def test_edge_lengths(dtype, d):
    w = W.custom(20 + d, EDGE, 300, 3, d, dtype)
    check_full(w, f"edge lengths d={d}")


@pytest.mark.parametrize("dtype", [W.FP32, W.BF16])
def test_ragged_mixed(dtype):
    rng = np.random.default_rng(31)
    L = np.concatenate([rng.integers(1, 50, size=150), [1500, 777, 2048], rng.integers(100, 400, size=5)])
    L = rng.permutation(L).astype(np.int32)
    w = W.custom(32, L, 2048, 4, 64, dtype)
    check_full(w, "ragged mixed")


def test_single_sequence_and_single_token():
    check_full(W.custom(40, [1], 1, 2, 64, W.FP32), "one token")
    check_full(W.custom(41, [1, 1, 1, 1, 1], 4, 2, 64, W.BF16), "all length one")
    check_full(W.custom(42, [4000], 4096, 2, 64, W.BF16), "one long sequence")


def test_closed_forms_on_gpu():
    # identical keys in a sequence give the mean of its values; constant values pass through
    w = W.custom(43, [37, 1, 300], 300, 2, 64, W.FP32)
    w.k[0:37] = w.k[0]
    w.k[38:338] = w.k[38]
    w.v[38:338] = 0.25
    cu_ref, q, k, v, cu, out, lse = gpu_forward(w)
    o = to_f64(out)
    np.testing.assert_allclose(o[0:37], np.broadcast_to(w.v[0:37].astype(np.float64).mean(0), (37, 2, 64)),
                               atol=1e-5)
    np.testing.assert_array_equal(o[37], w.v[37].astype(np.float64))   # length one: its own V row
    np.testing.assert_allclose(o[38:338], 0.25, atol=1e-6)


SHORT_EDGE = [64, 1, 63, 33, 32, 31, 1, 1, 64, 64, 2, 17, 48, 49, 5, 64, 1]


@pytest.mark.parametrize("d", [8, 32, 64, 128])
@pytest.mark.parametrize("S", [64, 48, 16])
def test_short_length_bounds(d, S):
    # length bounds <= 64 take the one-wave-per-sequence kernel for bf16 d 32/64 (the
    # packed-tile kernel for other d): lengths at the bound, of one token, and straddling
    # 32-key blocks
    rng = np.random.default_rng(48 + S + d)
    L = np.concatenate([np.minimum(SHORT_EDGE, S), rng.integers(1, S + 1, size=300)])
    L = rng.permutation(L).astype(np.int32)
    check_full(W.custom(49 + d, L, S, 3, d, W.BF16), f"short bound S={S} d={d}")


def test_short_bound_far_above_lengths():
    # a bound much larger than every length: the window holds many foreign rows
    check_full(W.custom(50, W.random_lengths(51, 400, 1, 9), 64, 2, 64, W.BF16), "bound 64, lengths <= 9")


@pytest.mark.parametrize("d", [32, 64, 128])
def test_running_max_paths(d):
    # logits that drift along the keys: for some queries the running max creeps up
    # block after block (small steps that add up), for others it is set by the first
    # keys, and a late block of much larger keys forces a jump in every row
    L = np.array([2000, 700, 45], dtype=np.int32)
    w = W.custom(47 + d, L, 2048, 2, d, W.BF16)
    k = W.bf16_bits_to_f32(w.k)
    ramp = np.linspace(0.0, 3.0, 2000, dtype=np.float32)[:, None, None]
    k[0:2000] = k[0] * ramp + 0.1 * k[0:2000]
    k[1500:1530] *= 4.0
    w.k = W.f32_to_bf16_bits(k)
    check_full(w, f"running max paths d={d}")


def test_isolation_bitwise():
    L = np.array([50, 130, 7, 260, 90, 1, 128], dtype=np.int32)
    w = W.custom(44, L, 260, 2, 64, W.BF16)
    cu_ref, _, _, _, _, out1, lse1 = gpu_forward(w)
    cu64 = cu_ref.astype(np.int64)
    b = 3
    for x in (w.q, w.k, w.v):
        x[cu64[b]:cu64[b + 1]] = W.f32_to_bf16_bits(
            10 * np.random.default_rng(1).standard_normal(x[cu64[b]:cu64[b + 1]].shape, dtype=np.float32))
    _, _, _, _, _, out2, lse2 = gpu_forward(w)
    other = np.r_[0:cu64[b], cu64[b + 1]:cu64[-1]]
    a1, a2 = from_dev(out1), from_dev(out2)
    assert np.array_equal(a1[other], a2[other])
    assert np.array_equal(from_dev(lse1)[:, other], from_dev(lse2)[:, other])
    assert not np.array_equal(a1[cu64[b]:cu64[b + 1]], a2[cu64[b]:cu64[b + 1]])


def test_deterministic_and_no_lse():
    w = W.custom(45, W.random_lengths(46, 200, 1, 400), 400, 4, 64, W.BF16)
    _, _, _, _, _, out1, lse1 = gpu_forward(w)
    _, _, _, _, _, out2, lse2 = gpu_forward(w)
    _, _, _, _, _, out3, _ = gpu_forward(w, with_lse=False)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))


# ---------------------------------------------------------------- full-size standing workloads

def check_sampled(w: W.Workload, label: str, n_random=160, first_token=True):
    say(f"[fwd] {label} full size: B={w.num_seqs} N={w.total_tokens} H={w.num_heads} {w.dtype}")
    cu_ref, q, k, v, cu, out, lse = gpu_forward(w)
    o = from_dev(out)
    ls = from_dev(lse)
    assert not np.isnan(o.view(np.float32) if o.dtype == np.float32 else W.bf16_bits_to_f32(o)).any()
    assert not np.isnan(ls).any()
    rows = sample_rows(cu_ref, TILE, n_random, seed=w.num_seqs)
    qf64 = W.to_f64(w.q, w.dtype)
    kf64 = W.to_f64(w.k, w.dtype)
    vf64 = W.to_f64(w.v, w.dtype)
    o_ref, l_ref = oracle.attention_rows(qf64, kf64, vf64, cu_ref, w.scale, rows)
    og = W.to_f64(o[rows], w.dtype)
    check_out(og, o_ref, w.dtype, f"{label} sampled out")
    check_lse(ls[:, rows].astype(np.float64), l_ref, w.dtype, f"{label} sampled lse")
    if first_token:
        say(f"[first] {label} full size")
        of, lf = gpu_first(w, q, k, v, cu, cu_ref)
        seqs = sorted(set(range(0, w.num_seqs, max(1, w.num_seqs // 512))) | {w.num_seqs - 1})
        of_ref, lf_ref = oracle.attention_first_token(qf64[cu_ref[:-1]], kf64, vf64, cu_ref, w.scale, seqs)
        check_out(to_f64(of)[seqs], of_ref, w.dtype, f"{label} first-token out")
        check_lse(from_dev(lf)[:, seqs].astype(np.float64), lf_ref, w.dtype, f"{label} first-token lse")
        # first-token output equals the full output at rows cu[:-1] up to accumulation order
        full_rows = W.to_f64(o[cu_ref[:-1]], w.dtype)
        check_out(to_f64(of), full_rows, w.dtype, f"{label} first-token vs full rows")


def test_graph_transformer_full():
    check_sampled(W.graph_transformer(grid=False, with_grad=False), "graph-transformer")


def test_short_query_full():
    check_sampled(W.short_query(grid=False), "short-query")


def test_long_document_full():
    check_sampled(W.long_document(), "long-document", first_token=False)


def test_mixed_training_forward_full():
    check_sampled(W.mixed_training(), "mixed-training", first_token=False)
