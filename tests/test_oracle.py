"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here touches a GPU. Each check compares the oracle with something other
than itself: printed worked examples, closed forms, an independent padded route,
torch's own SDPA and autograd in float64 (the library routine the GiGL CPU path
calls), finite differences, symmetries and isolation. The last section plants
plausible mistakes in calls of the oracle and shows that the pins catch them.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from padding_free_packed_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_case(seed, lengths, H=2, d=8, scale=None):
    rng = np.random.default_rng(seed)
    N = int(np.sum(lengths))
    q, k, v, do = (rng.standard_normal((N, H, d)) for _ in range(4))
    cu, _, _ = oracle.layout(lengths, max(lengths))
    return q, k, v, do, cu, (1.0 / np.sqrt(d) if scale is None else scale)


# ------------------------------------------------------------ worked examples (golden)

def test_gigl_example_layout():
    g = _golden("gigl_pack_example.json")
    cu, flat, N = oracle.layout(g["lengths"], g["max_seq_len"])
    assert flat.tolist() == g["flat_index"]
    assert cu.tolist() == g["cu_seqlens"]
    assert N == sum(g["lengths"])
    assert cu.dtype == np.int32 and flat.dtype == np.int64


def test_gigl_example_shapes():
    g = _golden("gigl_pack_example.json")
    cu = np.array(g["cu_seqlens"])
    N = int(cu[-1])
    rng = np.random.default_rng(0)
    x = rng.standard_normal((N, g["num_heads"], g["head_dim"]))
    o, lse = oracle.attention(x, x, x, cu, 1 / np.sqrt(g["head_dim"]))
    assert list(o.shape) == g["output_shape"]
    assert lse.shape == (g["num_heads"], N)
    of, lf = oracle.attention_first_token(x[cu[:-1]], x, x, cu, 1 / np.sqrt(g["head_dim"]))
    assert list(of.shape) == g["first_token_output_shape"]


def test_packed_encoders_cu_example():
    g = _golden("packed_encoders_cu_example.json")
    cu, flat, N = oracle.layout(g["lengths"], max(g["lengths"]))
    assert cu.tolist() == g["cu_seqlens"]
    assert N == g["total_tokens"]


def test_tiny_workload_lengths_match_recipe():
    # The tiny workload's seeded lengths are stated with the workload description.
    w = W.tiny()
    assert w.lengths.tolist() == [55, 41, 33, 18, 20, 3, 5, 2]
    assert w.total_tokens == 177


# ------------------------------------------------------------ layout / pack / unpack

def test_layout_brute_force():
    # flat_index enumerates the real grid cells in row-major (sequence, position) order.
    rng = np.random.default_rng(1)
    for _ in range(20):
        S = int(rng.integers(1, 20))
        B = int(rng.integers(1, 12))
        L = rng.integers(1, S + 1, size=B)
        cu, flat, N = oracle.layout(L, S)
        mask = np.arange(S)[None, :] < L[:, None]
        assert flat.tolist() == np.flatnonzero(mask.reshape(-1)).tolist()
        assert cu.tolist() == [0] + np.cumsum(L).tolist()


@pytest.mark.parametrize("bad", [[3, 0, 2], [3, 4, 2], [-1]])
def test_layout_rejects_bad_lengths(bad):
    with pytest.raises(ValueError):
        oracle.layout(bad, 3)


def test_pack_unpack_are_bit_copies():
    w = W.tiny()
    cu, flat, N = oracle.layout(w.lengths, w.max_seq_len)
    packed = oracle.pack(w.grid, flat)
    assert packed.shape == (N, w.row_elems)
    assert not np.isnan(packed).any()                 # the NaN padding sentinel never leaks
    g = w.grid.reshape(-1, w.row_elems)
    for r in range(N):                                # element-wise definition
        assert packed[r].view(np.uint32).tolist() == g[flat[r]].view(np.uint32).tolist()
    grid2 = oracle.unpack(packed, cu, w.max_seq_len)
    mask = np.arange(w.max_seq_len)[None, :] < w.lengths[:, None]
    assert (grid2.view(np.uint32)[~mask] == 0).all()  # +0.0 fill
    assert (grid2.view(np.uint32)[mask] == w.grid.view(np.uint32)[mask]).all()
    assert (oracle.pack(grid2, flat).view(np.uint32) == packed.view(np.uint32)).all()


def test_pack_bf16_bits():
    w = W.custom(5, [3, 1, 2], 3, 2, 8, W.BF16, grid=True)
    cu, flat, N = oracle.layout(w.lengths, w.max_seq_len)
    packed = oracle.pack(w.grid, flat)
    assert packed.dtype == np.uint16
    g = w.grid.reshape(-1, 16)
    assert (packed == g[[0, 1, 2, 3, 6, 7]]).all()


# ------------------------------------------------------------ closed forms

def test_length_one_returns_own_value_row():
    q, k, v, _, cu, sc = _rand_case(2, [1, 1, 4, 1])
    o, lse = oracle.attention(q, k, v, cu, sc)
    for r in (0, 1, 6):
        np.testing.assert_array_equal(o[r], v[r])
        np.testing.assert_allclose(lse[:, r], sc * np.sum(q[r] * k[r], axis=-1), rtol=0, atol=1e-14)


def test_identical_keys_give_mean_of_values():
    q, k, v, _, cu, sc = _rand_case(3, [5, 7])
    k[0:5] = k[0]
    k[5:12] = k[5]
    o, lse = oracle.attention(q, k, v, cu, sc)
    np.testing.assert_allclose(o[0:5], np.broadcast_to(v[0:5].mean(0), (5, 2, 8)), atol=1e-14)
    np.testing.assert_allclose(o[5:12], np.broadcast_to(v[5:12].mean(0), (7, 2, 8)), atol=1e-14)
    s0 = sc * np.einsum("nhd,hd->hn", q[0:5], k[0])
    np.testing.assert_allclose(lse[:, 0:5], s0 + np.log(5), atol=1e-13)


def test_constant_values_pass_through():
    q, k, v, _, cu, sc = _rand_case(4, [9, 2, 30])
    c = np.random.default_rng(0).standard_normal((2, 8))
    v[:] = c
    o, _ = oracle.attention(q, k, v, cu, sc)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-14)


def test_two_keys_logistic():
    # Two keys: weights are the logistic function of the logit difference.
    q, k, v, _, cu, sc = _rand_case(5, [2])
    o, lse = oracle.attention(q, k, v, cu, sc)
    for i in range(2):
        for h in range(2):
            s0, s1 = sc * q[i, h] @ k[0, h], sc * q[i, h] @ k[1, h]
            w1 = 1.0 / (1.0 + np.exp(s0 - s1))
            np.testing.assert_allclose(o[i, h], (1 - w1) * v[0, h] + w1 * v[1, h], atol=1e-14)
            np.testing.assert_allclose(lse[h, i], np.logaddexp(s0, s1), atol=1e-14)


# ------------------------------------------------------------ independent routes

def test_packed_equals_padded_twin():
    w = W.tiny()
    q, k, v = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v))
    cu, _, _ = oracle.layout(w.lengths, w.max_seq_len)
    o, lse = oracle.attention(q, k, v, cu, w.scale)
    o2, lse2 = oracle.padded_attention(q, k, v, cu, w.max_seq_len, w.scale)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-14)
    of, lf = oracle.attention_first_token(q[cu[:-1]], k, v, cu, w.scale)
    of2, lf2 = oracle.padded_attention(q[cu[:-1]], k, v, cu, w.max_seq_len, w.scale, True)
    np.testing.assert_allclose(of, of2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lf, lf2, rtol=1e-13, atol=1e-14)


def _torch_padded_sdpa(q, k, v, cu, S, scale):
    """The GiGL CPU route written with torch: dense grid, finfo.min/2 key bias, SDPA, [mask]."""
    q, k, v = (torch.from_numpy(x) for x in (q, k, v))
    cu = torch.from_numpy(np.asarray(cu, dtype=np.int64))
    lengths = cu[1:] - cu[:-1]
    B = lengths.numel()
    N, H, d = k.shape
    seq = torch.repeat_interleave(torch.arange(B), lengths)
    pos = torch.arange(N) - cu[:-1][seq]
    mask = torch.zeros(B, S, dtype=torch.bool)
    mask[seq, pos] = True

    def grid(x):
        g = torch.zeros(B, S, H, d, dtype=x.dtype)
        g = g.index_put((seq, pos), x)
        return g.transpose(1, 2)

    bias = torch.zeros(B, S, dtype=torch.float64).masked_fill(~mask, torch.finfo(torch.float64).min / 2)
    out = F.scaled_dot_product_attention(grid(q), grid(k), grid(v),
                                         attn_mask=bias.view(B, 1, 1, S), scale=scale)
    return out.transpose(1, 2)[mask]


def test_matches_torch_sdpa_float64():
    w = W.tiny()
    q, k, v = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v))
    cu, _, _ = oracle.layout(w.lengths, w.max_seq_len)
    o, lse = oracle.attention(q, k, v, cu, w.scale)
    ref = _torch_padded_sdpa(q, k, v, cu, w.max_seq_len, w.scale).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    # log-sum-exp against torch.logsumexp of the masked logits of each sequence
    qt, kt = torch.from_numpy(q), torch.from_numpy(k)
    for b in range(len(cu) - 1):
        c0, c1 = int(cu[b]), int(cu[b + 1])
        s = w.scale * torch.einsum("ihd,jhd->hij", qt[c0:c1], kt[c0:c1])
        np.testing.assert_allclose(lse[:, c0:c1], torch.logsumexp(s, dim=-1).numpy(), rtol=1e-13, atol=1e-13)


def test_backward_matches_torch_autograd_float64():
    w = W.tiny()
    q, k, v, do = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v, w.dout))
    cu, _, _ = oracle.layout(w.lengths, w.max_seq_len)
    dq, dk, dv = oracle.attention_backward(do, q, k, v, cu, w.scale)
    qt, kt, vt = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    out = _torch_padded_sdpa_autograd(qt, kt, vt, cu, w.max_seq_len, w.scale)
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-11, atol=1e-12)


def _torch_padded_sdpa_autograd(q, k, v, cu, S, scale):
    cu = torch.from_numpy(np.asarray(cu, dtype=np.int64))
    lengths = cu[1:] - cu[:-1]
    B = lengths.numel()
    N, H, d = k.shape
    seq = torch.repeat_interleave(torch.arange(B), lengths)
    pos = torch.arange(N) - cu[:-1][seq]
    mask = torch.zeros(B, S, dtype=torch.bool)
    mask[seq, pos] = True

    def grid(x):
        g = torch.zeros(B, S, H, d, dtype=x.dtype).index_put((seq, pos), x)
        return g.transpose(1, 2)

    bias = torch.zeros(B, S, dtype=torch.float64).masked_fill(~mask, torch.finfo(torch.float64).min / 2)
    out = F.scaled_dot_product_attention(grid(q), grid(k), grid(v),
                                         attn_mask=bias.view(B, 1, 1, S), scale=scale)
    return out.transpose(1, 2)[mask]


def test_backward_given_output_and_lse():
    # With the exact forward passed in, the result is unchanged; an output
    # perturbation delta at row i moves only the D term: dQ_i changes by
    # -scale * <dO_i, delta> * sum_j P_ij K_j and dK_j by -scale * P_ij <dO_i, delta> Q_i.
    lengths = [4, 7]
    q, k, v, do, cu, sc = _rand_case(12, lengths)
    o, lse = oracle.attention(q, k, v, cu, sc)
    base = oracle.attention_backward(do, q, k, v, cu, sc)
    same = oracle.attention_backward(do, q, k, v, cu, sc, out=o, lse=lse)
    for a, b in zip(base, same):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    i, h = 6, 1
    delta = np.zeros_like(o)
    delta[i, h] = np.random.default_rng(4).standard_normal(8) * 1e-3
    pert = oracle.attention_backward(do, q, k, v, cu, sc, out=o + delta, lse=lse)
    c0, c1 = 4, 11
    p = np.exp(sc * q[i, h] @ k[c0:c1, h].T - lse[h, i])
    dD = float(do[i, h] @ delta[i, h])
    np.testing.assert_allclose(pert[0][i, h] - base[0][i, h], -sc * dD * (p @ k[c0:c1, h]), rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(pert[1][c0:c1, h] - base[1][c0:c1, h], -sc * dD * np.outer(p, q[i, h]),
                               rtol=1e-9, atol=1e-15)
    np.testing.assert_array_equal(pert[2], base[2])          # dV does not involve D
    others = [r for r in range(11) if r != i]
    np.testing.assert_allclose(pert[0][others], base[0][others], rtol=1e-12, atol=1e-15)


def test_backward_finite_differences():
    lengths = [1, 5, 13, 3]
    q, k, v, do, cu, sc = _rand_case(6, lengths)
    dq, dk, dv = oracle.attention_backward(do, q, k, v, cu, sc)

    def f(q_, k_, v_):
        return float(np.sum(do * oracle.attention(q_, k_, v_, cu, sc)[0]))

    h = 1e-6
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7)


# ------------------------------------------------------------ invariants

def test_first_token_equals_full_rows():
    w = W.tiny()
    q, k, v = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v))
    cu, _, _ = oracle.layout(w.lengths, w.max_seq_len)
    o, lse = oracle.attention(q, k, v, cu, w.scale)
    of, lf = oracle.attention_first_token(q[cu[:-1]], k, v, cu, w.scale)
    # same definition, evaluated as a matrix-vector product: equal up to rounding order
    np.testing.assert_allclose(of, o[cu[:-1]], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lf, lse[:, cu[:-1]], rtol=1e-13, atol=1e-15)


def test_rows_equal_full():
    w = W.tiny()
    q, k, v = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v))
    cu, _, _ = oracle.layout(w.lengths, w.max_seq_len)
    o, lse = oracle.attention(q, k, v, cu, w.scale)
    rows = [0, 54, 55, 100, 176]
    o2, l2 = oracle.attention_rows(q, k, v, cu, w.scale, rows)
    np.testing.assert_allclose(o2, o[rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l2, lse[:, rows], rtol=1e-13, atol=1e-14)


def test_permuting_sequences_permutes_outputs():
    lengths = [4, 9, 1, 6]
    q, k, v, do, cu, sc = _rand_case(7, lengths)
    o, lse = oracle.attention(q, k, v, cu, sc)
    dq, dk, dv = oracle.attention_backward(do, q, k, v, cu, sc)
    perm = [2, 0, 3, 1]
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in perm])
    cu2, _, _ = oracle.layout([lengths[b] for b in perm], 9)
    o2, lse2 = oracle.attention(q[rows], k[rows], v[rows], cu2, sc)
    np.testing.assert_allclose(o2, o[rows], atol=1e-14)
    np.testing.assert_allclose(lse2, lse[:, rows], atol=1e-14)
    g2 = oracle.attention_backward(do[rows], q[rows], k[rows], v[rows], cu2, sc)
    for a, b in zip(g2, (dq, dk, dv)):
        np.testing.assert_allclose(a, b[rows], atol=1e-13)


def test_permuting_keys_within_sequence_is_invariant():
    lengths = [11]
    q, k, v, _, cu, sc = _rand_case(8, lengths)
    o, lse = oracle.attention(q, k, v, cu, sc)
    p = np.random.default_rng(1).permutation(11)
    o2, lse2 = oracle.attention(q, k[p], v[p], cu, sc)
    np.testing.assert_allclose(o2, o, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, atol=1e-14)


def test_isolation_between_sequences():
    lengths = [6, 3, 8]
    q, k, v, do, cu, sc = _rand_case(9, lengths)
    o, lse = oracle.attention(q, k, v, cu, sc)
    g = oracle.attention_backward(do, q, k, v, cu, sc)
    q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
    for x in (q2, k2, v2, do2):
        x[6:9] = 100.0 * np.random.default_rng(3).standard_normal(x[6:9].shape)
    o2, lse2 = oracle.attention(q2, k2, v2, cu, sc)
    g2 = oracle.attention_backward(do2, q2, k2, v2, cu, sc)
    other = np.r_[0:6, 9:17]
    np.testing.assert_array_equal(o2[other], o[other])
    np.testing.assert_array_equal(lse2[:, other], lse[:, other])
    for a, b in zip(g2, g):
        np.testing.assert_array_equal(a[other], b[other])


def test_worklist_brute_force():
    rng = np.random.default_rng(10)
    for R in (1, 4, 32, 128):
        L = rng.integers(1, 50, size=17)
        cu, _, N = oracle.layout(L, 50)
        wl = oracle.worklist(cu, R)
        T = (N + R - 1) // R
        assert wl.shape == (T + 1,) and wl[-1] == 17
        for t in range(T):
            b = wl[t]
            assert cu[b] <= t * R < cu[b + 1]


# ------------------------------------------------------------ planted mistakes are caught

def _forward_pins_pass(attn):
    """Run the closed-form and independent-route pins against an attention function."""
    try:
        q, k, v, _, cu, sc = _rand_case(2, [1, 1, 4, 1])
        o, lse = attn(q, k, v, cu, sc)
        np.testing.assert_array_equal(o[0], v[0])
        np.testing.assert_allclose(lse[:, 0], sc * np.sum(q[0] * k[0], axis=-1), atol=1e-14)
        q, k, v, _, cu, sc = _rand_case(4, [9, 2, 30])
        c = np.ones((2, 8))
        v[:] = c
        o, _ = attn(q, k, v, cu, sc)
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-14)
        w = W.tiny()
        q, k, v = (W.to_f64(x, w.dtype) for x in (w.q, w.k, w.v))
        cu, _, _ = oracle.layout(w.lengths, w.max_seq_len)
        o, _ = attn(q, k, v, cu, w.scale)
        ref = _torch_padded_sdpa(q, k, v, cu, w.max_seq_len, w.scale).numpy()
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
        return True
    except AssertionError:
        return False


@pytest.mark.parametrize("mutant", ["scale_dropped", "value_is_key", "no_boundaries", "lse_log2"])
def test_planted_forward_mistakes_are_caught(mutant):
    def attn(q, k, v, cu, sc):
        if mutant == "scale_dropped":
            return oracle.attention(q, k, v, cu, 1.0)
        if mutant == "value_is_key":
            return oracle.attention(q, k, k, cu, sc)
        if mutant == "no_boundaries":
            return oracle.attention(q, k, v, [0, int(cu[-1])], sc)
        if mutant == "lse_log2":
            o, lse = oracle.attention(q, k, v, cu, sc)
            return o, lse / np.log(2.0)
    assert _forward_pins_pass(oracle.attention)
    assert not _forward_pins_pass(attn)


@pytest.mark.parametrize("mutant", ["dk_sign", "dq_dk_swapped", "dv_untransposed"])
def test_planted_backward_mistakes_are_caught(mutant):
    lengths = [1, 5, 3]
    q, k, v, do, cu, sc = _rand_case(11, lengths)

    def bwd(*a):
        dq, dk, dv = oracle.attention_backward(*a)
        if mutant == "dk_sign":
            return dq, -dk, dv
        if mutant == "dq_dk_swapped":
            return dk, dq, dv
        if mutant == "dv_untransposed":
            # dV = P dO instead of P^T dO, on each sequence
            out = dv.copy()
            for b in range(len(cu) - 1):
                c0, c1 = int(cu[b]), int(cu[b + 1])
                for h in range(q.shape[1]):
                    s = sc * q[c0:c1, h] @ k[c0:c1, h].T
                    p = np.exp(s - s.max(1, keepdims=True))
                    p /= p.sum(1, keepdims=True)
                    out[c0:c1, h] = p @ do[c0:c1, h]
            return dq, dk, out

    def f(q_, k_, v_):
        return float(np.sum(do * oracle.attention(q_, k_, v_, cu, sc)[0]))

    def fd_ok(grads):
        h = 1e-6
        for grad, which in zip(grads, (0, 1, 2)):
            for idx in list(np.ndindex(*grad.shape))[::7]:
                a_p = [q.copy(), k.copy(), v.copy()]
                a_m = [q.copy(), k.copy(), v.copy()]
                a_p[which][idx] += h
                a_m[which][idx] -= h
                if abs((f(*a_p) - f(*a_m)) / (2 * h) - grad[idx]) > 1e-6 + 1e-6 * abs(grad[idx]):
                    return False
        return True

    assert fd_ok(oracle.attention_backward(do, q, k, v, cu, sc))
    assert not fd_ok(bwd(do, q, k, v, cu, sc))


def test_planted_layout_mistake_is_caught():
    g = _golden("gigl_pack_example.json")
    cu, flat, _ = oracle.layout(g["lengths"], g["max_seq_len"])
    wrong = flat + np.repeat(np.arange(3), g["lengths"])  # b*(S+1)+t instead of b*S+t
    assert flat.tolist() == g["flat_index"]
    assert wrong.tolist() != g["flat_index"]
