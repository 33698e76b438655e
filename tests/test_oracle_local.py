"""Pins of the oracle's local (sliding-window) attention.

Query i sees the keys j of its own sequence with |i - j| <= w. Independent routes:
torch's SDPA in float64 over the whole packed buffer with a dense boolean mask
(same sequence and inside the band), its autograd, pure-Python loops on a tiny
case, closed forms (w = 0, w at least the longest sequence) and the padded twin.
A planted off-by-one in the band is shown to be caught.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

LENGTHS = [1, 5, 13, 3, 20, 2]


def _case(seed, lengths=LENGTHS, H=2, d=8):
    rng = np.random.default_rng(seed)
    N = int(np.sum(lengths))
    q, k, v, do = (rng.standard_normal((N, H, d)) for _ in range(4))
    cu, _, _ = oracle.layout(lengths, max(lengths))
    return q, k, v, do, cu, 1.0 / np.sqrt(d)


def _dense_mask(cu, window):
    cu = torch.from_numpy(np.asarray(cu, dtype=np.int64))
    lengths = cu[1:] - cu[:-1]
    seq = torch.repeat_interleave(torch.arange(lengths.numel()), lengths)
    i = torch.arange(seq.numel())
    return (seq[:, None] == seq[None, :]) & ((i[:, None] - i[None, :]).abs() <= window)


def _torch_dense(q, k, v, cu, window, scale):
    """SDPA over the packed buffer as one [H, N, N] problem with a boolean mask."""
    allowed = _dense_mask(cu, window)
    qt, kt, vt = (x.transpose(0, 1)[None] for x in (q, k, v))
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed[None, None], scale=scale)
    logits = scale * torch.einsum("ihd,jhd->hij", q, k).masked_fill(~allowed[None], float("-inf"))
    return out[0].transpose(0, 1), torch.logsumexp(logits, dim=-1)


@pytest.mark.parametrize("window", [0, 1, 3, 10, 19, 100])
def test_local_matches_torch_dense_mask(window):
    q, k, v, _, cu, sc = _case(1)
    o, lse = oracle.attention(q, k, v, cu, sc, window=window)
    ot, lt = _torch_dense(*(torch.from_numpy(x) for x in (q, k, v)), cu, window, sc)
    np.testing.assert_allclose(o, ot.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lt.numpy(), rtol=1e-13, atol=1e-13)


def test_window_zero_is_own_value_row():
    q, k, v, _, cu, sc = _case(2)
    o, lse = oracle.attention(q, k, v, cu, sc, window=0)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, sc * np.einsum("ihd,ihd->hi", q, k), rtol=1e-15, atol=1e-15)


def test_window_covering_every_sequence_is_global():
    q, k, v, do, cu, sc = _case(3)
    for a, b in zip(oracle.attention(q, k, v, cu, sc, window=max(LENGTHS) - 1), oracle.attention(q, k, v, cu, sc)):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(oracle.attention_backward(do, q, k, v, cu, sc, window=max(LENGTHS) - 1),
                    oracle.attention_backward(do, q, k, v, cu, sc)):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("window", [0, 2, 7])
def test_local_padded_twin(window):
    q, k, v, _, cu, sc = _case(4)
    o, lse = oracle.attention(q, k, v, cu, sc, window=window)
    o2, lse2 = oracle.padded_attention(q, k, v, cu, max(LENGTHS), sc, window=window)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-14)
    of, lf = oracle.attention_first_token(q[cu[:-1]], k, v, cu, sc, window=window)
    of2, lf2 = oracle.padded_attention(q[cu[:-1]], k, v, cu, max(LENGTHS), sc, True, window=window)
    np.testing.assert_allclose(of, of2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lf, lf2, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("window", [1, 4])
def test_local_rows_and_first_token_agree_with_full(window):
    q, k, v, _, cu, sc = _case(5)
    o, lse = oracle.attention(q, k, v, cu, sc, window=window)
    rows = [0, 3, 7, 17, 20, 40, 43]
    orow, lrow = oracle.attention_rows(q, k, v, cu, sc, rows, window=window)
    np.testing.assert_allclose(orow, o[rows], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lrow, lse[:, rows], rtol=1e-14, atol=1e-15)
    of, lf = oracle.attention_first_token(q[cu[:-1]], k, v, cu, sc, window=window)
    np.testing.assert_allclose(of, o[cu[:-1]], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lf, lse[:, cu[:-1]], rtol=1e-14, atol=1e-15)


def test_local_brute_force_python_loops():
    lengths, window = [3, 6], 2
    q, k, v, _, cu, sc = _case(6, lengths, H=1, d=4)
    o, lse = oracle.attention(q, k, v, cu, sc, window=window)
    for b in range(2):
        c0, c1 = int(cu[b]), int(cu[b + 1])
        for i in range(c0, c1):
            keys = [j for j in range(c0, c1) if abs(i - j) <= window]
            s = [sc * sum(q[i, 0, c] * k[j, 0, c] for c in range(4)) for j in keys]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            tot = sum(w)
            for c in range(4):
                assert abs(o[i, 0, c] - sum(wj * v[j, 0, c] for wj, j in zip(w, keys)) / tot) < 1e-13
            assert abs(lse[0, i] - (mx + math.log(tot))) < 1e-13


@pytest.mark.parametrize("window", [0, 2, 6])
def test_local_backward_matches_torch_autograd(window):
    q, k, v, do, cu, sc = _case(7)
    dq, dk, dv = oracle.attention_backward(do, q, k, v, cu, sc, window=window)
    qt, kt, vt = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    out, _ = _torch_dense(qt, kt, vt, cu, window, sc)
    (out * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_local_backward_finite_differences():
    lengths, window = [4, 7], 2
    q, k, v, do, cu, sc = _case(8, lengths, H=1, d=4)
    grads = oracle.attention_backward(do, q, k, v, cu, sc, window=window)

    def f(q_, k_, v_):
        return float(np.sum(do * oracle.attention(q_, k_, v_, cu, sc, window=window)[0]))

    h = 1e-6
    for grad, which in zip(grads, (0, 1, 2)):
        for idx in np.ndindex(*grad.shape):
            a_p, a_m = [q.copy(), k.copy(), v.copy()], [q.copy(), k.copy(), v.copy()]
            a_p[which][idx] += h
            a_m[which][idx] -= h
            assert abs((f(*a_p) - f(*a_m)) / (2 * h) - grad[idx]) < 1e-7 + 1e-6 * abs(grad[idx])


def test_planted_band_off_by_one_is_caught(monkeypatch):
    q, k, v, _, cu, sc = _case(9)
    ref = _torch_dense(*(torch.from_numpy(x) for x in (q, k, v)), cu, 3, sc)[0].numpy()
    np.testing.assert_allclose(oracle.attention(q, k, v, cu, sc, window=3)[0], ref, rtol=1e-12, atol=1e-13)

    def band_strict(rows, cols, window):  # |i - j| < w instead of <= w
        if window is None:
            return None
        i = np.asarray(rows, dtype=np.int64)[:, None]
        j = np.asarray(cols, dtype=np.int64)[None, :]
        return np.abs(i - j) < max(int(window), 1)

    monkeypatch.setattr(oracle, "_band", band_strict)
    assert not np.allclose(oracle.attention(q, k, v, cu, sc, window=3)[0], ref, rtol=1e-12, atol=1e-13)
