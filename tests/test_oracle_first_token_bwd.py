"""Pins of the oracle's first-token backward.

Independent routes: the full backward (itself pinned) with every output gradient
zero except at the first rows; torch autograd in float64 through the GiGL padded
first-token route (queries placed in the first rows of a zero grid, SDPA with
the finfo.min/2 key bias, first rows kept); finite differences. A planted
mistake (the D term dropped) is shown to be caught.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle

LENGTHS = [1, 5, 13, 3, 2]


def _case(seed, lengths=LENGTHS, H=2, d=8):
    rng = np.random.default_rng(seed)
    N = int(np.sum(lengths))
    B = len(lengths)
    k, v = (rng.standard_normal((N, H, d)) for _ in range(2))
    qf, dof = (rng.standard_normal((B, H, d)) for _ in range(2))
    cu, _, _ = oracle.layout(lengths, max(lengths))
    return qf, k, v, dof, cu, 1.0 / np.sqrt(d)


def test_equals_full_backward_with_first_row_gradients_only():
    qf, k, v, dof, cu, sc = _case(1)
    q = np.zeros_like(k)
    q[cu[:-1]] = qf
    rng = np.random.default_rng(2)
    q += rng.standard_normal(q.shape) * (np.isin(np.arange(k.shape[0]), cu[:-1]) == 0)[:, None, None]
    do = np.zeros_like(k)
    do[cu[:-1]] = dof
    dq_full, dk_full, dv_full = oracle.attention_backward(do, q, k, v, cu, sc)
    dq, dk, dv = oracle.attention_first_token_backward(dof, qf, k, v, cu, sc)
    np.testing.assert_allclose(dq, dq_full[cu[:-1]], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk, dk_full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv, dv_full, rtol=1e-12, atol=1e-14)


def _torch_first_token_route(qf, k, v, cu, S, scale):
    cu = torch.from_numpy(np.asarray(cu, dtype=np.int64))
    lengths = cu[1:] - cu[:-1]
    B = lengths.numel()
    N, H, d = k.shape
    seq = torch.repeat_interleave(torch.arange(B), lengths)
    pos = torch.arange(N) - cu[:-1][seq]
    mask = torch.zeros(B, S, dtype=torch.bool)
    mask[seq, pos] = True
    q = torch.zeros_like(k).index_copy(0, cu[:-1], qf)

    def grid(x):
        return torch.zeros(B, S, H, d, dtype=x.dtype).index_put((seq, pos), x).transpose(1, 2)

    bias = torch.zeros(B, S, dtype=torch.float64).masked_fill(~mask, torch.finfo(torch.float64).min / 2)
    out = F.scaled_dot_product_attention(grid(q), grid(k), grid(v), attn_mask=bias.view(B, 1, 1, S), scale=scale)
    return out.transpose(1, 2)[mask][cu[:-1]]


def test_matches_torch_autograd_of_the_padded_route():
    qf, k, v, dof, cu, sc = _case(3)
    dq, dk, dv = oracle.attention_first_token_backward(dof, qf, k, v, cu, sc)
    qt, kt, vt = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (qf, k, v))
    (_torch_first_token_route(qt, kt, vt, cu, max(LENGTHS), sc) * torch.from_numpy(dof)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-10, atol=1e-12)


def _fd_ok(grads, qf, k, v, dof, cu, sc):
    def f(a, b, c):
        return float(np.sum(dof * oracle.attention_first_token(a, b, c, cu, sc)[0]))

    h = 1e-6
    for grad, which in zip(grads, (0, 1, 2)):
        for idx in np.ndindex(*grad.shape):
            a_p, a_m = [qf.copy(), k.copy(), v.copy()], [qf.copy(), k.copy(), v.copy()]
            a_p[which][idx] += h
            a_m[which][idx] -= h
            if abs((f(*a_p) - f(*a_m)) / (2 * h) - grad[idx]) > 1e-7 + 1e-6 * abs(grad[idx]):
                return False
    return True


def test_finite_differences_and_planted_mistake():
    qf, k, v, dof, cu, sc = _case(4, [4, 1, 6], H=1, d=4)
    grads = oracle.attention_first_token_backward(dof, qf, k, v, cu, sc)
    assert _fd_ok(grads, qf, k, v, dof, cu, sc)
    # planted mistake: the D = <dO, O> term dropped from dS (the output passed as zero)
    wrong = oracle.attention_first_token_backward(dof, qf, k, v, cu, sc, out_first=np.zeros_like(qf))
    assert not _fd_ok(wrong, qf, k, v, dof, cu, sc)


def test_given_output_and_lse_are_used():
    qf, k, v, dof, cu, sc = _case(5)
    o, lse = oracle.attention_first_token(qf, k, v, cu, sc)
    a = oracle.attention_first_token_backward(dof, qf, k, v, cu, sc)
    b = oracle.attention_first_token_backward(dof, qf, k, v, cu, sc, out_first=o, lse_first=lse)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    # a shifted log-sum-exp scales every probability of that (b, h) by exp(-delta)
    lse2 = lse.copy()
    lse2[1, 2] += 0.5
    c = oracle.attention_first_token_backward(dof, qf, k, v, cu, sc, out_first=o, lse_first=lse2)
    c0, c1 = int(cu[2]), int(cu[3])
    np.testing.assert_allclose(c[2][c0:c1, 1], a[2][c0:c1, 1] * np.exp(-0.5), rtol=1e-13)
