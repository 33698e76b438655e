"""GPU parity (bit-exact) of the packing-metadata calls: position and document
ids, NeMo metadata flattening in both forms with its error and capacity
protocol, row gather/scatter by flat index, and the whole chain feeding the
attention forward."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, check_lse, check_out, from_dev, say, to_dev, to_f64
from tests.test_oracle_metadata import _random_rows

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


@pytest.mark.parametrize("name", ["tiny", "graph_transformer", "short_query", "ones", "single"])
def test_position_and_document_ids(name):
    L = {"tiny": W.tiny().lengths, "graph_transformer": W.graph_transformer(False, False).lengths,
         "short_query": W.random_lengths(2, 32768, 8, 48), "ones": np.ones(777, dtype=np.int32),
         "single": np.array([5000])}[name]
    cu = _cu(L)
    N = int(cu[-1])
    say(f"[ids] {name}: B={len(L)} N={N}")
    pos = torch.full((N,), -7, dtype=torch.int64, device=DEV)
    doc = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    pe.pe_position_ids(torch.from_numpy(cu).to(DEV), len(L), N, pos, doc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pos.cpu().numpy(), oracle.position_ids(cu))
    np.testing.assert_array_equal(doc.cpu().numpy(), oracle.document_ids(cu))


def _flatten_gpu(ti, cl, mask, width, cap=None, dcap=None):
    rows = ti.shape[0]
    ws = pe.workspace(pe.pe_flatten_workspace_size(rows), DEV)
    res = {}
    for form in ("meta", "mask"):
        n_ref = int((ti >= 0).sum())
        d_ref = int(np.maximum((cl >= 0).sum(1) - 1, 0).sum())
        flat = torch.full((n_ref if cap is None else cap,), -5, dtype=torch.int64, device=DEV)
        cu = torch.full(((d_ref if dcap is None else dcap) + 1,), -5, dtype=torch.int32, device=DEV)
        if form == "meta":
            got = pe.pe_flatten_packed_metadata(torch.from_numpy(ti).to(DEV), torch.from_numpy(cl).to(DEV), flat, cu,
                                                ws)
        else:
            got = pe.pe_flatten_document_mask(torch.from_numpy(mask).to(DEV), flat, cu, ws)
        torch.cuda.synchronize()
        res[form] = (got, flat.cpu().numpy(), cu.cpu().numpy())
    return res


@pytest.mark.parametrize("seed,rows", [(1, 12), (2, 1500), (3, 2500)])
def test_flatten_both_forms_bit_exact(seed, rows):
    ti, cl, mask, width = _random_rows(seed, rows=rows, width=96, max_docs=8)
    f_ref, c_ref = oracle.flatten_packed_metadata(ti, cl, width)
    for form, (got, flat, cu) in _flatten_gpu(ti, cl, mask, width).items():
        assert got == (len(f_ref), len(c_ref) - 1), form
        np.testing.assert_array_equal(flat, f_ref, err_msg=form)
        np.testing.assert_array_equal(cu, c_ref, err_msg=form)


def test_flatten_capacity_protocol():
    ti, cl, mask, width = _random_rows(4, rows=40, width=64)
    f_ref, c_ref = oracle.flatten_packed_metadata(ti, cl, width)
    ws = pe.workspace(pe.pe_flatten_workspace_size(40), DEV)
    flat = torch.full((len(f_ref) - 1,), -5, dtype=torch.int64, device=DEV)
    cu = torch.full((len(c_ref),), -5, dtype=torch.int32, device=DEV)
    with pytest.raises(pe.PeError) as ei:
        pe.pe_flatten_packed_metadata(torch.from_numpy(ti).to(DEV), torch.from_numpy(cl).to(DEV), flat, cu, ws)
    assert ei.value.status == pe.PE_ERR_CAPACITY and ei.value.total_tokens == len(f_ref)
    assert (flat.cpu().numpy() == -5).all() and (cu.cpu().numpy() == -5).all()  # outputs untouched


BAD_META = [
    ([[0, 1, 2, -1]], [[0, 2, -1]]),
    ([[0, 1, -1, 3]], [[0, 2, -1]]),
    ([[0, 2, 1, -1]], [[0, 3, -1]]),
    ([[0, 1, 4, -1]], [[0, 3, -1]]),
    ([[0, 1, -1, -1]], [[1, 2, -1]]),
    ([[0, 1, -1, -1]], [[0, 1, 1, 2]]),
    ([[0, 1, -1, -1]], [[0, 2, -2]]),
]


@pytest.mark.parametrize("k", range(len(BAD_META)))
def test_flatten_rejects_what_the_oracle_rejects(k):
    ti, cl = (np.array(x, dtype=np.int32) for x in BAD_META[k])
    good_ti, good_cl, _, _ = _random_rows(5, rows=3, width=4, max_docs=3)
    ti = np.concatenate([good_ti, ti])          # the bad row after good ones
    cl = np.concatenate([good_cl[:, :cl.shape[1]] if good_cl.shape[1] >= cl.shape[1] else
                         np.pad(good_cl, ((0, 0), (0, cl.shape[1] - good_cl.shape[1])), constant_values=-1), cl])
    with pytest.raises(oracle.MetadataError):
        oracle.flatten_packed_metadata(ti, cl, 4)
    ws = pe.workspace(pe.pe_flatten_workspace_size(ti.shape[0]), DEV)
    flat = torch.zeros(64, dtype=torch.int64, device=DEV)
    cu = torch.zeros(65, dtype=torch.int32, device=DEV)
    with pytest.raises(pe.PeError) as ei:
        pe.pe_flatten_packed_metadata(torch.from_numpy(ti).to(DEV), torch.from_numpy(cl).to(DEV), flat, cu, ws)
    assert ei.value.status == pe.PE_ERR_METADATA


@pytest.mark.parametrize("mask", [[[1, 1, 0, 1]], [[2, 2, 0, 0]], [[1, 3, 0, 0]], [[1, 2, 1, 0]], [[1, -1, 0, 0]]])
def test_flatten_mask_rejects(mask):
    m = np.array(mask, dtype=np.int32)
    with pytest.raises(oracle.MetadataError):
        oracle.flatten_document_mask(m)
    ws = pe.workspace(pe.pe_flatten_workspace_size(1), DEV)
    with pytest.raises(pe.PeError) as ei:
        pe.pe_flatten_document_mask(torch.from_numpy(m).to(DEV), torch.zeros(8, dtype=torch.int64, device=DEV),
                                    torch.zeros(9, dtype=torch.int32, device=DEV), ws)
    assert ei.value.status == pe.PE_ERR_METADATA


@pytest.mark.parametrize("dtype,row_elems", [(torch.float32, 512), (torch.bfloat16, 768), (torch.bfloat16, 3),
                                             (torch.float32, 1)])
def test_gather_scatter_bit_exact(dtype, row_elems):
    rng = np.random.default_rng(row_elems)
    rows, n = 900, 700
    flat_np = rng.choice(rows, size=n, replace=False).astype(np.int64)
    flat_np[::97] = rows + 5      # out of range: a zero row on gather, skipped on scatter
    src = torch.randn(rows, row_elems, device=DEV).to(dtype)
    flat = torch.from_numpy(flat_np).to(DEV)
    g = torch.full((n, row_elems), float("nan"), device=DEV).to(dtype)
    pe.pe_gather_rows(src, flat, g)
    s = torch.full((rows, row_elems), float("nan"), device=DEV).to(dtype)
    pe.pe_scatter_rows(g, flat, s)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    src_b = bits(src)
    ok = flat_np < rows
    exp_g = np.zeros((n, row_elems), dtype=src_b.dtype)
    exp_g[ok] = oracle.gather_rows(src_b, flat_np[ok])
    np.testing.assert_array_equal(bits(g), exp_g)
    exp_s = oracle.scatter_rows(exp_g[ok], flat_np[ok], rows)
    np.testing.assert_array_equal(bits(s), exp_s)


def test_nemo_rows_through_attention():
    """Several documents per row: flatten the mask, gather Q/K/V rows of the padded
    grid, attend per document, scatter back; against the oracle on the same chain."""
    ti, cl, mask, width = _random_rows(6, rows=64, width=128, max_docs=5)
    H, d = 4, 64
    rng = np.random.default_rng(7)
    grids = [W.f32_to_bf16_bits(rng.standard_normal((64 * width, H, d), dtype=np.float32)) for _ in range(3)]
    f_ref, c_ref = oracle.flatten_document_mask(mask)
    N, B = len(f_ref), len(c_ref) - 1
    ws = pe.workspace(pe.pe_flatten_workspace_size(64), DEV)
    flat = torch.empty(N, dtype=torch.int64, device=DEV)
    cu = torch.empty(B + 1, dtype=torch.int32, device=DEV)
    assert pe.pe_flatten_document_mask(torch.from_numpy(mask).to(DEV), flat, cu, ws) == (N, B)
    dev_grids = [to_dev(g, W.BF16) for g in grids]
    q, k, v = (torch.empty(N, H, d, dtype=torch.bfloat16, device=DEV) for _ in range(3))
    for src, dst in zip(dev_grids, (q, k, v)):
        pe.pe_gather_rows(src, flat, dst)
    out = torch.empty_like(q)
    lse = torch.empty(H, N, device=DEV)
    aws = pe.workspace(pe.pe_attn_workspace_size(B, N, H, d, pe.PE_BF16, False), DEV)
    S = int(np.diff(c_ref).max())
    pe.pe_varlen_attn_fwd(q, k, v, cu, B, N, S, 0.125, out, lse, aws)
    grid_out = torch.empty_like(dev_grids[0])
    pe.pe_scatter_rows(out, flat, grid_out)
    torch.cuda.synchronize()
    qf, kf, vf = (W.to_f64(oracle.gather_rows(g, f_ref), W.BF16) for g in grids)
    o_ref, l_ref = oracle.attention(qf, kf, vf, c_ref, 0.125)
    check_out(to_f64(out), o_ref, W.BF16, "nemo rows out")
    check_lse(to_f64(lse), l_ref, W.BF16, "nemo rows lse")
    got = from_dev(grid_out)
    assert (got[np.setdiff1d(np.arange(64 * width), f_ref)] == 0).all()   # padding rows are +0.0
    np.testing.assert_array_equal(got[f_ref], from_dev(out))
