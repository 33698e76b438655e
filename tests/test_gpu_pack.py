"""GPU parity of the packing calls: pe_pack (offsets, flat_index, gather),
pe_unpack and pe_worklist, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")


def _run_pack_unpack(w: W.Workload, label: str):
    say(f"[pack] {label}: B={w.num_seqs} S={w.max_seq_len} D={w.row_elems} {w.dtype}")
    cu_ref, flat_ref, N = oracle.layout(w.lengths, w.max_seq_len)
    lengths = torch.from_numpy(w.lengths.astype(np.int32)).to(DEV)
    grid = to_dev(w.grid, w.dtype)
    cu, flat, packed, n = pe.pack(lengths, w.max_seq_len, grid, capacity=N)
    torch.cuda.synchronize()
    assert n == N
    assert from_dev(cu).tolist() == cu_ref.tolist()
    assert np.array_equal(from_dev(flat), flat_ref)
    packed_ref = oracle.pack(w.grid, flat_ref)
    p = from_dev(packed)
    assert p.view(np.uint8).tobytes() == np.ascontiguousarray(packed_ref).view(np.uint8).tobytes()
    # unpack into a NaN-poisoned grid: every byte must be overwritten
    out = torch.full_like(grid, float("nan"))
    say(f"[unpack] {label}")
    pe.pe_unpack(packed, cu, w.num_seqs, w.max_seq_len, N, out)
    torch.cuda.synchronize()
    g = from_dev(out)
    g_ref = oracle.unpack(packed_ref, cu_ref, w.max_seq_len)
    assert g.view(np.uint8).tobytes() == np.ascontiguousarray(g_ref).view(np.uint8).tobytes()


def test_pack_unpack_tiny():
    _run_pack_unpack(W.tiny(), "tiny")


def test_pack_unpack_gigl_example():
    _run_pack_unpack(W.custom(5, [3, 1, 2], 3, 2, 8, W.FP32, grid=True), "gigl example")


@pytest.mark.parametrize("dtype,H,d", [(W.FP32, 1, 3), (W.BF16, 1, 5), (W.BF16, 3, 4), (W.FP32, 2, 2),
                                       (W.BF16, 12, 64)])
def test_pack_unpack_row_widths(dtype, H, d):
    # row widths of 12, 10, 24, 16 and 1536 bytes exercise every copy unit size
    L = W.random_lengths(7, 57, 1, 40)
    w = W.custom(8, L, 40, H, d, dtype, grid=True)
    _run_pack_unpack(w, f"rows {dtype} {H}x{d}")


def test_pack_unpack_single_and_full():
    _run_pack_unpack(W.custom(9, [1], 1, 1, 8, W.FP32, grid=True), "one token")
    _run_pack_unpack(W.custom(10, [17, 17, 17], 17, 2, 8, W.BF16, grid=True), "all full")


def test_pack_unpack_short_query_full_size():
    _run_pack_unpack(W.short_query(grid=True), "short-query 32768x48x768 bf16")


def test_pack_layout_only_and_capacity():
    w = W.custom(11, W.random_lengths(12, 300, 1, 90), 90, 2, 8, W.FP32, grid=True)
    cu_ref, flat_ref, N = oracle.layout(w.lengths, w.max_seq_len)
    lengths = torch.from_numpy(w.lengths).to(DEV)
    B = w.num_seqs
    say("[pack] layout only / capacity")
    ws = pe.workspace(pe.pe_pack_workspace_size(B, w.max_seq_len, w.row_elems, pe.PE_FP32), DEV)
    cu = torch.empty(B + 1, dtype=torch.int32, device=DEV)
    n = pe.pe_pack(lengths, w.max_seq_len, None, cu, None, None, 0, ws)
    assert n == N and from_dev(cu).tolist() == cu_ref.tolist()
    flat = torch.full((N,), -7, dtype=torch.int64, device=DEV)
    n = pe.pe_pack(lengths, w.max_seq_len, None, cu, flat, None, N, ws)
    assert np.array_equal(from_dev(flat), flat_ref)
    grid = to_dev(w.grid, w.dtype)
    small = torch.empty(N - 1, w.row_elems, device=DEV)
    flat2 = torch.full((N,), -7, dtype=torch.int64, device=DEV)
    with pytest.raises(pe.PeError) as e:
        pe.pe_pack(lengths, w.max_seq_len, grid, cu, flat2, small, N - 1, ws)
    assert e.value.status == pe.PE_ERR_CAPACITY and e.value.total_tokens == N
    assert (from_dev(flat2) == -7).all()       # untouched on a capacity error


@pytest.mark.parametrize("bad", [[3, 0, 2], [3, 4, 2], [-5, 1]])
def test_pack_bad_lengths(bad):
    say(f"[pack] bad lengths {bad}")
    lengths = torch.tensor(bad, dtype=torch.int32, device=DEV)
    ws = pe.workspace(pe.pe_pack_workspace_size(len(bad), 3, 1, pe.PE_FP32), DEV)
    cu = torch.empty(len(bad) + 1, dtype=torch.int32, device=DEV)
    with pytest.raises(pe.PeError) as e:
        pe.pe_pack(lengths, 3, None, cu, None, None, 0, ws)
    assert e.value.status == pe.PE_ERR_LENGTHS


@pytest.mark.parametrize("R", [1, 7, 128, 1000])
def test_worklist(R):
    L = W.random_lengths(13, 777, 1, 300)
    cu_ref, _, N = oracle.layout(L, 300)
    say(f"[worklist] R={R} N={N}")
    cu = torch.from_numpy(cu_ref).to(DEV)
    T = (N + R - 1) // R
    items = torch.full((T + 1,), -1, dtype=torch.int32, device=DEV)
    pe.pe_worklist(cu, len(L), N, R, items)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(items), oracle.worklist(cu_ref, R))


@pytest.mark.parametrize("B", [8191, 8192, 12345, 100000])
def test_pack_layout_many_sequences(B):
    # from 8192 sequences on the scan runs over many workgroups (4096 lengths each, two
    # launches): offsets, a length error in a late workgroup, and (pe_pack_async) the
    # rejected batch that must leave every offset 0
    S = 90
    L = W.random_lengths(14 + B, B, 1, S)
    cu_ref, _, N = oracle.layout(L, S)
    say(f"[pack] layout of {B} sequences")
    ws = pe.workspace(pe.pe_pack_workspace_size(B, S, 1, pe.PE_FP32), DEV)
    cu = torch.full((B + 1,), -3, dtype=torch.int32, device=DEV)
    n = pe.pe_pack(torch.from_numpy(L).to(DEV), S, None, cu, None, None, 0, ws)
    assert n == N and from_dev(cu).tolist() == cu_ref.tolist()
    bad = L.copy()
    bad[B - 5] = 0
    with pytest.raises(pe.PeError) as e:
        pe.pe_pack(torch.from_numpy(bad).to(DEV), S, None, cu, None, None, 0, ws)
    assert e.value.status == pe.PE_ERR_LENGTHS
    # the running sum of the given values, as the call documents
    assert from_dev(cu).tolist() == np.concatenate([[0], np.cumsum(bad.astype(np.int64))]).tolist()
    for lengths, cap, code in ((L, N, pe.PACK_OK), (bad, B * S, pe.PACK_BAD_LENGTH), (L, N - 1, pe.PACK_OVER_CAPACITY)):
        cu = torch.full((B + 1,), -3, dtype=torch.int32, device=DEV)
        flat = torch.full((max(cap, 1),), -3, dtype=torch.int64, device=DEV)
        status = torch.full((2,), -3, dtype=torch.int64, device=DEV)
        pe.pe_pack_async(torch.from_numpy(lengths).to(DEV), S, None, cu, flat, None, cap, status, ws)
        torch.cuda.synchronize()
        assert status.tolist() == [int(lengths.astype(np.int64).sum()), code]
        if code == pe.PACK_OK:
            assert from_dev(cu).tolist() == cu_ref.tolist()
        else:
            assert (cu == 0).all() and (flat == -3).all()
