"""Pins of the oracle's packing metadata: position ids, document ids, NeMo's
metadata flattening (token indices + row-local cumulative lengths, or an indexed
document mask) and the row gather/scatter by flat index.

Anchors: the packed-encoders README's position-id expression and cu_seqlens, the
NeMo indexed-mask example, the GiGL layout (one document per row) through the
already pinned ``layout``/``pack``/``unpack``, brute force, and agreement of the
two flattening routes. A planted mistake is shown to be caught."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_position_ids_match_the_readme_expression():
    g = _golden("packed_encoders_cu_example.json")
    pos = oracle.position_ids(g["cu_seqlens"])
    expr = torch.cat([torch.arange(n) for n in g["lengths"]]).numpy()  # the README's own expression
    assert pos.dtype == np.int64
    np.testing.assert_array_equal(pos, expr)
    np.testing.assert_array_equal(pos, g["position_ids"])


def test_nemo_indexed_mask_example():
    g = _golden("nemo_indexed_mask_example.json")
    flat, cu = oracle.flatten_document_mask(np.array([g["mask_row"]]))
    np.testing.assert_array_equal(cu, g["cu_seqlens"])
    np.testing.assert_array_equal(flat, g["flat_index"])
    np.testing.assert_array_equal(np.diff(cu), g["document_lengths"])
    # and document_ids of that stream is the mask without its padding
    np.testing.assert_array_equal(oracle.document_ids(cu), [x for x in g["mask_row"] if x > 0])


def test_ids_brute_force():
    rng = np.random.default_rng(0)
    L = rng.integers(1, 20, size=30)
    cu = np.concatenate([[0], np.cumsum(L)])
    pos, doc = oracle.position_ids(cu), oracle.document_ids(cu)
    for r in range(int(cu[-1])):
        b = int(np.searchsorted(cu, r, side="right")) - 1
        assert pos[r] == r - cu[b] and doc[r] == b + 1


def _random_rows(seed, rows=12, width=40, max_docs=6):
    """Random valid NeMo batch-major metadata: each row holds 0..max_docs documents back to back."""
    rng = np.random.default_rng(seed)
    ti = -np.ones((rows, width), dtype=np.int32)
    cl = -np.ones((rows, max_docs + 1), dtype=np.int32)
    mask = np.zeros((rows, width), dtype=np.int32)
    for r in range(rows):
        k = int(rng.integers(0, max_docs + 1))
        lens = []
        room = width
        for _ in range(k):
            if room == 0:
                break
            n = int(rng.integers(1, min(room, 12) + 1))
            lens.append(n)
            room -= n
        tot = sum(lens)
        ti[r, :tot] = np.arange(tot)
        cl[r, 0] = 0
        cl[r, 1:len(lens) + 1] = np.cumsum(lens)
        for i, n in enumerate(lens):
            s0 = sum(lens[:i])
            mask[r, s0:s0 + n] = i + 1
    return ti, cl, mask, width


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_two_flattening_routes_agree(seed):
    ti, cl, mask, width = _random_rows(seed)
    f1, c1 = oracle.flatten_packed_metadata(ti, cl, width)
    f2, c2 = oracle.flatten_document_mask(mask)
    np.testing.assert_array_equal(f1, f2)
    np.testing.assert_array_equal(c1, c2)
    assert c1[-1] == len(f1) and np.all(np.diff(c1) > 0)


def test_one_document_per_row_is_the_gigl_layout():
    g = _golden("gigl_pack_example.json")
    L, S = g["lengths"], g["max_seq_len"]
    cu, flat, N = oracle.layout(L, S)
    ti = -np.ones((len(L), S), dtype=np.int32)
    cl = -np.ones((len(L), 2), dtype=np.int32)
    for b, n in enumerate(L):
        ti[b, :n] = np.arange(n)
        cl[b] = [0, n]
    f, c = oracle.flatten_packed_metadata(ti, cl, S)
    np.testing.assert_array_equal(f, flat)
    np.testing.assert_array_equal(c, cu)


def test_gather_scatter_are_pack_unpack_on_the_gigl_layout():
    rng = np.random.default_rng(4)
    L, S, D = [3, 1, 2, 5], 5, 6
    cu, flat, N = oracle.layout(L, S)
    grid = rng.standard_normal((len(L), S, D)).astype(np.float32)
    packed = oracle.pack(grid, flat)
    np.testing.assert_array_equal(oracle.gather_rows(grid.reshape(-1, D), flat).view(np.uint32),
                                  packed.view(np.uint32))
    np.testing.assert_array_equal(oracle.scatter_rows(packed, flat, len(L) * S).reshape(len(L), S, D).view(np.uint32),
                                  oracle.unpack(packed, cu, S).view(np.uint32))


@pytest.mark.parametrize("ti,cl", [
    ([[0, 1, 2, -1]], [[0, 2, -1]]),          # boundaries add up to 2, the row has 3 tokens
    ([[0, 1, -1, 3]], [[0, 2, -1]]),          # a valid index after the -1 padding
    ([[0, 2, 1, -1]], [[0, 3, -1]]),          # token indices out of order
    ([[0, 1, 4, -1]], [[0, 3, -1]]),          # token index outside the row (width 4)
    ([[0, 1, -1, -1]], [[1, 2, -1]]),         # boundaries not starting at 0
    ([[0, 1, -1, -1]], [[0, 1, 1, 2]]),       # an empty document
    ([[0, 1, -1, -1]], [[0, 2, -2]]),         # padding other than -1
])
def test_flatten_rejects_inconsistent_metadata(ti, cl):
    with pytest.raises(oracle.MetadataError):
        oracle.flatten_packed_metadata(np.array(ti), np.array(cl), 4)


@pytest.mark.parametrize("mask", [[[1, 1, 0, 1]], [[2, 2, 0, 0]], [[1, 3, 0, 0]], [[1, 2, 1, 0]], [[1, -1, 0, 0]]])
def test_flatten_mask_rejects_inconsistent_masks(mask):
    with pytest.raises(oracle.MetadataError):
        oracle.flatten_document_mask(np.array(mask))


def test_planted_position_ids_mistake_is_caught():
    g = _golden("packed_encoders_cu_example.json")
    wrong = oracle.position_ids(g["cu_seqlens"]) + 1  # 1-based positions
    assert not np.array_equal(wrong, torch.cat([torch.arange(n) for n in g["lengths"]]).numpy())
