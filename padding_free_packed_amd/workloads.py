"""Seeded synthetic workloads shared by the oracle side and the HIP side.

This module only draws inputs. It holds none of the attention, packing or
gradient arithmetic: both implementations receive the same arrays from here and
compute on their own.

Every workload follows one recipe:

* ``rng = numpy.random.default_rng(seed)``;
* draw the sequence lengths first, then (if the workload has one) the padded
  grid ``[B, S, D]``, then Q, K, V and dO, each ``rng.standard_normal(shape,
  dtype=float32)`` with shape ``[N, H, d]``;
* "uniform int in [a, b]" is ``rng.integers(a, b + 1)``; "round" is
  ``numpy.rint`` (half to even), clipped after rounding;
* bf16 and fp16 values are the round-to-nearest-even images of those fp32
  draws (bf16 produced on the bit patterns below, fp16 by numpy's IEEE
  conversion); arrays of either are ``uint16`` bit arrays;
* padding cells of a grid hold NaN, so a pack that reads padding is caught.

The length distributions and shapes are those of the workloads described on the
GiGL packed-attention page (graph-transformer sequences of at most 256 tokens,
about 90 real, hidden 512 in 8 heads) and the packed-encoders page (queries of
about 30 tokens, documents of hundreds to thousands, contrastive batches that
mix both, hidden 768 in 12 heads and 1024 in 16 heads).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FP32 = "fp32"
BF16 = "bf16"
FP16 = "fp16"

BF16_NAN = np.uint16(0x7FC0)
FP16_NAN = np.uint16(0x7E00)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to IEEE fp16 (nearest, ties to even) and return the uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of fp16 bit patterns to fp32."""
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def is16(dtype: str) -> bool:
    return dtype in (BF16, FP16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> the workload encoding of dtype (fp32 values, or 16-bit bits)."""
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    if dtype == FP16:
        return f32_to_f16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a workload array (fp32 values or 16-bit bits) to float64."""
    if dtype == BF16:
        return bf16_bits_to_f32(x).astype(np.float64)
    if dtype == FP16:
        return f16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


@dataclass
class Workload:
    name: str
    dtype: str
    lengths: np.ndarray            # int32 [B]
    max_seq_len: int               # S, the grid width and the bound on every length
    num_heads: int
    head_dim: int
    scale: float                   # softmax scale as the fp32 value both sides receive
    q: np.ndarray | None = None    # [N, H, d] fp32 values or bf16 bits
    k: np.ndarray | None = None
    v: np.ndarray | None = None
    dout: np.ndarray | None = None
    grid: np.ndarray | None = None  # [B, S, D] with NaN padding, D = H * d
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.lengths.astype(np.int64).sum())

    @property
    def row_elems(self) -> int:
        return self.num_heads * self.head_dim


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bits(x, dtype) if is16(dtype) else x


def _draw_grid(rng, lengths, S, D, dtype):
    g = rng.standard_normal((lengths.shape[0], S, D), dtype=np.float32)
    g = _cast(g, dtype)
    pad = np.arange(S)[None, :] >= lengths[:, None]
    g[pad] = {BF16: BF16_NAN, FP16: FP16_NAN}.get(dtype, np.float32("nan"))
    return g


def _draw_tensors(rng, N, H, d, dtype, names):
    out = {}
    for nm in names:
        out[nm] = _cast(rng.standard_normal((N, H, d), dtype=np.float32), dtype)
    return out


def _finish(name, dtype, rng, lengths, S, H, d, grid, names):
    lengths = np.asarray(lengths, dtype=np.int32)
    N = int(lengths.astype(np.int64).sum())
    g = _draw_grid(rng, lengths, S, H * d, dtype) if grid else None
    t = _draw_tensors(rng, N, H, d, dtype, names)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    return Workload(name, dtype, lengths, S, H, d, scale, t.get("q"), t.get("k"),
                    t.get("v"), t.get("dout"), g)


# The five standing workloads. Numbers in the names are those of the list of
# configurations this library is measured on. Each draws its lengths first from
# its own seed (so `standing_lengths` gives the same lengths without drawing any
# tensor), then its grid and tensors.

def _lengths_tiny(rng):
    return rng.integers(1, 65, size=8)


def _lengths_graph_transformer(rng):
    return np.clip(np.rint(rng.normal(90.0, 40.0, size=4096)), 1, 256).astype(np.int64)


def _lengths_short_query(rng):
    return rng.integers(8, 49, size=32768)


def _lengths_long_document(rng):
    return np.clip(np.rint(rng.lognormal(np.log(512.0), 0.8, size=1024)), 64, 8192).astype(np.int64)


def _lengths_mixed_training(rng):
    queries = rng.integers(16, 49, size=2048)
    docs = np.clip(np.rint(rng.lognormal(np.log(1024.0), 0.7, size=256)), 128, 8192).astype(np.int64)
    return rng.permutation(np.concatenate([queries, docs]))


# name: (seed, lengths, S, H, d, dtype, has a padded grid, carries dO)
SPECS = {
    "tiny": (0, _lengths_tiny, 64, 2, 8, FP32, True, True),
    "graph_transformer": (1, _lengths_graph_transformer, 256, 8, 64, FP32, True, True),
    "short_query": (2, _lengths_short_query, 48, 12, 64, BF16, True, False),
    "long_document": (3, _lengths_long_document, 8192, 12, 64, BF16, False, False),
    "mixed_training": (4, _lengths_mixed_training, 8192, 16, 64, BF16, False, True),
}


def _standing(name, grid=None, with_grad=None):
    seed, draw, S, H, d, dtype, g, grad = SPECS[name]
    rng = np.random.default_rng(seed)
    lengths = draw(rng)
    g = g if grid is None else grid
    grad = grad if with_grad is None else with_grad
    names = ("q", "k", "v", "dout") if grad else ("q", "k", "v")
    return _finish(name, dtype, rng, lengths, S, H, d, g, names)


def standing_lengths(name) -> Workload:
    """The standing workload `name` with its lengths, shape and scale but no tensors
    (the same lengths as the full workload: they are drawn first from its seed)."""
    seed, draw, S, H, d, dtype, _, _ = SPECS[name]
    lengths = np.asarray(draw(np.random.default_rng(seed)), dtype=np.int32)
    return Workload(name, dtype, lengths, S, H, d, float(np.float32(1.0 / np.sqrt(d))))


def tiny(with_grad: bool = True) -> Workload:
    """8 sequences, lengths uniform in [1, 64], S = 64, 2 heads x 8, fp32, grid [8, 64, 16]."""
    return _standing("tiny", with_grad=with_grad)


def graph_transformer(grid: bool = True, with_grad: bool = True) -> Workload:
    """4096 sequences, lengths round(N(90, 40)) clipped to [1, 256], S = 256, 8 x 64, fp32."""
    return _standing("graph_transformer", grid=grid, with_grad=with_grad)


def short_query(grid: bool = True) -> Workload:
    """32768 sequences, lengths uniform in [8, 48], S = 48, 12 x 64, bf16."""
    return _standing("short_query", grid=grid)


def long_document() -> Workload:
    """1024 sequences, lengths round(lognormal(ln 512, 0.8)) clipped to [64, 8192], S = 8192, 12 x 64, bf16."""
    return _standing("long_document")


def mixed_training() -> Workload:
    """2048 queries U[16, 48] + 256 documents round(lognormal(ln 1024, 0.7)) clipped to [128, 8192],
    shuffled together, S = 8192, 16 x 64, bf16, with dO for the backward."""
    return _standing("mixed_training")


def short_batch(num_seqs: int = 64) -> Workload:
    """The short-query recipe at a serving batch: num_seqs sequences, lengths uniform in
    [8, 48], S = 48, 12 x 64, bf16 (the launch-bound case of a captured bucket forward)."""
    rng = np.random.default_rng(5)
    lengths = rng.integers(8, 49, size=num_seqs)
    return _finish("short_batch", BF16, rng, lengths, 48, 12, 64, False, ("q", "k", "v"))


def nemo_rows(base: Workload, width: int):
    """The documents of `base`, in their order, packed NeMo-style into rows of `width`
    tokens (a document goes to the current row while it fits, else opens a new row).
    Returns the indexed document mask int32 [rows, width] (document i of a row marked i,
    padding 0) and, for each of q, k, v, a padded row grid [rows * width, H, d] holding the
    packed tensors of `base` at the document positions (padding NaN, as the other grids)."""
    rows_of, starts, row, fill = [], [], 0, 0
    for L in base.lengths.astype(np.int64):
        if fill + L > width:
            row, fill = row + 1, 0
        rows_of.append(row)
        starts.append(fill)
        fill += int(L)
    R = row + 1
    mask = np.zeros((R, width), dtype=np.int32)
    dest = np.empty(base.total_tokens, dtype=np.int64)
    pos, per_row = 0, {}
    for b, L in enumerate(base.lengths.astype(np.int64)):
        r, s0 = rows_of[b], starts[b]
        per_row[r] = per_row.get(r, 0) + 1
        mask[r, s0:s0 + L] = per_row[r]
        dest[pos:pos + L] = r * width + s0 + np.arange(L)
        pos += L
    nan = BF16_NAN if base.dtype == BF16 else np.float32("nan")
    grids = {}
    for nm in ("q", "k", "v"):
        x = getattr(base, nm)
        g = np.full((R * width,) + x.shape[1:], nan, dtype=x.dtype)
        g[dest] = x
        grids[nm] = g
    return mask, grids


STANDING = {
    "tiny": tiny,
    "graph_transformer": graph_transformer,
    "short_query": short_query,
    "long_document": long_document,
    "mixed_training": mixed_training,
}


def device_inputs(w: Workload, device, seed: int, grid: bool = False, with_grad: bool = False) -> dict:
    """Q, K, V (and dO, and the padded grid [B, S, D] with NaN padding) of the
    shape and dtype of `w`, drawn on the device by torch's seeded generator:
    N(0, 1) fp32 values rounded to nearest-even in the workload's dtype. Same
    shapes and distributions as the host recipe above, not the same values; for
    timing runs, where drawing the host arrays would take minutes."""
    import torch

    dt = {FP32: torch.float32, BF16: torch.bfloat16, FP16: torch.float16}[w.dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    N, H, d, B, S = w.total_tokens, w.num_heads, w.head_dim, w.num_seqs, w.max_seq_len

    def draw(shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dt)

    out = {}
    if grid:
        g = draw((B, S, H * d))
        pad = torch.arange(S, device=device)[None, :] >= torch.from_numpy(w.lengths).to(device)[:, None]
        g[pad] = float("nan")
        out["grid"] = g
    for nm in (("q", "k", "v", "dout") if with_grad else ("q", "k", "v")):
        out[nm] = draw((N, H, d))
    return out


def custom(seed: int, lengths, max_seq_len: int, num_heads: int, head_dim: int, dtype: str,
           grid: bool = False, with_grad: bool = False, scale: float | None = None) -> Workload:
    """A workload with given lengths (drawn by the caller or fixed) and seeded N(0, 1) tensors."""
    rng = np.random.default_rng(seed)
    names = ("q", "k", "v", "dout") if with_grad else ("q", "k", "v")
    w = _finish(f"custom{seed}", dtype, rng, np.asarray(lengths), max_seq_len, num_heads,
                head_dim, grid, names)
    if scale is not None:
        w.scale = float(np.float32(scale))
    return w


def random_lengths(seed: int, num_seqs: int, lo: int, hi: int) -> np.ndarray:
    """Lengths uniform in [lo, hi], seeded; used for the ragged parity cases."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=num_seqs).astype(np.int32)
