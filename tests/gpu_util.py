"""Shared pieces of the GPU tests: moving workload arrays to the device and
back, and the tolerance checks against the fp64 oracle.

Tolerances (written here once, used by every parity test):
* fp32: max |gpu - ref| <= 1e-5, and |gpu - ref| / |ref| <= 1e-4 wherever
  |ref| >= 0.1 (below that the absolute bound governs);
* bf16 or fp16 in / fp32 accumulate: max |gpu - ref| <= 2e-2, and the cosine between
  the GPU and oracle vectors of every token row (all heads and head dims of
  that row) >= 0.999 for rows whose oracle norm exceeds 1e-4; a row at or below
  that norm (the exactly-zero dQ and dK of a length-1 sequence, or a row that
  cancels to the level of fp32 accumulation error) has no meaningful direction
  and must instead come back with a norm of at most 2e-3 (a wrong row of a few
  hundred elements inside the 2e-2 element bound has a norm of up to ~0.5);
* log-sum-exp (always fp32): |delta| <= 1e-5 * max(1, |lse|) for fp32 inputs,
  |delta| <= 1e-3 for bf16 or fp16 inputs;
  (fp16 is held to the bf16 bar: the same 16-bit storage with fp32
  accumulation, and 8 times finer rounding;)
* integer and byte outputs: bit-exact.
"""
import sys

import numpy as np
import torch

from padding_free_packed_amd import workloads as W

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


TORCH_DTYPE = {W.FP32: torch.float32, W.BF16: torch.bfloat16, W.FP16: torch.float16}


def pe_code(dtype: str) -> int:
    from padding_free_packed_amd import pe
    return {W.FP32: pe.PE_FP32, W.BF16: pe.PE_BF16, W.FP16: pe.PE_FP16}[dtype]


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if W.is16(dtype):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(TORCH_DTYPE[dtype]).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def from_dev(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_f64(t: torch.Tensor) -> np.ndarray:
    a = from_dev(t)
    if t.dtype == torch.float16:
        return W.f16_bits_to_f32(a).astype(np.float64)
    return W.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def check_out(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = "out"):
    """gpu, ref: float64 arrays whose first axis is the token (or query) row."""
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite values"
    err = np.abs(gpu - ref)
    if dtype == W.FP32:
        assert err.max() <= 1e-5, f"{what}: max abs err {err.max():.3e} > 1e-5"
        big = np.abs(ref) >= 0.1
        if big.any():
            rel = (err[big] / np.abs(ref[big])).max()
            assert rel <= 1e-4, f"{what}: max rel err {rel:.3e} > 1e-4"
    else:
        assert err.max() <= 2e-2, f"{what}: max abs err {err.max():.3e} > 2e-2"
        g = gpu.reshape(gpu.shape[0], -1)
        r = ref.reshape(ref.shape[0], -1)
        c, i, nrm, e = min_cosine(g, r, where=True)
        assert c >= 0.999, f"{what}: min per-token cosine {c:.6f} < 0.999 at row {i} (ref norm {nrm:.4g}, max err {e:.3g})"
    return float(err.max())


COS_MIN_NORM = 1e-4     # rows with a smaller reference norm are checked by their norm instead
SMALL_ROW_NORM = 2e-3    # the largest GPU norm such a row may have


def min_cosine(g: np.ndarray, r: np.ndarray, where: bool = False):
    """Smallest per-row cosine over rows whose reference norm exceeds COS_MIN_NORM
    (with where=True also the row index, its reference norm and max abs error).
    Rows at or below that reference norm must have a GPU norm of at most
    SMALL_ROW_NORM (asserted here)."""
    ng, nr = np.linalg.norm(g, axis=1), np.linalg.norm(r, axis=1)
    keep = nr > COS_MIN_NORM
    small = ~keep
    if small.any():
        j = int(np.argmax(np.where(small, ng, -1.0)))
        assert ng[j] <= SMALL_ROW_NORM, f"row {j}: reference norm {nr[j]:.3g} but GPU norm {ng[j]:.3g}"
    if not keep.any():
        return (1.0, -1, 0.0, 0.0) if where else 1.0
    cos = np.where(keep, (g * r).sum(1) / np.maximum(ng * nr, 1e-300), 2.0)
    i = int(np.argmin(cos))
    if where:
        return float(cos[i]), i, float(nr[i]), float(np.abs(g[i] - r[i]).max())
    return float(cos[i])


def check_lse(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = "lse"):
    assert gpu.shape == ref.shape
    assert np.isfinite(gpu).all(), f"{what}: non-finite values"
    d = np.abs(gpu - ref)
    if dtype == W.FP32:
        bound = 1e-5 * np.maximum(1.0, np.abs(ref))
    else:
        bound = np.full_like(ref, 1e-3)
    assert (d <= bound).all(), f"{what}: max |delta| {d.max():.3e}"
    return float(d.max())


def sample_rows(cu: np.ndarray, tile: int, n_random: int, seed: int):
    """Rows to check at full size: first/last rows, tile edges, sequence edges,
    every row of the longest sequence's first and last tile, and random rows."""
    cu = np.asarray(cu, dtype=np.int64)
    N = int(cu[-1])
    rng = np.random.default_rng(seed)
    rows = {0, 1, N - 1, N - 2}
    for t in (1, 2, N // tile // 2, N // tile - 1):
        for r in (t * tile - 1, t * tile, t * tile + 1):
            if 0 <= r < N:
                rows.add(r)
    L = cu[1:] - cu[:-1]
    b = int(np.argmax(L))
    for r in list(range(int(cu[b]), min(int(cu[b]) + 40, int(cu[b + 1])))) + \
            list(range(max(int(cu[b + 1]) - 40, int(cu[b])), int(cu[b + 1]))):
        rows.add(r)
    for bb in rng.integers(0, len(L), size=16):
        rows.update({int(cu[bb]), int(cu[bb + 1]) - 1})
    rows.update(int(x) for x in rng.integers(0, N, size=n_random))
    return sorted(rows)
