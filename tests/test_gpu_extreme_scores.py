"""GPU parity of the 16-bit forward on scores far outside the usual range.

Some sequences of a batch get scores near +800 or -800 (a softmax reference
far from zero, probabilities that would overflow or underflow fp32 against
a fixed one), or one key per sequence ~40 log2 units above the rest (an fp16
probability past 65504 against any reference but the running maximum); the
other sequences keep N(0, 1) scores, and several sequences span more than one
128-row tile. Every row is checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, check_lse, check_out, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")

LENGTHS = [700, 33, 1, 300, 129, 450, 64, 200]   # several 128-row tiles, ragged ends, a length-1 sequence
H, D, S = 2, 64, 1024


def _inputs(dtype, kind, seed):
    """The lengths and q, k, v [N, H, d] in the workload encoding of dtype. Sequences
    0, 3 and 5 get extreme scores of the given kind; the others stay N(0, 1)."""
    rng = np.random.default_rng(seed)
    L = np.array(LENGTHS, dtype=np.int32)
    N = int(L.sum())
    q = rng.standard_normal((N, H, D), dtype=np.float32)
    k = rng.standard_normal((N, H, D), dtype=np.float32)
    v = rng.standard_normal((N, H, D), dtype=np.float32)
    u = rng.standard_normal(D).astype(np.float32)
    u /= np.linalg.norm(u)
    cu = np.concatenate([[0], np.cumsum(L)])
    for b in (0, 3, 5):
        r = slice(int(cu[b]), int(cu[b + 1]))
        if kind == "overflow":        # every score near +800: c s ~ +144 in log2 units
            q[r] = 0.3 * q[r] + 28.0 * u
            k[r] = 0.3 * k[r] + 28.0 * u
        elif kind == "underflow":     # every score near -800
            q[r] = 0.3 * q[r] + 28.0 * u
            k[r] = 0.3 * k[r] - 28.0 * u
        else:                         # one key per sequence ~40 log2 units above the rest
            q[r] = q[r] + 10.0 * u
            k[int(cu[b]) + 7 % int(L[b])] += 22.0 * u
    return L, W.to_bits(q, dtype), W.to_bits(k, dtype), W.to_bits(v, dtype)


@pytest.mark.parametrize("dtype,kind,seed", [(W.BF16, "overflow", 61), (W.BF16, "underflow", 62), (W.BF16, "spike", 63),
                                             (W.FP16, "spike", 64), (W.FP16, "underflow", 65)])
def test_extreme_scores_match_the_oracle(dtype, kind, seed):
    L, q, k, v = _inputs(dtype, kind, seed)
    cu_ref, _, N = oracle.layout(L, S)
    say(f"[extreme scores] {dtype} {kind}: N={N}")
    code = pe.PE_BF16 if dtype == W.BF16 else pe.PE_FP16
    cu = torch.from_numpy(cu_ref).to(DEV)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    ws = pe.workspace(pe.pe_attn_workspace_size(len(L), N, H, D, code, False), DEV)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((H, N), float("nan"), device=DEV)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    pe.pe_varlen_attn_fwd(qd, kd, vd, cu, len(L), N, S, scale, out, lse, ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(*(W.to_f64(x, dtype) for x in (q, k, v)), cu_ref, scale)
    check_out(to_f64(out), o_ref, dtype, f"{kind} out")
    check_lse(to_f64(lse), l_ref, dtype, f"{kind} lse")
