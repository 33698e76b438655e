"""pe_varlen_attn_fwd_noalloc (the forward whose work list lives in the library's
fixed scratch array) against pe_varlen_attn_fwd with a caller workspace: the same
kernels on the same list, so out and lse must agree bit for bit; two calls in a
row, the second on a smaller batch (the array keeps the first call's list), for
each work-list kind (fp32 32-row tiles, bf16 sequence-aligned 128-row tiles, packed 128-row
tiles). The first batch of each kind is also checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, check_lse, check_out, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


CASES = [  # dtype, head dim, length bound: the three work-list kinds
    (W.FP32, 64, 300),   # sequence-aligned 32-row tiles
    (W.BF16, 64, 300),   # sequence-aligned 128-row tiles
    (W.BF16, 64, 64),    # packed 128-row tiles
    (W.FP16, 40, 300),   # packed 128-row tiles, generic kernel
]


@pytest.mark.parametrize("dtype,d,S", CASES)
def test_noalloc_forward_matches_the_workspace_forward(dtype, d, S):
    rng = np.random.default_rng(90 + d + S)
    big = np.concatenate([[S, 1, S - 1], rng.integers(1, S + 1, size=400)]).astype(np.int32)
    small = rng.integers(1, S + 1, size=37).astype(np.int32)
    for rep, L in enumerate((big, small)):
        w = W.custom(91 + rep + d, L, S, 3, d, dtype)
        cu_ref, _, N = oracle.layout(w.lengths, S)
        say(f"[noalloc] {dtype} d={d} S={S} call {rep}: B={w.num_seqs} N={N}")
        cu = torch.from_numpy(cu_ref).to(DEV)
        q, k, v = (to_dev(x, dtype) for x in (w.q, w.k, w.v))
        code = {W.FP32: pe.PE_FP32, W.BF16: pe.PE_BF16, W.FP16: pe.PE_FP16}[dtype]
        ws = pe.workspace(pe.pe_attn_workspace_size(w.num_seqs, N, 3, d, code, False), DEV)
        assert ws.numel() <= pe.pe_noalloc_scratch_size()
        out_a, out_b = torch.full_like(q, float("nan")), torch.full_like(q, float("nan"))
        lse_a = torch.full((3, N), float("nan"), device=DEV)
        lse_b = torch.full((3, N), float("nan"), device=DEV)
        pe.pe_varlen_attn_fwd_noalloc(q, k, v, cu, w.num_seqs, N, S, w.scale, out_a, lse_a)
        pe.pe_varlen_attn_fwd(q, k, v, cu, w.num_seqs, N, S, w.scale, out_b, lse_b, ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_a), _bits(out_b))
        assert torch.equal(lse_a, lse_b)
        if rep == 0:
            o_ref, l_ref = oracle.attention(*(W.to_f64(x, dtype) for x in (w.q, w.k, w.v)), cu_ref, w.scale)
            check_out(to_f64(out_a), o_ref, dtype, "noalloc out")
            check_lse(to_f64(lse_a), l_ref, dtype, "noalloc lse")
