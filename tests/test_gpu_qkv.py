"""GPU parity of the fused-QKV calls (pe_varlen_attn_fwd_qkv / _bwd_qkv): the
same kernels reading Q, K, V (and writing dQ, dK, dV) through a row stride of
3*H*d. Each case checks against the fp64 oracle and, bit for bit, against the
calls on separate dense tensors."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, check_lse, check_out, say, to_dev, to_f64
from tests.test_gpu_bwd import check_grad

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")

EDGE = [1, 127, 128, 129, 5, 256, 257, 3, 300, 64, 65, 1, 1, 2, 31, 32, 33, 16, 15, 17, 200]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = [  # dtype, d, max_seq_len: every kernel family
    (W.FP32, 64, 300),    # fp32 one-wave kernels
    (W.FP32, 16, 300),    # generic fp32
    (W.BF16, 64, 300),    # bf16 sequence-aligned 128-row tiles, forward and three-pass backward
    (W.BF16, 128, 300),   # bf16 LDS-DMA forward, head dim 128, generic backward
    (W.BF16, 64, 64),     # bf16 short bound: one-wave forward, single-pass backward
]


@pytest.mark.parametrize("dtype,d,S", CASES)
@pytest.mark.parametrize("window", [-1, 20])
def test_fused_qkv_forward_and_backward(dtype, d, S, window):
    L = np.minimum(EDGE, S)
    w = W.custom(90 + d + S, L, S, 2, d, dtype, with_grad=True)
    say(f"[qkv] {dtype} d={d} S={S} window={window}: N={w.total_tokens}")
    cu_ref, _, N = oracle.layout(w.lengths, w.max_seq_len)
    cu = torch.from_numpy(cu_ref).to(DEV)
    q, k, v, do = (to_dev(x, dtype) for x in (w.q, w.k, w.v, w.dout))
    qkv = torch.stack([q, k, v], dim=1).contiguous()     # [N, 3, H, d]
    code = pe.PE_BF16 if dtype == W.BF16 else pe.PE_FP32
    ws = pe.workspace(pe.pe_attn_bwd_workspace_size(w.num_seqs, N, S, 2, d, code), DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((2, N), float("nan"), device=DEV)
    pe.pe_varlen_attn_fwd_qkv(qkv, cu, w.num_seqs, N, S, w.scale, window, out, lse, ws)
    dqkv = torch.full_like(qkv, float("nan"))
    pe.pe_varlen_attn_bwd_qkv(do, qkv, out, lse, cu, w.num_seqs, N, S, w.scale, window, dqkv, ws)
    # the same on separate dense tensors
    out2, lse2 = torch.empty_like(q), torch.empty_like(lse)
    g2 = [torch.empty_like(q) for _ in range(3)]
    if window < 0:
        pe.pe_varlen_attn_fwd(q, k, v, cu, w.num_seqs, N, S, w.scale, out2, lse2, ws)
        pe.pe_varlen_attn_bwd(do, q, k, v, out2, lse2, cu, w.num_seqs, N, S, w.scale, *g2, ws)
    else:
        pe.pe_varlen_attn_fwd_local(q, k, v, cu, w.num_seqs, N, S, w.scale, window, out2, lse2, ws)
        pe.pe_varlen_attn_bwd_local(do, q, k, v, out2, lse2, cu, w.num_seqs, N, S, w.scale, window, *g2, ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(out2)) and torch.equal(lse, lse2)
    for i in range(3):
        assert torch.equal(_bits(dqkv[:, i].contiguous()), _bits(g2[i])), i
    # against the oracle
    win = None if window < 0 else window
    qd, kd, vd, dod = (W.to_f64(x, dtype) for x in (w.q, w.k, w.v, w.dout))
    o_ref, l_ref = oracle.attention(qd, kd, vd, cu_ref, w.scale, window=win)
    check_out(to_f64(out), o_ref, dtype, "qkv out")
    check_lse(to_f64(lse), l_ref, dtype, "qkv lse")
    out_given = None
    if dtype == W.BF16:
        out_given = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o_ref.astype(np.float32))).astype(np.float64)
    ref = oracle.attention_backward(dod, qd, kd, vd, cu_ref, w.scale, out=out_given, window=win)
    for i, name in enumerate(("dq", "dk", "dv")):
        check_grad(to_f64(dqkv[:, i].contiguous()), ref[i], dtype, f"qkv {name}")
