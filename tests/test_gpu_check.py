"""The checked mode (PE_CHECK=1): every attention call first checks cu_seqlens on
the device (cu[0] = 0, every length in [1, max_seq_len], cu[B] <= total_tokens)
and waits for the answer. Offsets that break the contract give PE_ERR_LENGTHS
with nothing launched (outputs keep their poison); valid offsets give the same
bits as the unchecked call. Only the check kernel ever reads the bad offsets."""
import numpy as np
import pytest
import torch

from tests.gpu_util import DEV, say

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")

H, D = 2, 64


def _tensors(n, dtype, seed=0):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(n, H, D, generator=g).to(dtype).to(DEV) for _ in range(4)]


def _fwd(q, k, v, cu, B, N, S, out, lse, code):
    ws = pe.workspace(pe.pe_attn_workspace_size(B, N, H, D, code, True), DEV)
    pe.pe_varlen_attn_fwd(q, k, v, cu, B, N, S, 0.125, out, lse, ws)


@pytest.mark.parametrize("dtype,code", [(torch.float32, pe.PE_FP32), (torch.bfloat16, pe.PE_BF16)])
def test_valid_offsets_give_the_unchecked_bits(dtype, code, monkeypatch):
    L = np.array([5, 33, 1, 64, 17], dtype=np.int32)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(L)]).astype(np.int32)).to(DEV)
    B, N, S = len(L), int(L.sum()), 64
    q, k, v, do = _tensors(N, dtype)
    outs = []
    for checked in (False, True):
        if checked:
            monkeypatch.setenv("PE_CHECK", "1")
        out = torch.empty_like(q)
        lse = torch.empty(H, N, device=DEV)
        _fwd(q, k, v, cu, B, N, S, out, lse, code)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        ws = pe.workspace(pe.pe_attn_workspace_size(B, N, H, D, code, True), DEV)
        pe.pe_varlen_attn_bwd(do, q, k, v, out, lse, cu, B, N, S, 0.125, dq, dk, dv, ws)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (out, lse, dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


# (lengths or offsets, max_seq_len, total_tokens given) breaking one clause of the contract
BAD = {
    "zero_length": ([0, 5, 5, 8], 8, 8),
    "too_long": ([0, 5, 12, 15], 6, 15),
    "offset_not_zero": ([2, 7, 14, 17], 8, 17),
    "past_total_tokens": ([0, 5, 12, 15], 8, 12),
}


@pytest.mark.parametrize("case", sorted(BAD))
def test_bad_offsets_are_refused_before_any_launch(case, monkeypatch):
    cu_l, S, N = BAD[case]
    B = len(cu_l) - 1
    say(f"[check] {case}: cu={cu_l} S={S} N={N}")
    cu = torch.tensor(cu_l, dtype=torch.int32, device=DEV)
    q, k, v, do = _tensors(N, torch.float32, seed=1)
    monkeypatch.setenv("PE_CHECK", "1")
    out = torch.full_like(q, float("nan"))
    lse = torch.full((H, N), float("nan"), device=DEV)
    with pytest.raises(pe.PeError) as e:
        _fwd(q, k, v, cu, B, N, S, out, lse, pe.PE_FP32)
    assert e.value.status == pe.PE_ERR_LENGTHS
    dq = torch.full_like(q, float("nan"))
    ws = pe.workspace(pe.pe_attn_workspace_size(B, N, H, D, pe.PE_FP32, True), DEV)
    with pytest.raises(pe.PeError) as e:
        pe.pe_varlen_attn_bwd(do, q, k, v, q, lse, cu, B, N, S, 0.125, dq, dq.clone(), dq.clone(), ws)
    assert e.value.status == pe.PE_ERR_LENGTHS
    qf = torch.randn(B, H, D, device=DEV)
    of = torch.full_like(qf, float("nan"))
    with pytest.raises(pe.PeError) as e:
        pe.pe_varlen_attn_fwd_first_token(qf, k, v, cu, B, N, S, 0.125, of, None)
    assert e.value.status == pe.PE_ERR_LENGTHS
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(lse).all() and torch.isnan(dq).all() and torch.isnan(of).all()


def test_overlapping_checked_calls(monkeypatch):
    # two threads on their own streams, one with valid offsets and one with a zero length,
    # checking at the same time: each call reads its own answer
    import threading
    monkeypatch.setenv("PE_CHECK", "1")
    S = 8
    cases = {"good": [0, 5, 12, 15], "bad": [0, 5, 5, 8]}
    results = {}

    def worker(name):
        cu_l = cases[name]
        B, N = len(cu_l) - 1, cu_l[-1]
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            cu = torch.tensor(cu_l, dtype=torch.int32, device=DEV)
            q, k, v, _ = _tensors(N, torch.float32, seed=2)
            out = torch.empty_like(q)
            lse = torch.empty(H, N, device=DEV)
            ws = pe.workspace(pe.pe_attn_workspace_size(B, N, H, D, pe.PE_FP32, False), DEV)
            got = []
            for _ in range(40):
                try:
                    pe.pe_varlen_attn_fwd(q, k, v, cu, B, N, S, 0.125, out, lse, ws)
                    got.append(pe.PE_OK)
                except pe.PeError as e:
                    got.append(e.status)
            stream.synchronize()
        results[name] = got

    threads = [threading.Thread(target=worker, args=(n,)) for n in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert results["good"] == [pe.PE_OK] * 40
    assert results["bad"] == [pe.PE_ERR_LENGTHS] * 40
