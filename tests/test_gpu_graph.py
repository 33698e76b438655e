"""GPU tests of the launch path without host reads: pe_pack_async (bit-exact
layout and rows, device-side error codes that leave no rows), every forward
kernel family with total_tokens given as a capacity above cu[B] (bit-exact
against the exact count, tail rows neither read nor written), and the captured
bucket forward, replayed several times with eager work and synchronisations
between replays, each replay checked bit for bit against the eager calls and
the first against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from padding_free_packed_amd import workloads as W
from tests.gpu_util import DEV, check_lse, check_out, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

pe = pytest.importorskip("padding_free_packed_amd.pe")
graphs = pytest.importorskip("padding_free_packed_amd.graphs")


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def _code(dtype):
    return {torch.bfloat16: pe.PE_BF16, torch.float16: pe.PE_FP16}.get(dtype, pe.PE_FP32)


def _wdt(dtype):
    return {torch.bfloat16: W.BF16, torch.float16: W.FP16}.get(dtype, W.FP32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pack_async_matches_the_oracle(dtype):
    rng = np.random.default_rng(11)
    B, S, D = 300, 77, 24
    L = rng.integers(1, S + 1, size=B).astype(np.int32)
    cu_ref, flat_ref, N = oracle.layout(L, S)
    grid = torch.randn(B, S, D, device=DEV).to(dtype)
    packed_ref = oracle.pack(_bits(grid).cpu().numpy(), flat_ref)
    lengths = torch.from_numpy(L).to(DEV)
    ws = pe.workspace(pe.pe_pack_workspace_size(B, S, D, _code(dtype)), DEV)
    for cap in (N, N + 1000, B * S, 10 * B * S):
        say(f"[pack_async] {dtype} B={B} S={S} N={N} capacity={cap}")
        cu = torch.full((B + 1,), -3, dtype=torch.int32, device=DEV)
        flat = torch.full((cap,), -3, dtype=torch.int64, device=DEV)
        packed = torch.full((cap, D), float("nan"), device=DEV).to(dtype)
        status = torch.full((2,), -3, dtype=torch.int64, device=DEV)
        pe.pe_pack_async(lengths, S, grid, cu, flat, packed, cap, status, ws)
        torch.cuda.synchronize()
        assert status.tolist() == [N, pe.PACK_OK]
        np.testing.assert_array_equal(cu.cpu().numpy(), cu_ref)
        np.testing.assert_array_equal(flat[:N].cpu().numpy(), flat_ref)
        assert (flat[N:] == -3).all()
        np.testing.assert_array_equal(_bits(packed[:N]).cpu().numpy(), packed_ref)
        assert torch.isnan(packed[N:].float()).all()


@pytest.mark.parametrize("case", ["too_long", "zero", "over_capacity"])
def test_pack_async_errors_leave_no_rows(case):
    rng = np.random.default_rng(12)
    B, S, D = 50, 40, 8
    L = rng.integers(1, S + 1, size=B).astype(np.int32)
    cap = B * S
    if case == "too_long":
        L[B - 1] = S + 1            # the last sequence would read past the grid
    elif case == "zero":
        L[3] = 0
    else:
        cap = int(L.sum()) - 1
    say(f"[pack_async error] {case}")
    ws = pe.workspace(pe.pe_pack_workspace_size(B, S, D, pe.PE_FP32), DEV)
    grid = torch.randn(B, S, D, device=DEV)
    cu = torch.full((B + 1,), -3, dtype=torch.int32, device=DEV)
    flat = torch.full((cap,), -3, dtype=torch.int64, device=DEV)
    packed = torch.full((cap, D), 7.0, device=DEV)
    status = torch.zeros(2, dtype=torch.int64, device=DEV)
    pe.pe_pack_async(torch.from_numpy(L).to(DEV), S, grid, cu, flat, packed, cap, status, ws)
    torch.cuda.synchronize()
    expect = pe.PACK_OVER_CAPACITY if case == "over_capacity" else pe.PACK_BAD_LENGTH
    assert status.tolist() == [int(L.sum()), expect]
    assert (cu == 0).all() and (flat == -3).all() and (packed == 7.0).all()


EDGE = [1, 127, 128, 129, 5, 256, 257, 3, 300, 64, 65, 1, 1, 2, 31, 32, 33, 16, 15, 17, 200]

CAP_CASES = [  # dtype, d, max_seq_len: every forward kernel family
    (W.FP32, 64, 300),    # fp32 one-wave kernel
    (W.FP32, 16, 300),    # generic fp32
    (W.BF16, 64, 300),    # bf16 sequence-aligned 128-row-tile kernel
    (W.BF16, 128, 300),   # bf16 LDS-DMA kernel
    (W.BF16, 64, 64),     # generic bf16 (short bound)
]


@pytest.mark.parametrize("dtype,d,S", CAP_CASES)
@pytest.mark.parametrize("window", [-1, 20])
def test_forward_with_a_capacity_row_count(dtype, d, S, window):
    L = np.minimum(EDGE, S)
    H = 2
    w = W.custom(70 + d + S, L, S, H, d, dtype)
    cu_ref, _, N = oracle.layout(w.lengths, w.max_seq_len)
    B = w.num_seqs
    cap = N + min(333, B * S - N)
    say(f"[capacity fwd] {dtype} d={d} S={S} window={window}: N={N} capacity={cap}")
    cu = torch.from_numpy(cu_ref).to(DEV)
    # rows past N hold NaN: a kernel that read one would spread NaN into real rows
    q, k, v = (torch.cat([to_dev(x, dtype), torch.full((cap - N, H, d), float("nan"), device=DEV).to(
        torch.bfloat16 if dtype == W.BF16 else torch.float32)]) for x in (w.q, w.k, w.v))
    code = pe.PE_BF16 if dtype == W.BF16 else pe.PE_FP32
    out_c = torch.full_like(q, 5.0)
    lse_c = torch.full((H, cap), 5.0, device=DEV)
    ws_c = pe.workspace(pe.pe_attn_workspace_size(B, cap, H, d, code, False), DEV)
    out_n = torch.empty_like(q[:N])
    lse_n = torch.empty((H, N), device=DEV)
    ws_n = pe.workspace(pe.pe_attn_workspace_size(B, N, H, d, code, False), DEV)
    if window < 0:
        pe.pe_varlen_attn_fwd(q, k, v, cu, B, cap, S, w.scale, out_c, lse_c, ws_c)
        pe.pe_varlen_attn_fwd(q[:N], k[:N], v[:N], cu, B, N, S, w.scale, out_n, lse_n, ws_n)
    else:
        pe.pe_varlen_attn_fwd_local(q, k, v, cu, B, cap, S, w.scale, window, out_c, lse_c, ws_c)
        pe.pe_varlen_attn_fwd_local(q[:N], k[:N], v[:N], cu, B, N, S, w.scale, window, out_n, lse_n, ws_n)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out_c[:N]), _bits(out_n)) and torch.equal(lse_c[:, :N], lse_n)
    assert (out_c[N:].float() == 5.0).all() and (lse_c[:, N:] == 5.0).all()
    o_ref, l_ref = oracle.attention(*(W.to_f64(x, dtype) for x in (w.q, w.k, w.v)), cu_ref, w.scale,
                                    window=None if window < 0 else window)
    check_out(to_f64(out_c[:N]), o_ref, dtype, "capacity out")
    check_lse(to_f64(lse_c[:, :N]), l_ref, dtype, "capacity lse")


def _eager(bucket, scale, window):
    """The same forward by the eager calls (pe_pack with its host read)."""
    slots, S = bucket.slots, bucket.max_seq_len
    H, d = bucket.out_grid.shape[2:]
    cu, _, packed, n = pe.pack(bucket.lengths, S, bucket.qkv_grid.view(slots, S, -1))
    qkv = packed.view(n, 3, H, d)
    out = torch.empty(n, H, d, dtype=qkv.dtype, device=DEV)
    lse = torch.empty(H, n, device=DEV)
    ws = pe.workspace(pe.pe_attn_workspace_size(slots, n, H, d, _code(qkv.dtype), False), DEV)
    pe.pe_varlen_attn_fwd_qkv(qkv, cu, slots, n, S, scale, window, out, lse, ws)
    grid = torch.empty_like(bucket.out_grid)
    pe.pe_unpack(out, cu, slots, S, n, grid)
    torch.cuda.synchronize()
    return grid, lse, n, cu


GRAPH_CASES = [  # dtype, H, d, window, slots, length bound
    (torch.bfloat16, 12, 64, -1, 64, 48), (torch.float32, 8, 64, -1, 64, 48), (torch.bfloat16, 12, 64, 16, 64, 48),
    (torch.bfloat16, 4, 128, -1, 64, 48),
    # bounds above 128: the 16-bit forward is the LDS-DMA kernel on sequence-aligned tiles
    # of the bucket's capacity rows (lengths crossing 128 and 256, fewer sequences than slots)
    (torch.bfloat16, 4, 64, -1, 16, 300), (torch.bfloat16, 4, 64, 20, 16, 300),
    (torch.float16, 4, 32, -1, 16, 300), (torch.float16, 4, 32, 20, 16, 300),
]


def _to_wdt(x, wdt):
    return W.to_bits(x, wdt) if W.is16(wdt) else x


@pytest.mark.parametrize("dtype,H,d,window,slots,S", GRAPH_CASES)
def test_bucket_graph_replays(dtype, H, d, window, slots, S):
    scale = 1.0 / np.sqrt(d)
    say(f"[graph] {dtype} H={H} d={d} window={window}: bucket ({slots}, {S})")
    bucket = graphs.ForwardBucket(slots, S, H, d, dtype, scale, window, with_lse=True, device=DEV)
    rng = np.random.default_rng(21 + d + H + S)
    wdt = _wdt(dtype)
    try:
        for rep, B in enumerate([slots, slots * 37 // 64, slots, 5, 1]):
            L = rng.integers(8, S + 1, size=B).astype(np.int32)
            L[0] = 1 if rep == 4 else L[0]
            Sb = int(L.max())
            x = rng.standard_normal((B, Sb, 3, H, d), dtype=np.float32)
            xq = _to_wdt(x, wdt)
            got = bucket.run(torch.from_numpy(L).to(DEV), to_dev(xq, wdt))
            torch.cuda.synchronize()
            ref_grid, ref_lse, n, cu = _eager(bucket, scale, window)
            say(f"  replay {rep}: B={B} N={n}")
            assert bucket.status.tolist() == [n, pe.PACK_OK]
            assert torch.equal(_bits(bucket.out_grid), _bits(ref_grid))
            assert torch.equal(bucket.lse[:, :n], ref_lse)
            assert torch.equal(bucket.cu_seqlens, cu)
            if rep in (0, 1):   # against the oracle on the real sequences
                cu_ref = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
                rows = [W.to_f64(np.concatenate([xq[b, :L[b], j] for b in range(B)]), wdt) for j in range(3)]
                o_ref, l_ref = oracle.attention(*rows, cu_ref, scale, window=None if window < 0 else window)
                out_rows = torch.cat([got[b, :L[b]] for b in range(B)])
                check_out(to_f64(out_rows), o_ref, wdt, "graph out")
                check_lse(to_f64(bucket.lse[:, :int(cu_ref[-1])]), l_ref, wdt, "graph lse")
                assert (got[0, L[0]:].float() == 0).all()     # padding positions are +0.0
        # a batch with a length past the bucket's bound: an error code and an all-zero output
        bad = np.full(slots, 3, dtype=np.int32)
        bad[10] = S + 1
        bucket.lengths.copy_(torch.from_numpy(bad))
        bucket.replay()
        torch.cuda.synchronize()
        assert bucket.status.tolist() == [int(bad.sum()), pe.PACK_BAD_LENGTH]
        assert (bucket.out_grid.float() == 0).all()
        # and the next good batch replays correctly
        L = rng.integers(8, S + 1, size=slots).astype(np.int32)
        x = rng.standard_normal((slots, S, 3, H, d), dtype=np.float32)
        bucket.run(torch.from_numpy(L).to(DEV), to_dev(_to_wdt(x, wdt), wdt))
        torch.cuda.synchronize()
        ref_grid, _, n, _ = _eager(bucket, scale, window)
        assert bucket.status.tolist() == [n, pe.PACK_OK]
        assert torch.equal(_bits(bucket.out_grid), _bits(ref_grid))
    finally:
        bucket.close()


@pytest.mark.parametrize("dtype,H,d", [(torch.bfloat16, 12, 64), (torch.float32, 8, 64)])
def test_large_bucket_replays_the_six_kernel_capture(dtype, H, d):
    """A bucket whose work lists exceed what the single-workgroup plan kernel takes
    (here one pack tile per 12 x 64 bf16 row: 300 x 64 = 19,200 entries) is captured
    as scan, two work lists, pack, attention, unpack; its replays match the eager calls
    bit for bit, like the small buckets' four-kernel replays."""
    slots, S = 300, 64
    scale = 1.0 / np.sqrt(d)
    say(f"[graph large] {dtype} H={H} d={d}: bucket ({slots}, {S})")
    bucket = graphs.ForwardBucket(slots, S, H, d, dtype, scale, -1, with_lse=True, device=DEV)
    rng = np.random.default_rng(77 + H)
    wdt = W.BF16 if dtype == torch.bfloat16 else W.FP32
    try:
        for rep, B in enumerate([slots, 123]):
            L = rng.integers(1, S + 1, size=B).astype(np.int32)
            x = rng.standard_normal((B, S, 3, H, d), dtype=np.float32)
            bucket.run(torch.from_numpy(L).to(DEV), to_dev(W.f32_to_bf16_bits(x) if wdt == W.BF16 else x, wdt))
            torch.cuda.synchronize()
            ref_grid, ref_lse, n, cu = _eager(bucket, scale, -1)
            say(f"  replay {rep}: B={B} N={n}")
            assert bucket.status.tolist() == [n, pe.PACK_OK]
            assert torch.equal(_bits(bucket.out_grid), _bits(ref_grid))
            assert torch.equal(bucket.lse[:, :n], ref_lse)
            assert torch.equal(bucket.cu_seqlens, cu)
    finally:
        bucket.close()
