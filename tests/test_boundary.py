"""The C ABI on the CPU: the library loads, exports every symbol include/pe.h
declares, sizes workspaces, and rejects bad host arguments before launching
anything (so no GPU is needed). Device pointers here are fake addresses that
the library never dereferences on these paths."""
import ctypes
import os
import re

import pytest

from padding_free_packed_amd import pe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
lib = pe.library()

P = 1 << 20          # a 16-byte aligned fake device address
MIS = P + 4           # misaligned
NUL = None


def _header_functions():
    with open(os.path.join(ROOT, "include", "pe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pe_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = _header_functions()
    assert len(names) == 32
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(pe.EXPORTS) == names


def test_status_strings():
    for s in range(9):
        assert lib.pe_status_string(s).decode().startswith("PE_")
    assert b"unknown" in lib.pe_status_string(99)


def test_tile_rows():
    assert pe.pe_attn_tile_rows() == 128


def test_workspace_sizes():
    # work list: ceil(N/32)+1 int32, rounded to 256 bytes; backward adds a second list and two fp32 [H, N] arrays
    assert pe.pe_attn_workspace_size(4, 1000, 8, 64, pe.PE_FP32, False) == 256
    assert pe.pe_attn_workspace_size(4, 1000, 8, 64, pe.PE_FP32, True) == 256 + 256 + 2 * 32000
    # the fastest backward: fp32 at d 32/64 adds one 4 KiB block per (query tile, key block) slot
    base = pe.pe_attn_workspace_size(4, 1000, 8, 64, pe.PE_FP32, True)
    assert pe.pe_attn_bwd_workspace_size(4, 1000, 64, 8, 64, pe.PE_FP32) == base + 8 * (1000 // 32 + 4) * 2 * 4096
    assert pe.pe_attn_bwd_workspace_size(4, 1000, 64, 8, 64, pe.PE_BF16) == base
    assert pe.pe_attn_bwd_workspace_size(4, 1000, 64, 8, 48, pe.PE_FP32) == base
    assert pe.pe_attn_bwd_workspace_size(0, 1000, 64, 8, 64, pe.PE_FP32) == 0
    # the dS region is offered up to a length bound of 256 (8 blocks per query tile)
    assert pe.pe_attn_bwd_workspace_size(4, 1000, 256, 8, 64, pe.PE_FP32) == base + 8 * (1000 // 32 + 4) * 8 * 4096
    assert pe.pe_attn_bwd_workspace_size(4, 1000, 257, 8, 64, pe.PE_FP32) == base
    big = pe.pe_attn_workspace_size(4096, 368449, 8, 64, pe.PE_FP32, False)
    assert big >= (368449 // 128 + 2) * 4 and big % 256 == 0
    assert pe.pe_pack_workspace_size(8, 64, 16, pe.PE_FP32) >= 256 + 8
    assert pe.pe_pack_workspace_size(0, 64, 16, pe.PE_FP32) == 0


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, cu=P, B=4, N=100, S=64, H=2, d=64, dt=pe.PE_FP32, scale=0.125, out=P, lse=NUL,
             ws=P, wsb=1 << 20)
    a.update(kw)
    return lib.pe_varlen_attn_fwd(a["q"], a["k"], a["v"], a["cu"], a["B"], a["N"], a["S"], a["H"], a["d"],
                                  a["dt"], a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NUL), pe.PE_ERR_NULL),
    (dict(cu=NUL), pe.PE_ERR_NULL),
    (dict(out=NUL), pe.PE_ERR_NULL),
    (dict(B=0), pe.PE_ERR_ARG),
    (dict(S=0), pe.PE_ERR_ARG),
    (dict(H=0), pe.PE_ERR_ARG),
    (dict(N=3), pe.PE_ERR_ARG),                 # fewer tokens than sequences: an empty sequence
    (dict(N=4 * 64 + 1), pe.PE_ERR_ARG),        # more tokens than B * max_seq_len
    (dict(N=2**31, B=2**20, S=2**12), pe.PE_ERR_ARG),   # token count beyond int32
    (dict(d=12), pe.PE_ERR_UNSUPPORTED),        # not a supported multiple of 8
    (dict(d=256), pe.PE_ERR_UNSUPPORTED),
    (dict(dt=5), pe.PE_ERR_UNSUPPORTED),
    (dict(scale=0.0), pe.PE_ERR_ARG),
    (dict(scale=float("nan")), pe.PE_ERR_ARG),
    (dict(q=MIS), pe.PE_ERR_ARG),
    (dict(ws=NUL), pe.PE_ERR_WORKSPACE),
    (dict(wsb=8), pe.PE_ERR_WORKSPACE),
])
def test_fwd_rejects(kw, code):
    assert _fwd(**kw) == code


def test_first_token_rejects():
    f = lib.pe_varlen_attn_fwd_first_token
    assert f(NUL, P, P, P, 4, 100, 64, 2, 64, 0, 0.125, P, NUL, None) == pe.PE_ERR_NULL
    assert f(P, P, P, P, 4, 100, 64, 2, 20, 0, 0.125, P, NUL, None) == pe.PE_ERR_UNSUPPORTED
    assert f(P, P, P, P, 4, 100, 64, 2, 136, 0, 0.125, P, NUL, None) == pe.PE_ERR_UNSUPPORTED
    assert f(P, P, P, P, 4, 100, 64, 2, 64, 0, -1.0, P, NUL, None) == pe.PE_ERR_ARG
    assert f(P, P, P, P, 4, 100, 64, 2, 64, 0, 0.125, P, MIS, None) == pe.PE_ERR_ARG


def test_first_row_and_first_token_backward_reject():
    f = lib.pe_varlen_attn_fwd_first_row
    assert f(NUL, P, P, P, 4, 100, 64, 2, 64, 0, 0.125, P, NUL, None) == pe.PE_ERR_NULL
    assert f(P, P, P, P, 4, 3, 64, 2, 64, 0, 0.125, P, NUL, None) == pe.PE_ERR_ARG
    assert f(P, P, P, P, 4, 100, 64, 2, 64, 0, 0.125, MIS, NUL, None) == pe.PE_ERR_ARG
    b = lib.pe_varlen_attn_bwd_first_token
    ok = [P, P, P, P, P, P, P, 4, 100, 64, 2, 64, 0, 0.125, P, P, P, None]
    for i in (0, 1, 2, 3, 4, 5, 6, 14, 15, 16):  # lse_first is required too
        a = list(ok); a[i] = NUL
        assert b(*a) == pe.PE_ERR_NULL, i
    a = list(ok); a[11] = 44
    assert b(*a) == pe.PE_ERR_UNSUPPORTED
    a = list(ok); a[16] = MIS
    assert b(*a) == pe.PE_ERR_ARG


def test_metadata_calls_reject():
    assert lib.pe_position_ids(NUL, 4, 100, P, P, None) == pe.PE_ERR_NULL
    assert lib.pe_position_ids(P, 0, 100, P, P, None) == pe.PE_ERR_ARG
    assert lib.pe_position_ids(P, 4, 100, MIS, NUL, None) == pe.PE_ERR_ARG
    assert lib.pe_position_ids(P, 4, 100, NUL, NUL, None) == pe.PE_OK    # nothing asked, nothing launched
    assert pe.pe_flatten_workspace_size(0) == 0 and pe.pe_flatten_workspace_size(10) >= 256 + 80 + 160
    n, m = ctypes.c_int64(0), ctypes.c_int64(0)
    f = lib.pe_flatten_packed_metadata
    ok = [P, P, 4, 16, 3, P, P, 64, 8, ctypes.byref(n), ctypes.byref(m), P, 1 << 20, None]
    for i in (0, 1, 6, 9, 10):
        a = list(ok); a[i] = NUL
        assert f(*a) == pe.PE_ERR_NULL, i
    a = list(ok); a[2] = 0
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[4] = -1
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[12] = 16
    assert f(*a) == pe.PE_ERR_WORKSPACE
    g = lib.pe_flatten_document_mask
    assert g(NUL, 4, 16, P, P, 64, 8, ctypes.byref(n), ctypes.byref(m), P, 1 << 20, None) == pe.PE_ERR_NULL
    assert g(P, 4, 0, P, P, 64, 8, ctypes.byref(n), ctypes.byref(m), P, 1 << 20, None) == pe.PE_ERR_ARG
    assert lib.pe_gather_rows(NUL, 4, P, 4, 16, 0, P, None) == pe.PE_ERR_NULL
    assert lib.pe_gather_rows(P, 4, P, 4, 0, 0, P, None) == pe.PE_ERR_ARG
    assert lib.pe_gather_rows(P, 4, P, 4, 16, 7, P, None) == pe.PE_ERR_UNSUPPORTED
    assert lib.pe_scatter_rows(P, NUL, 4, 16, 0, P, 4, None) == pe.PE_ERR_NULL
    assert lib.pe_scatter_rows(P, P, 4, 16, 0, P, -1, None) == pe.PE_ERR_ARG


def test_qkv_rejects():
    f = lib.pe_varlen_attn_fwd_qkv
    ok = [P, P, 4, 100, 64, 2, 64, 0, 0.125, -1, P, NUL, P, 1 << 20, None]
    a = list(ok); a[0] = NUL
    assert f(*a) == pe.PE_ERR_NULL
    a = list(ok); a[9] = -2
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[6] = 20
    assert f(*a) == pe.PE_ERR_UNSUPPORTED
    a = list(ok); a[13] = 8
    assert f(*a) == pe.PE_ERR_WORKSPACE
    b = lib.pe_varlen_attn_bwd_qkv
    okb = [P, P, P, P, P, 4, 100, 64, 2, 64, 0, 0.125, 3, P, P, 1 << 20, None]
    for i in (0, 1, 2, 3, 4, 13):
        a = list(okb); a[i] = NUL
        assert b(*a) == pe.PE_ERR_NULL, i
    a = list(okb); a[12] = -7
    assert b(*a) == pe.PE_ERR_ARG


def test_local_rejects():
    f = lib.pe_varlen_attn_fwd_local
    ok = [P, P, P, P, 4, 100, 64, 2, 64, 0, 0.125, 32, P, NUL, P, 1 << 20, None]
    a = list(ok); a[11] = -1                     # a negative radius
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[0] = NUL
    assert f(*a) == pe.PE_ERR_NULL
    a = list(ok); a[8] = 12
    assert f(*a) == pe.PE_ERR_UNSUPPORTED
    a = list(ok); a[15] = 8
    assert f(*a) == pe.PE_ERR_WORKSPACE
    b = lib.pe_varlen_attn_bwd_local
    okb = [P, P, P, P, P, P, P, 4, 100, 64, 2, 64, 0, 0.125, 32, P, P, P, P, 1 << 20, None]
    a = list(okb); a[14] = -5
    assert b(*a) == pe.PE_ERR_ARG
    a = list(okb); a[5] = NUL
    assert b(*a) == pe.PE_ERR_NULL
    a = list(okb); a[19] = 8
    assert b(*a) == pe.PE_ERR_WORKSPACE


def test_bwd_rejects():
    f = lib.pe_varlen_attn_bwd
    ok = [P, P, P, P, P, P, P, 4, 100, 64, 2, 64, 0, 0.125, P, P, P, P, 1 << 20, None]
    for i in (0, 1, 2, 3, 4, 5, 6, 14, 15, 16):
        a = list(ok)
        a[i] = NUL
        assert f(*a) == pe.PE_ERR_NULL, i
    a = list(ok)
    a[18] = 100
    assert f(*a) == pe.PE_ERR_WORKSPACE
    a = list(ok)
    a[11] = 36          # not a multiple of 8
    assert f(*a) == pe.PE_ERR_UNSUPPORTED


def test_pack_rejects():
    f = lib.pe_pack
    n = ctypes.c_int64(0)
    ok = [P, 4, 64, P, 16, 0, P, P, P, 100, ctypes.byref(n), P, 1 << 20, None]
    a = list(ok); a[0] = NUL
    assert f(*a) == pe.PE_ERR_NULL
    a = list(ok); a[10] = NUL
    assert f(*a) == pe.PE_ERR_NULL
    a = list(ok); a[8] = NUL                     # grid without a packed output
    assert f(*a) == pe.PE_ERR_NULL
    a = list(ok); a[3] = NUL                     # packed output without a grid
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[1] = 0
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[2] = 0
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[9] = -1
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[5] = 7
    assert f(*a) == pe.PE_ERR_UNSUPPORTED
    a = list(ok); a[4] = 0
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[12] = 10
    assert f(*a) == pe.PE_ERR_WORKSPACE
    a = list(ok); a[6] = MIS
    assert f(*a) == pe.PE_ERR_ARG


def test_unpack_and_worklist_reject():
    u = lib.pe_unpack
    assert u(NUL, P, 4, 64, 100, 16, 0, P, None) == pe.PE_ERR_NULL
    assert u(P, P, 4, 64, 3, 16, 0, P, None) == pe.PE_ERR_ARG
    assert u(P, P, 4, 64, 100, 0, 0, P, None) == pe.PE_ERR_ARG
    assert u(P, P, 4, 64, 100, 16, 9, P, None) == pe.PE_ERR_UNSUPPORTED
    w = lib.pe_worklist
    assert w(NUL, 4, 100, 128, P, None) == pe.PE_ERR_NULL
    assert w(P, 4, 100, 0, P, None) == pe.PE_ERR_ARG
    assert w(P, 0, 100, 128, P, None) == pe.PE_ERR_ARG


def test_pack_async_rejects():
    f = lib.pe_pack_async
    ok = [P, 4, 64, P, 16, 0, P, P, P, 100, P, P, 1 << 20, None]
    a = list(ok); a[0] = NUL
    assert f(*a) == pe.PE_ERR_NULL
    a = list(ok); a[10] = NUL                    # no status buffer
    assert f(*a) == pe.PE_ERR_NULL
    a = list(ok); a[8] = NUL
    assert f(*a) == pe.PE_ERR_NULL
    a = list(ok); a[3] = NUL
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[9] = -1
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[1] = 1 << 20; a[2] = 1 << 12  # slots * length bound above INT32_MAX
    assert f(*a) == pe.PE_ERR_ARG
    a = list(ok); a[5] = 7
    assert f(*a) == pe.PE_ERR_UNSUPPORTED
    a = list(ok); a[12] = 10
    assert f(*a) == pe.PE_ERR_WORKSPACE
    a = list(ok); a[10] = MIS
    assert f(*a) == pe.PE_ERR_ARG


def test_forward_graph_rejects_before_any_capture():
    f = lib.pe_forward_graph_create
    g = ctypes.c_void_p(P)
    ws = pe.pe_forward_graph_workspace_size(8, 64, 2, 64, pe.PE_BF16)
    assert pe.pe_forward_graph_workspace_size(256, 512, 2, 64, pe.PE_BF16) > ws > 0
    assert pe.pe_forward_graph_workspace_size(0, 64, 2, 64, pe.PE_BF16) == 0
    ok = [P, 8, 64, P, 2, 64, pe.PE_BF16, 0.125, -1, P, P, P, NUL, P, P, P, ws, ctypes.byref(g)]
    a = list(ok); a[17] = NUL
    assert f(*a) == pe.PE_ERR_NULL
    for i, bad, code in [(0, NUL, pe.PE_ERR_NULL), (3, NUL, pe.PE_ERR_NULL), (14, NUL, pe.PE_ERR_NULL),
                         (8, -2, pe.PE_ERR_ARG), (1, 0, pe.PE_ERR_ARG), (6, 7, pe.PE_ERR_UNSUPPORTED),
                         (5, 28, pe.PE_ERR_UNSUPPORTED), (7, 0.0, pe.PE_ERR_ARG), (16, ws - 1, pe.PE_ERR_WORKSPACE),
                         (13, MIS, pe.PE_ERR_ARG)]:
        a = list(ok); a[i] = bad
        g.value = P
        assert f(*a) == code, i
        assert g.value is None, i                # no handle on an error
    assert lib.pe_graph_launch(NUL, None) == pe.PE_ERR_NULL
    assert lib.pe_graph_destroy(NUL) == pe.PE_OK


def test_noalloc_forward_rejects_batches_beyond_its_scratch_before_touching_the_device():
    assert lib.pe_noalloc_scratch_size() == 1 << 20
    f = lib.pe_varlen_attn_fwd_noalloc
    # a work list of 2^28 / 32 + 5 int32 entries (32 MiB) cannot fit: refused on sizes alone
    assert f(P, P, P, P, 4, 2**28, 2**26, 2, 64, 0, 0.125, P, NUL, None) == pe.PE_ERR_WORKSPACE
    assert f(P, P, P, P, 2**20, 2**24, 64, 2, 64, 1, 0.125, P, NUL, None) == pe.PE_ERR_WORKSPACE
