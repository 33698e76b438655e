"""Python binding of ``libpe.so`` (include/pe.h): argument marshalling only.

Each ``pe_*`` function takes torch tensors (device memory) and host ints, passes
their pointers and the current HIP stream to the C function of the same name,
and raises :class:`PeError` on any status other than ``PE_OK``. Every step of
the computation runs in the library's HIP kernels; nothing here computes.

Loading fails loudly if the library has not been built
(``python -m padding_free_packed_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpe.so")

PE_OK, PE_ERR_NULL, PE_ERR_ARG, PE_ERR_UNSUPPORTED, PE_ERR_LENGTHS, PE_ERR_CAPACITY, \
    PE_ERR_WORKSPACE, PE_ERR_HIP, PE_ERR_METADATA = range(9)
PE_FP32, PE_BF16, PE_FP16 = 0, 1, 2

EXPORTS = (
    "pe_status_string", "pe_attn_tile_rows", "pe_pack_workspace_size", "pe_pack", "pe_unpack",
    "pe_worklist", "pe_attn_workspace_size", "pe_varlen_attn_fwd", "pe_varlen_attn_fwd_first_token",
    "pe_varlen_attn_bwd", "pe_varlen_attn_fwd_local", "pe_varlen_attn_bwd_local", "pe_varlen_attn_fwd_first_row",
    "pe_varlen_attn_bwd_first_token", "pe_position_ids", "pe_flatten_workspace_size", "pe_flatten_packed_metadata",
    "pe_flatten_document_mask", "pe_gather_rows", "pe_scatter_rows", "pe_varlen_attn_fwd_qkv",
    "pe_varlen_attn_bwd_qkv", "pe_timing_enable", "pe_timing_read", "pe_pack_async",
    "pe_forward_graph_workspace_size", "pe_forward_graph_create", "pe_graph_launch", "pe_graph_destroy",
    "pe_noalloc_scratch_size", "pe_varlen_attn_fwd_noalloc", "pe_attn_bwd_workspace_size",
)

# status[1] codes of pe_pack_async
PACK_OK, PACK_BAD_LENGTH, PACK_OVER_CAPACITY = 0, 1, 2


class PeError(RuntimeError):
    def __init__(self, fn: str, status: int, total_tokens: int | None = None):
        self.status = status
        self.total_tokens = total_tokens
        super().__init__(f"{fn}: {_lib.pe_status_string(status).decode()}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m padding_free_packed_amd.build`"
                          " (or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "pe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "pe_attn_tile_rows": (I32, []),
        "pe_pack_workspace_size": (SZ, [I32, I32, I64, ctypes.c_int]),
        "pe_pack": (ctypes.c_int, [P, I32, I32, P, I64, ctypes.c_int, P, P, P, I64, P, P, SZ, P]),
        "pe_unpack": (ctypes.c_int, [P, P, I32, I32, I64, I64, ctypes.c_int, P, P]),
        "pe_worklist": (ctypes.c_int, [P, I32, I64, I32, P, P]),
        "pe_attn_workspace_size": (SZ, [I32, I64, I32, I32, ctypes.c_int, ctypes.c_int]),
        "pe_attn_bwd_workspace_size": (SZ, [I32, I64, I32, I32, I32, ctypes.c_int]),
        "pe_varlen_attn_fwd": (ctypes.c_int, [P, P, P, P, I32, I64, I32, I32, I32, ctypes.c_int, F, P, P, P,
                                               SZ, P]),
        "pe_varlen_attn_fwd_first_token": (ctypes.c_int, [P, P, P, P, I32, I64, I32, I32, I32, ctypes.c_int,
                                                           F, P, P, P]),
        "pe_varlen_attn_bwd": (ctypes.c_int, [P, P, P, P, P, P, P, I32, I64, I32, I32, I32, ctypes.c_int, F,
                                               P, P, P, P, SZ, P]),
        "pe_varlen_attn_fwd_local": (ctypes.c_int, [P, P, P, P, I32, I64, I32, I32, I32, ctypes.c_int, F, I32,
                                                     P, P, P, SZ, P]),
        "pe_varlen_attn_bwd_local": (ctypes.c_int, [P, P, P, P, P, P, P, I32, I64, I32, I32, I32, ctypes.c_int,
                                                     F, I32, P, P, P, P, SZ, P]),
        "pe_varlen_attn_fwd_first_row": (ctypes.c_int, [P, P, P, P, I32, I64, I32, I32, I32, ctypes.c_int, F,
                                                         P, P, P]),
        "pe_varlen_attn_bwd_first_token": (ctypes.c_int, [P, P, P, P, P, P, P, I32, I64, I32, I32, I32,
                                                           ctypes.c_int, F, P, P, P, P]),
        "pe_position_ids": (ctypes.c_int, [P, I32, I64, P, P, P]),
        "pe_flatten_workspace_size": (SZ, [I32]),
        "pe_flatten_packed_metadata": (ctypes.c_int, [P, P, I32, I32, I32, P, P, I64, I64, P, P, P, SZ, P]),
        "pe_flatten_document_mask": (ctypes.c_int, [P, I32, I32, P, P, I64, I64, P, P, P, SZ, P]),
        "pe_gather_rows": (ctypes.c_int, [P, I64, P, I64, I64, ctypes.c_int, P, P]),
        "pe_scatter_rows": (ctypes.c_int, [P, P, I64, I64, ctypes.c_int, P, I64, P]),
        "pe_varlen_attn_fwd_qkv": (ctypes.c_int, [P, P, I32, I64, I32, I32, I32, ctypes.c_int, F, I32, P, P, P,
                                                   SZ, P]),
        "pe_varlen_attn_bwd_qkv": (ctypes.c_int, [P, P, P, P, P, I32, I64, I32, I32, I32, ctypes.c_int, F, I32, P,
                                                   P, SZ, P]),
        "pe_pack_async": (ctypes.c_int, [P, I32, I32, P, I64, ctypes.c_int, P, P, P, I64, P, P, SZ, P]),
        "pe_forward_graph_workspace_size": (SZ, [I32, I32, I32, I32, ctypes.c_int]),
        "pe_forward_graph_create": (ctypes.c_int, [P, I32, I32, P, I32, I32, ctypes.c_int, F, I32, P, P, P, P, P,
                                                    P, P, SZ, ctypes.POINTER(ctypes.c_void_p)]),
        "pe_graph_launch": (ctypes.c_int, [P, P]),
        "pe_graph_destroy": (ctypes.c_int, [P]),
        "pe_noalloc_scratch_size": (SZ, []),
        "pe_varlen_attn_fwd_noalloc": (ctypes.c_int, [P, P, P, P, I32, I64, I32, I32, I32, ctypes.c_int, F, P, P,
                                                       P]),
        "pe_timing_enable": (ctypes.c_int, [ctypes.c_int]),
        "pe_timing_read": (ctypes.c_int, [P, P, ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library():
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PE_FP32
    if t.dtype == torch.bfloat16:
        return PE_BF16
    if t.dtype == torch.float16:
        return PE_FP16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(fn, status, total=None):
    if status != PE_OK:
        raise PeError(fn, status, total)


# ------------------------------------------------------------------ sizes

def pe_attn_tile_rows() -> int:
    return int(_lib.pe_attn_tile_rows())


def pe_pack_workspace_size(num_seqs: int, max_seq_len: int, row_elems: int, dtype: int) -> int:
    return int(_lib.pe_pack_workspace_size(num_seqs, max_seq_len, row_elems, dtype))


def pe_attn_workspace_size(num_seqs: int, total_tokens: int, num_heads: int, head_dim: int, dtype: int,
                           for_backward: bool) -> int:
    return int(_lib.pe_attn_workspace_size(num_seqs, total_tokens, num_heads, head_dim, dtype,
                                           int(for_backward)))


def pe_attn_bwd_workspace_size(num_seqs: int, total_tokens: int, max_seq_len: int, num_heads: int, head_dim: int,
                               dtype: int) -> int:
    return int(_lib.pe_attn_bwd_workspace_size(num_seqs, total_tokens, max_seq_len, num_heads, head_dim, dtype))


# ------------------------------------------------------------------ calls

def pe_pack(lengths, max_seq_len, grid, cu_seqlens, flat_index, packed, capacity, workspace,
            dtype: int | None = None) -> int:
    """Returns the token count N. Raises PeError (``.total_tokens`` set) on failure."""
    if dtype is None:
        dtype = _dtype_code(grid) if grid is not None else PE_FP32
    row_elems = 0 if grid is None else grid.numel() // (lengths.numel() * max_seq_len)
    n = ctypes.c_int64(0)
    st = _lib.pe_pack(_ptr(lengths), lengths.numel(), max_seq_len, _ptr(grid), row_elems, dtype,
                      _ptr(cu_seqlens), _ptr(flat_index), _ptr(packed), capacity, ctypes.byref(n),
                      _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream())
    _check("pe_pack", st, n.value)
    return n.value


def pe_pack_async(lengths, max_seq_len, grid, cu_seqlens, flat_index, packed, capacity, status, workspace,
                  dtype: int | None = None) -> None:
    """pe_pack with no host read: the token count and an error code land in the
    device int64 tensor ``status`` ([N, code], code one of PACK_*)."""
    if dtype is None:
        dtype = _dtype_code(grid) if grid is not None else PE_FP32
    row_elems = 0 if grid is None else grid.numel() // (lengths.numel() * max_seq_len)
    st = _lib.pe_pack_async(_ptr(lengths), lengths.numel(), max_seq_len, _ptr(grid), row_elems, dtype,
                            _ptr(cu_seqlens), _ptr(flat_index), _ptr(packed), capacity, _ptr(status),
                            _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream())
    _check("pe_pack_async", st)


def pe_unpack(packed, cu_seqlens, num_seqs, max_seq_len, total_tokens, grid):
    row_elems = packed.numel() // max(total_tokens, 1)
    st = _lib.pe_unpack(_ptr(packed), _ptr(cu_seqlens), num_seqs, max_seq_len, total_tokens, row_elems,
                        _dtype_code(packed), _ptr(grid), _stream())
    _check("pe_unpack", st)


def pe_worklist(cu_seqlens, num_seqs, total_tokens, tile_rows, items):
    _check("pe_worklist", _lib.pe_worklist(_ptr(cu_seqlens), num_seqs, total_tokens, tile_rows,
                                           _ptr(items), _stream()))


def pe_varlen_attn_fwd(q, k, v, cu_seqlens, num_seqs, total_tokens, max_seq_len, softmax_scale, out,
                       lse, workspace):
    N, H, d = q.shape
    st = _lib.pe_varlen_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), num_seqs, total_tokens,
                                 max_seq_len, H, d, _dtype_code(q), softmax_scale, _ptr(out), _ptr(lse),
                                 _ptr(workspace), workspace.numel(), _stream())
    _check("pe_varlen_attn_fwd", st)


def pe_noalloc_scratch_size() -> int:
    return int(_lib.pe_noalloc_scratch_size())


def pe_varlen_attn_fwd_noalloc(q, k, v, cu_seqlens, num_seqs, total_tokens, max_seq_len, softmax_scale, out, lse):
    N, H, d = q.shape
    st = _lib.pe_varlen_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), num_seqs, total_tokens,
                                         max_seq_len, H, d, _dtype_code(q), softmax_scale, _ptr(out), _ptr(lse),
                                         _stream())
    _check("pe_varlen_attn_fwd_noalloc", st)


def pe_varlen_attn_fwd_first_token(q_first, k, v, cu_seqlens, num_seqs, total_tokens, max_seq_len,
                                   softmax_scale, out_first, lse_first):
    B, H, d = q_first.shape
    st = _lib.pe_varlen_attn_fwd_first_token(_ptr(q_first), _ptr(k), _ptr(v), _ptr(cu_seqlens), num_seqs,
                                             total_tokens, max_seq_len, H, d, _dtype_code(q_first),
                                             softmax_scale, _ptr(out_first), _ptr(lse_first), _stream())
    _check("pe_varlen_attn_fwd_first_token", st)


def pe_varlen_attn_fwd_first_row(q, k, v, cu_seqlens, num_seqs, total_tokens, max_seq_len, softmax_scale,
                                 out_first, lse_first):
    N, H, d = q.shape
    st = _lib.pe_varlen_attn_fwd_first_row(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), num_seqs, total_tokens,
                                           max_seq_len, H, d, _dtype_code(q), softmax_scale, _ptr(out_first),
                                           _ptr(lse_first), _stream())
    _check("pe_varlen_attn_fwd_first_row", st)


def pe_varlen_attn_bwd_first_token(dout_first, q_first, k, v, out_first, lse_first, cu_seqlens, num_seqs,
                                   total_tokens, max_seq_len, softmax_scale, dq_first, dk, dv):
    B, H, d = q_first.shape
    st = _lib.pe_varlen_attn_bwd_first_token(_ptr(dout_first), _ptr(q_first), _ptr(k), _ptr(v), _ptr(out_first),
                                             _ptr(lse_first), _ptr(cu_seqlens), num_seqs, total_tokens,
                                             max_seq_len, H, d, _dtype_code(q_first), softmax_scale,
                                             _ptr(dq_first), _ptr(dk), _ptr(dv), _stream())
    _check("pe_varlen_attn_bwd_first_token", st)


def pe_varlen_attn_bwd(dout, q, k, v, out, lse, cu_seqlens, num_seqs, total_tokens, max_seq_len,
                       softmax_scale, dq, dk, dv, workspace):
    N, H, d = q.shape
    st = _lib.pe_varlen_attn_bwd(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                 _ptr(cu_seqlens), num_seqs, total_tokens, max_seq_len, H, d,
                                 _dtype_code(q), softmax_scale, _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(workspace), workspace.numel(), _stream())
    _check("pe_varlen_attn_bwd", st)


def pe_varlen_attn_fwd_local(q, k, v, cu_seqlens, num_seqs, total_tokens, max_seq_len, softmax_scale, window,
                             out, lse, workspace):
    N, H, d = q.shape
    st = _lib.pe_varlen_attn_fwd_local(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), num_seqs, total_tokens,
                                       max_seq_len, H, d, _dtype_code(q), softmax_scale, window, _ptr(out),
                                       _ptr(lse), _ptr(workspace), workspace.numel(), _stream())
    _check("pe_varlen_attn_fwd_local", st)


def pe_varlen_attn_bwd_local(dout, q, k, v, out, lse, cu_seqlens, num_seqs, total_tokens, max_seq_len,
                             softmax_scale, window, dq, dk, dv, workspace):
    N, H, d = q.shape
    st = _lib.pe_varlen_attn_bwd_local(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                       _ptr(cu_seqlens), num_seqs, total_tokens, max_seq_len, H, d,
                                       _dtype_code(q), softmax_scale, window, _ptr(dq), _ptr(dk), _ptr(dv),
                                       _ptr(workspace), workspace.numel(), _stream())
    _check("pe_varlen_attn_bwd_local", st)


def pe_varlen_attn_fwd_qkv(qkv, cu_seqlens, num_seqs, total_tokens, max_seq_len, softmax_scale, window, out, lse,
                           workspace):
    """qkv [N, 3, H, d] (fused projection rows); window -1 for global attention."""
    N, three, H, d = qkv.shape
    assert three == 3 and qkv.is_contiguous()
    st = _lib.pe_varlen_attn_fwd_qkv(_ptr(qkv), _ptr(cu_seqlens), num_seqs, total_tokens, max_seq_len, H, d,
                                     _dtype_code(qkv), softmax_scale, window, _ptr(out), _ptr(lse), _ptr(workspace),
                                     workspace.numel(), _stream())
    _check("pe_varlen_attn_fwd_qkv", st)


def pe_varlen_attn_bwd_qkv(dout, qkv, out, lse, cu_seqlens, num_seqs, total_tokens, max_seq_len, softmax_scale,
                           window, dqkv, workspace):
    N, three, H, d = qkv.shape
    assert three == 3 and qkv.is_contiguous() and dqkv.is_contiguous()
    st = _lib.pe_varlen_attn_bwd_qkv(_ptr(dout), _ptr(qkv), _ptr(out), _ptr(lse), _ptr(cu_seqlens), num_seqs,
                                     total_tokens, max_seq_len, H, d, _dtype_code(qkv), softmax_scale, window,
                                     _ptr(dqkv), _ptr(workspace), workspace.numel(), _stream())
    _check("pe_varlen_attn_bwd_qkv", st)


# ------------------------------------------------------------------ captured bucket forward

def pe_forward_graph_workspace_size(num_seqs: int, max_seq_len: int, num_heads: int, head_dim: int,
                                    dtype: int) -> int:
    return int(_lib.pe_forward_graph_workspace_size(num_seqs, max_seq_len, num_heads, head_dim, dtype))


def pe_forward_graph_create(lengths, qkv_grid, softmax_scale, window, cu_seqlens, qkv_packed, out_packed, lse,
                            out_grid, status, workspace):
    """qkv_grid [B, S, 3, H, d]; returns an opaque graph handle (int) for pe_graph_launch."""
    B, S, three, H, d = qkv_grid.shape
    assert three == 3 and qkv_grid.is_contiguous() and lengths.numel() == B
    handle = ctypes.c_void_p(None)
    st = _lib.pe_forward_graph_create(_ptr(lengths), B, S, _ptr(qkv_grid), H, d, _dtype_code(qkv_grid),
                                      softmax_scale, window, _ptr(cu_seqlens), _ptr(qkv_packed), _ptr(out_packed),
                                      _ptr(lse), _ptr(out_grid), _ptr(status), _ptr(workspace), workspace.numel(),
                                      ctypes.byref(handle))
    _check("pe_forward_graph_create", st)
    return handle.value


def pe_graph_launch(graph) -> None:
    _check("pe_graph_launch", _lib.pe_graph_launch(ctypes.c_void_p(graph), _stream()))


def pe_graph_destroy(graph) -> None:
    _check("pe_graph_destroy", _lib.pe_graph_destroy(ctypes.c_void_p(graph)))


# ------------------------------------------------------------------ packing metadata

def pe_position_ids(cu_seqlens, num_seqs, total_tokens, position_ids, document_ids):
    _check("pe_position_ids", _lib.pe_position_ids(_ptr(cu_seqlens), num_seqs, total_tokens, _ptr(position_ids),
                                                   _ptr(document_ids), _stream()))


def pe_flatten_workspace_size(rows: int) -> int:
    return int(_lib.pe_flatten_workspace_size(rows))


def _flatten_result(fn, status, tok, docs):
    if status != PE_OK:
        raise PeError(fn, status, tok.value)
    return tok.value, docs.value


def pe_flatten_packed_metadata(token_index, cu_local, flat_index, cu_seqlens, workspace):
    """token_index int32 [rows, width], cu_local int32 [rows, max_docs + 1] (device);
    fills flat_index (int64, its length is the capacity) and cu_seqlens (int32); returns
    (tokens, documents). PeError carries the status (capacity: token count in total_tokens)."""
    rows, width = token_index.shape
    tok, docs = ctypes.c_int64(0), ctypes.c_int64(0)
    st = _lib.pe_flatten_packed_metadata(_ptr(token_index), _ptr(cu_local), rows, width, cu_local.shape[1] - 1,
                                         _ptr(flat_index), _ptr(cu_seqlens),
                                         0 if flat_index is None else flat_index.numel(), cu_seqlens.numel() - 1,
                                         ctypes.byref(tok), ctypes.byref(docs), _ptr(workspace), workspace.numel(),
                                         _stream())
    return _flatten_result("pe_flatten_packed_metadata", st, tok, docs)


def pe_flatten_document_mask(document_mask, flat_index, cu_seqlens, workspace):
    rows, width = document_mask.shape
    tok, docs = ctypes.c_int64(0), ctypes.c_int64(0)
    st = _lib.pe_flatten_document_mask(_ptr(document_mask), rows, width, _ptr(flat_index), _ptr(cu_seqlens),
                                       0 if flat_index is None else flat_index.numel(), cu_seqlens.numel() - 1,
                                       ctypes.byref(tok), ctypes.byref(docs), _ptr(workspace), workspace.numel(),
                                       _stream())
    return _flatten_result("pe_flatten_document_mask", st, tok, docs)


def pe_gather_rows(src, flat_index, dst):
    """dst[r] = src[flat_index[r]]; src [rows, ...], dst [n, ...] of the same dtype."""
    row_elems = src[0].numel() if src.shape[0] > 0 else int(torch.tensor(src.shape[1:]).prod())
    _check("pe_gather_rows", _lib.pe_gather_rows(_ptr(src), src.shape[0], _ptr(flat_index), flat_index.numel(),
                                                 row_elems, _dtype_code(src), _ptr(dst), _stream()))


def pe_scatter_rows(src, flat_index, dst):
    """dst[flat_index[r]] = src[r], every other row of dst zero."""
    row_elems = dst[0].numel() if dst.shape[0] > 0 else int(torch.tensor(dst.shape[1:]).prod())
    _check("pe_scatter_rows", _lib.pe_scatter_rows(_ptr(src), _ptr(flat_index), flat_index.numel(), row_elems,
                                                   _dtype_code(src), _ptr(dst), dst.shape[0], _stream()))


# ------------------------------------------------------------------ kernel timing

def pe_timing_enable(on: bool) -> None:
    _check("pe_timing_enable", _lib.pe_timing_enable(int(bool(on))))


def pe_timing_read(max_records: int = 4096):
    """[(kernel name, milliseconds)] of the kernels launched since the last read."""
    names = ctypes.create_string_buffer(32 * max_records)
    ms = (ctypes.c_float * max_records)()
    n = _lib.pe_timing_read(ctypes.cast(names, ctypes.c_void_p), ctypes.cast(ms, ctypes.c_void_p), max_records)
    raw = names.raw
    return [(raw[32 * i:32 * i + 32].split(b"\0", 1)[0].decode(), float(ms[i])) for i in range(n)]


# ------------------------------------------------------------------ allocating helpers

def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def pack(lengths, max_seq_len, grid=None, capacity=None):
    """Layout (and packed rows) from device lengths; allocates outputs.

    With ``capacity`` unknown, a first call computes the layout only; its token
    count sizes the outputs of the second call.
    """
    dev = lengths.device
    B = lengths.numel()
    row_elems = 0 if grid is None else grid.numel() // (B * max_seq_len)
    dt = _dtype_code(grid) if grid is not None else PE_FP32
    ws = workspace(pe_pack_workspace_size(B, max_seq_len, max(row_elems, 1), dt), dev)
    cu = torch.empty(B + 1, dtype=torch.int32, device=dev)
    if capacity is None:
        capacity = pe_pack(lengths, max_seq_len, None, cu, None, None, 0, ws, dt)
    flat = torch.empty(capacity, dtype=torch.int64, device=dev)
    packed = None if grid is None else torch.empty(capacity, row_elems, dtype=grid.dtype, device=dev)
    n = pe_pack(lengths, max_seq_len, grid, cu, flat, packed, capacity, ws, dt)
    return cu, flat[:n], (None if packed is None else packed[:n]), n
