"""Plain fp64 CPU oracle for packed, padding-free attention.

TEST INFRASTRUCTURE ONLY. Nothing in the library calls this module. Only the
tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it. It shares no code with the HIP path: it imports
numpy and nothing from the ``padding_free_packed_amd`` package, and the HIP path
imports nothing from here.

What it computes (sources are the GiGL page "Source code for
gigl.nn.packed_attention" and the packed-encoders README):

* ``layout``: the lengths-to-offsets prefix sum and the flat row index of every
  real token in the padded grid (GiGL module docstring, "Example" and the data
  flow diagram; packed-encoders "Fully packed execution (advanced)").
* ``pack`` / ``unpack``: the row gather ``grid.flatten()[flat_index]`` read as
  "flatten the (sequence, position) dimensions and gather rows", and its
  inverse, which writes zeros outside real rows (GiGL data flow diagram;
  ``_padded_packed_attention``, which scatters into ``zeros_like``).
* ``attention``: non-causal softmax attention in which every sequence attends
  only to itself, with the log-sum-exp of the scaled logits (GiGL module
  docstring; ``_varlen_attention`` docstring, "Query sequence i attends to key
  sequence i"). The result has a plain definition, so this is that definition
  written out per sequence and per head, with a matmul as a step.
* ``attention_first_token``: one query per sequence, the sequence's first token
  (GiGL ``packed_attention``, ``query_is_first_token``), and its backward
  ``attention_first_token_backward``: GiGL runs the readout through the same
  autograd-registered varlen op, with one query per sequence
  (``cu_seqlens_q = arange(B + 1)``), so it trains through it.
* ``attention_backward``: gradients of the same definition in Q, K and V, with no
  gradient flowing into the log-sum-exp (GiGL ``_varlen_attention_backward``
  drops the log-sum-exp's gradient). The pages give no formulas; these are the
  derivatives of softmax attention, written out from its definition. As GiGL's
  backward op does, it can take the forward's output and log-sum-exp as inputs
  (its D term is formed from the output it is given).
* ``padded_attention``: an independent second route, the padded grid with an
  additive ``finfo.min / 2`` key bias and a dense softmax over all positions,
  as ``_padded_packed_attention`` does.
* ``worklist``: for a tile height R, the sequence holding the first row of every
  R-row tile of the packed buffer (the library's work list; brute force).
* packing metadata (``position_ids``, ``document_ids``, ``flatten_packed_metadata``,
  ``flatten_document_mask``, ``gather_rows``, ``scatter_rows``): the metadata of
  the packed-encoders README's direct packed entry (position ids) and of NeMo's
  packing (indexed document masks, ``flatten_packed_sequence_metadata``), written
  out from their documented meaning with plain loops.
* local attention: every attention function takes an optional ``window`` w;
  query i then sees only the keys j of its own sequence with |i - j| <= w. This
  is the sliding-window ("local") non-causal attention that the packed-encoders
  README lists next to global attention for its short-sequence kernel and that
  its FlashAttention backend prunes; the README names a "local-64" variant
  without fixing how 64 maps to a radius, so w is a parameter here.

Every input array is float64 (attention) or raw bits (pack/unpack); callers widen
fp32 values and bf16 bit patterns exactly before calling.
"""
from __future__ import annotations

import numpy as np

INT32_MAX = 2**31 - 1


# ---------------------------------------------------------------- layout, pack, unpack

def layout(lengths, max_seq_len: int):
    """Offsets and flat row index of a packed batch.

    GiGL "Example": lengths [3, 1, 2] with max_seq_len 3 give flat_index
    [0, 1, 2, 3, 6, 7]; offsets are the exclusive running sum of the lengths.
    Every length lies in [1, max_seq_len] (``packed_attention`` docstring: an
    empty sequence is unsupported; the grid has max_seq_len positions) and the
    total fits int32 (module docstring, "Constraints").

    Returns ``(cu_seqlens int32 [B+1], flat_index int64 [N], N)``.
    """
    lengths = [int(x) for x in np.asarray(lengths).reshape(-1)]
    S = int(max_seq_len)
    for L in lengths:
        if L < 1 or L > S:
            raise ValueError(f"length {L} outside [1, {S}]")
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    N = cu[-1]
    if N > INT32_MAX:
        raise ValueError("total token count does not fit int32")
    flat = []
    for b, L in enumerate(lengths):
        for t in range(L):
            flat.append(b * S + t)
    return np.array(cu, dtype=np.int32), np.array(flat, dtype=np.int64), N


def pack(grid: np.ndarray, flat_index: np.ndarray) -> np.ndarray:
    """Gather the real rows of a padded grid ``[B, S, D]`` into ``[N, D]``.

    GiGL data flow: ``grid.flatten()[flat_index]`` yields ``[num_tokens, dim]``,
    so the (sequence, position) dimensions are flattened and whole rows of D
    values are gathered. The copy moves bits (the grid is viewed as unsigned
    integers of its element width) so NaN payloads survive unchanged.
    """
    B, S, D = grid.shape
    bits = _as_bits(grid).reshape(B * S, D)
    out = np.empty((len(flat_index), D), dtype=bits.dtype)
    for r, g in enumerate(flat_index):
        out[r, :] = bits[g, :]
    return out.view(grid.dtype)


def unpack(packed: np.ndarray, cu_seqlens: np.ndarray, max_seq_len: int) -> np.ndarray:
    """Scatter packed rows ``[N, D]`` back to a padded grid ``[B, S, D]``; padding is +0.0.

    Inverse of ``pack`` on real rows. The fill value is not stated on the pages;
    the first-token reference path scatters into ``zeros_like``, so every
    position past a sequence's length holds +0.0 (all-zero bits in fp32 and
    bf16).
    """
    cu = [int(x) for x in cu_seqlens]
    B = len(cu) - 1
    S = int(max_seq_len)
    N, D = packed.shape
    src = _as_bits(packed)
    out = np.zeros((B, S, D), dtype=src.dtype)
    for b in range(B):
        for t in range(cu[b + 1] - cu[b]):
            out[b, t, :] = src[cu[b] + t, :]
    return out.view(packed.dtype)


def _as_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    return x.view({2: np.uint16, 4: np.uint32, 8: np.uint64}[x.dtype.itemsize])


# ---------------------------------------------------------------- attention

def _check_f64(*arrays):
    for a in arrays:
        if a.dtype != np.float64:
            raise TypeError("oracle attention takes float64 arrays")


def _segments(cu_seqlens):
    cu = [int(x) for x in cu_seqlens]
    return [(cu[b], cu[b + 1]) for b in range(len(cu) - 1)]


def _band(rows, cols, window):
    """Allowed (query, key) pairs for packed row indices ``rows`` x ``cols`` of one
    sequence: all of them (global attention) or |i - j| <= window (local)."""
    if window is None:
        return None
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    return np.abs(i - j) <= int(window)


def _restrict(s, allowed):
    return s if allowed is None else np.where(allowed, s, -np.inf)


def attention(q, k, v, cu_seqlens, scale: float, window=None):
    """Non-causal attention confined to each sequence, plus its log-sum-exp.

    For sequence b (rows c0..c1-1) and head h, for every query row i:
    s_j = scale * <q_i, k_j> over the keys j of the same sequence only,
    m = max_j s_j, w_j = exp(s_j - m), l = sum_j w_j,
    o_i = sum_j w_j v_j / l and lse_i = m + ln l (natural log of the scaled
    logits). This is softmax(scale * Q K^T) V per sequence, the result of the
    varlen kernel and of the padded SDPA path on the GiGL page.

    With ``window`` w (local attention) the keys are further limited to
    |i - j| <= w.

    q, k, v: float64 [N, H, d]. Returns o float64 [N, H, d], lse float64 [H, N].
    """
    _check_f64(q, k, v)
    N, H, d = q.shape
    o = np.zeros((N, H, d))
    lse = np.zeros((H, N))
    for c0, c1 in _segments(cu_seqlens):
        allowed = _band(range(c0, c1), range(c0, c1), window)
        for h in range(H):
            s = _restrict(scale * (q[c0:c1, h, :] @ k[c0:c1, h, :].T), allowed)
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            l = w.sum(axis=1, keepdims=True)
            o[c0:c1, h, :] = (w @ v[c0:c1, h, :]) / l
            lse[h, c0:c1] = (m + np.log(l))[:, 0]
    return o, lse


def sequence_of_rows(cu_seqlens, rows):
    """Index of the sequence holding each packed row (linear scan, plain definition)."""
    cu = [int(x) for x in cu_seqlens]
    out = []
    for r in rows:
        r = int(r)
        b = 0
        while not (cu[b] <= r < cu[b + 1]):
            b += 1
        out.append(b)
    return out


def attention_rows(q, k, v, cu_seqlens, scale: float, rows, window=None):
    """``attention`` evaluated only at the given packed query rows (all heads).

    Used to check very large batches at sampled outputs: each sampled row needs
    only its own sequence's keys. Returns o float64 [len(rows), H, d] and
    lse float64 [H, len(rows)].
    """
    _check_f64(q, k, v)
    N, H, d = q.shape
    rows = list(rows)
    seqs = sequence_of_rows(cu_seqlens, rows)
    cu = [int(x) for x in cu_seqlens]
    o = np.zeros((len(rows), H, d))
    lse = np.zeros((H, len(rows)))
    for n, (r, b) in enumerate(zip(rows, seqs)):
        c0, c1 = cu[b], cu[b + 1]
        allowed = _band([r], range(c0, c1), window)
        allowed = None if allowed is None else allowed[0]
        for h in range(H):
            s = _restrict(scale * (k[c0:c1, h, :] @ q[r, h, :]), allowed)
            m = s.max()
            w = np.exp(s - m)
            l = w.sum()
            o[n, h, :] = (w @ v[c0:c1, h, :]) / l
            lse[h, n] = m + np.log(l)
    return o, lse


def attention_first_token(q_first, k, v, cu_seqlens, scale: float, seqs=None, window=None):
    """One query per sequence (its first token) attending over that sequence's keys.

    GiGL ``packed_attention`` with ``query_is_first_token``: ``query`` holds one
    row per sequence, the caller passes ``query[cu_seqlens[:-1]]``; the result is
    the full attention output at rows cu_seqlens[:-1].

    q_first float64 [B, H, d]; k, v float64 [N, H, d]. ``seqs`` optionally limits
    the computation to some sequences. Returns o float64 [B', H, d] and
    lse float64 [H, B'].
    """
    _check_f64(q_first, k, v)
    B, H, d = q_first.shape
    segs = _segments(cu_seqlens)
    seqs = list(range(B)) if seqs is None else list(seqs)
    o = np.zeros((len(seqs), H, d))
    lse = np.zeros((H, len(seqs)))
    for n, b in enumerate(seqs):
        c0, c1 = segs[b]
        allowed = _band([c0], range(c0, c1), window)
        allowed = None if allowed is None else allowed[0]
        for h in range(H):
            s = _restrict(scale * (k[c0:c1, h, :] @ q_first[b, h, :]), allowed)
            m = s.max()
            w = np.exp(s - m)
            l = w.sum()
            o[n, h, :] = (w @ v[c0:c1, h, :]) / l
            lse[h, n] = m + np.log(l)
    return o, lse


def attention_first_token_backward(dout_first, q_first, k, v, cu_seqlens, scale: float, out_first=None,
                                   lse_first=None):
    """Gradients of ``<dout_first, attention_first_token(q_first, k, v)>`` in q_first, k and v.

    The first-token readout is the full attention evaluated at rows cu[:-1] only,
    so its backward is the full backward with every other row's output gradient
    zero. Per sequence b and head h, with s_j = scale <q_b, k_j> over the keys j
    of sequence b, P_j = exp(s_j - lse_b), D_b = <dO_b, O_b>:
    dv_j = P_j dO_b; dS_j = P_j (<dO_b, v_j> - D_b); dq_b = scale sum_j dS_j k_j;
    dk_j = scale dS_j q_b. No gradient enters through the log-sum-exp.

    ``out_first`` [B, H, d] and ``lse_first`` [H, B] play the role of the forward's
    output and log-sum-exp (this module's own float64 forward when omitted).
    Returns dq_first float64 [B, H, d], dk and dv float64 [N, H, d].
    """
    _check_f64(dout_first, q_first, k, v)
    B, H, d = q_first.shape
    N = k.shape[0]
    dq = np.zeros((B, H, d))
    dk = np.zeros((N, H, d))
    dv = np.zeros((N, H, d))
    if out_first is None or lse_first is None:
        o_own, l_own = attention_first_token(q_first, k, v, cu_seqlens, scale)
        out_first = o_own if out_first is None else out_first
        lse_first = l_own if lse_first is None else lse_first
    out_first = np.asarray(out_first, dtype=np.float64)
    lse_first = np.asarray(lse_first, dtype=np.float64)
    for b, (c0, c1) in enumerate(_segments(cu_seqlens)):
        for h in range(H):
            qb, dob = q_first[b, h, :], dout_first[b, h, :]
            s = scale * (k[c0:c1, h, :] @ qb)
            p = np.exp(s - lse_first[h, b])
            dv[c0:c1, h, :] = np.outer(p, dob)
            ds = p * (v[c0:c1, h, :] @ dob - float(dob @ out_first[b, h, :]))
            dq[b, h, :] = scale * (ds @ k[c0:c1, h, :])
            dk[c0:c1, h, :] = scale * np.outer(ds, qb)
    return dq, dk, dv


def attention_backward(dout, q, k, v, cu_seqlens, scale: float, seqs=None, out=None, lse=None, window=None):
    """Gradients of ``<dout, attention(q, k, v)>`` in q, k and v.

    Per sequence and head, with P = softmax(scale * Q K^T) (rows) and O = P V:
    dV = P^T dO; dP = dO V^T; D_i = sum_c dO_ic O_ic; dS = P * (dP - D);
    dQ = scale * dS K; dK = scale * dS^T Q. No gradient enters through the
    log-sum-exp, as in GiGL's ``_varlen_attention_backward``.

    GiGL's backward op receives the forward's ``output`` and ``logsumexp`` as
    inputs; ``out`` [N, H, d] and ``lse`` [H, N] play those roles here: when
    given, D is formed from ``out`` and P = exp(s - lse) from ``lse``. When
    omitted they are this module's own float64 forward, and the result is the
    exact gradient.

    ``seqs`` optionally limits the computation to some sequences (rows of other
    sequences are left zero). With ``window`` the pairs outside |i - j| <= w
    have P = 0. Returns dq, dk, dv float64 [N, H, d].
    """
    _check_f64(dout, q, k, v)
    N, H, d = q.shape
    dq = np.zeros((N, H, d))
    dk = np.zeros((N, H, d))
    dv = np.zeros((N, H, d))
    segs = _segments(cu_seqlens)
    seqs = range(len(segs)) if seqs is None else seqs
    for b in seqs:
        c0, c1 = segs[b]
        allowed = _band(range(c0, c1), range(c0, c1), window)
        for h in range(H):
            qs, ks, vs, dos = q[c0:c1, h, :], k[c0:c1, h, :], v[c0:c1, h, :], dout[c0:c1, h, :]
            s = _restrict(scale * (qs @ ks.T), allowed)
            if lse is None:
                m = s.max(axis=1, keepdims=True)
                lse_b = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
            else:
                lse_b = np.asarray(lse, dtype=np.float64)[h, c0:c1][:, None]
            p = np.exp(s - lse_b)
            o = p @ vs if out is None else np.asarray(out, dtype=np.float64)[c0:c1, h, :]
            dv[c0:c1, h, :] = p.T @ dos
            dp = dos @ vs.T
            D = (dos * o).sum(axis=1, keepdims=True)
            ds = p * (dp - D)
            dq[c0:c1, h, :] = scale * (ds @ ks)
            dk[c0:c1, h, :] = scale * (ds.T @ qs)
    return dq, dk, dv


# ---------------------------------------------------------------- second route: padded grid

def padded_attention(q, k, v, cu_seqlens, max_seq_len: int, scale: float,
                     query_is_first_token: bool = False, window=None):
    """Attention by padding, following GiGL's ``_padded_packed_attention``.

    Tokens are placed on a ``[B, S]`` grid; padded key positions get the additive
    bias ``finfo(float64).min / 2``; a dense softmax runs over all S positions for
    every grid row; padded rows are dropped. With ``query_is_first_token`` the B
    queries are placed in the first row of their sequence (all other query rows
    zero) and only those rows are returned.

    This route shares no loop with ``attention``: it never slices a sequence's
    key range, it relies on the bias alone to exclude other positions.
    Returns o float64 [num_queries, H, d] and lse float64 [H, num_queries].
    """
    _check_f64(q, k, v)
    N, H, d = k.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = cu.shape[0] - 1
    S = int(max_seq_len)
    lengths = cu[1:] - cu[:-1]
    seq_of_token = np.repeat(np.arange(B), lengths)
    pos_of_token = np.arange(N) - cu[:-1][seq_of_token]
    if query_is_first_token:
        qfull = np.zeros_like(k)
        qfull[cu[:-1]] = q
        q = qfull
    mask = np.zeros((B, S), dtype=bool)
    mask[seq_of_token, pos_of_token] = True
    grids = []
    for x in (q, k, v):
        g = np.zeros((B, S, H, d))
        g[seq_of_token, pos_of_token] = x
        grids.append(g.transpose(0, 2, 1, 3))  # [B, H, S, d]
    qg, kg, vg = grids
    keep = np.broadcast_to(mask[:, None, None, :], (B, 1, S, S))
    if window is not None:  # grid positions stand for packed rows at the same offsets
        pos = np.arange(S)
        keep = keep & (np.abs(pos[:, None] - pos[None, :]) <= int(window))[None, None]
    bias = np.where(keep, 0.0, np.finfo(np.float64).min / 2.0)
    s = scale * np.einsum("bhid,bhjd->bhij", qg, kg) + bias
    m = s.max(axis=-1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=-1, keepdims=True)
    og = np.einsum("bhij,bhjd->bhid", w / l, vg)
    lg = (m + np.log(l))[..., 0]                        # [B, H, S]
    o = og.transpose(0, 2, 1, 3)[mask]                  # [N, H, d]
    lse = lg.transpose(0, 2, 1)[mask].T                 # [H, N]
    if query_is_first_token:
        return o[cu[:-1]], lse[:, cu[:-1]]
    return o, lse


# ---------------------------------------------------------------- work list

def worklist(cu_seqlens, tile_rows: int):
    """Sequence index holding the first row of every ``tile_rows``-row tile.

    Tile t covers packed rows [t*R, min((t+1)*R, N)); entry t is the b with
    cu[b] <= t*R < cu[b+1]. One extra entry, equal to B, closes the list.
    Brute force over rows.
    """
    cu = [int(x) for x in cu_seqlens]
    N = cu[-1]
    B = len(cu) - 1
    T = (N + tile_rows - 1) // tile_rows
    out = sequence_of_rows(cu, [t * tile_rows for t in range(T)])
    return np.array(out + [B], dtype=np.int32)


# ---------------------------------------------------------------- packing metadata

def position_ids(cu_seqlens):
    """Position of every packed token inside its own sequence, int64 [N].

    The packed-encoders README builds them for its direct packed entry as the
    concatenation of arange(L_b) over the sequences.
    """
    cu = [int(x) for x in cu_seqlens]
    return np.concatenate([np.arange(cu[b + 1] - cu[b], dtype=np.int64) for b in range(len(cu) - 1)])


def document_ids(cu_seqlens):
    """1-based index of the sequence (document) holding every packed token, int32 [N].

    NeMo's indexed packing mask marks document i (1-based) with the integer i and
    padding with 0; for a packed stream without padding this is that mask.
    """
    cu = [int(x) for x in cu_seqlens]
    return np.concatenate([np.full(cu[b + 1] - cu[b], b + 1, dtype=np.int32) for b in range(len(cu) - 1)])


class MetadataError(ValueError):
    """Inconsistent packed metadata (NeMo raises ValueError for these)."""


def _valid_prefix(row, width_limit=None):
    """Length of the prefix of non-negative entries of a -1-padded row; checks that
    only -1 follows it and that the prefix is strictly increasing."""
    row = [int(x) for x in row]
    n = 0
    while n < len(row) and row[n] >= 0:
        n += 1
    if any(x != -1 for x in row[n:]):
        raise MetadataError("padding other than -1, or -1 before a valid entry")
    if any(row[i + 1] <= row[i] for i in range(n - 1)):
        raise MetadataError("entries not strictly increasing")
    if width_limit is not None and n > 0 and row[n - 1] >= width_limit:
        raise MetadataError("token index outside the row")
    return n


def flatten_packed_metadata(token_index, cu_local, width: int):
    """NeMo ``flatten_packed_sequence_metadata`` for the batch-major form.

    token_index int [rows, width']: row-local indices of the real tokens of each
    row, -1 padded. cu_local int [rows, max_docs + 1]: row-local cumulative
    document lengths, -1 padded (a row without documents is all -1 or 0 then -1).
    Returns the flat token indices int64 [tokens] into the padded [rows, width]
    grid (row-major, rows in order) and the global cumulative lengths int32
    [documents + 1] of the same stream. Raises MetadataError when a row's
    boundaries are not 0 then strictly increasing, when its last boundary differs
    from its number of tokens, or when indices are out of order or outside the row.
    """
    token_index = np.asarray(token_index)
    cu_local = np.asarray(cu_local)
    rows = token_index.shape[0]
    if cu_local.shape[0] != rows:
        raise MetadataError("token_index and cu_seqlens disagree on the number of rows")
    flat, cu = [], [0]
    base = 0
    for r in range(rows):
        n = _valid_prefix(token_index[r], width)
        m = _valid_prefix(cu_local[r])
        if m == 0:
            docs_end = 0
        else:
            if int(cu_local[r, 0]) != 0:
                raise MetadataError("a row's cumulative lengths do not start at 0")
            docs_end = int(cu_local[r, m - 1])
        if docs_end != n:
            raise MetadataError("a row's cumulative lengths do not add up to its tokens")
        flat.extend(r * width + int(token_index[r, j]) for j in range(n))
        cu.extend(base + int(cu_local[r, i]) for i in range(1, m))
        base += n
    return np.asarray(flat, dtype=np.int64), np.asarray(cu, dtype=np.int32)


def flatten_document_mask(mask):
    """Flatten a NeMo indexed packing mask int [rows, width] (document i of a row,
    1-based, marked i; padding 0, at the end of the row) to flat token indices
    int64 [tokens] and global cumulative lengths int32 [documents + 1]. A document
    is a maximal run of equal ids. Raises MetadataError unless every row is
    1, then ids equal to or one above their predecessor, then only zeros.
    """
    mask = np.asarray(mask)
    rows, width = mask.shape
    flat, cu = [], [0]
    for r in range(rows):
        row = [int(x) for x in mask[r]]
        n = 0
        while n < width and row[n] > 0:
            n += 1
        if any(x != 0 for x in row[n:]):
            raise MetadataError("padding other than 0, or 0 before a document")
        for t in range(n):
            prev = 0 if t == 0 else row[t - 1]
            if row[t] != prev and row[t] != prev + 1:
                raise MetadataError("document ids must start at 1 and grow by one")
        start = len(flat)
        flat.extend(r * width + t for t in range(n))
        for t in range(1, n + 1):  # a document ends where the id changes or the row's tokens end
            if t == n or row[t] != row[t - 1]:
                cu.append(start + t)
    return np.asarray(flat, dtype=np.int64), np.asarray(cu, dtype=np.int32)


def gather_rows(src, flat_index):
    """dst[r] = src[flat_index[r]] for rows of any width (bit copy)."""
    src = np.asarray(src)
    return src.reshape(src.shape[0], -1)[np.asarray(flat_index, dtype=np.int64)].reshape(
        (len(flat_index),) + src.shape[1:])


def scatter_rows(src, flat_index, dst_rows: int):
    """dst[flat_index[r]] = src[r]; every other row of dst is +0.0 (zero bits)."""
    src = np.asarray(src)
    bits = _as_bits(src)
    dst = np.zeros((dst_rows,) + src.shape[1:], dtype=bits.dtype)
    dst[np.asarray(flat_index, dtype=np.int64)] = bits
    return dst.view(src.dtype)
