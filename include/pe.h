/*
 * pe.h - packed, padding-free attention for AMD MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels. Many variable-length sequences share
 * one buffer with no padding; each sequence attends only to itself, and the
 * sequence boundaries come from int32 offsets (cu_seqlens). The operations are
 * those of the GiGL page "Source code for gigl.nn.packed_attention": packing a
 * padded grid (module docstring, data flow diagram and "Example"), attention
 * within each sequence (`_varlen_attention`), the first-token query variant
 * (`packed_attention` with `query_is_first_token`), the gradients
 * (`_varlen_attention_backward`) and the scatter back to the padded grid.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers without the `h_` prefix are DEVICE memory owned by the caller. The
 *   library never allocates or frees memory; scratch space comes from the
 *   caller's `workspace`, sized by the matching *_workspace_size call.
 * - Every device pointer must be 16-byte aligned. Outputs must not alias inputs.
 * - Token tensors are row-major [N, H, d]: token, then head, then head_dim,
 *   contiguous (the layout of a [tokens, heads, head_dim] tensor).
 * - cu_seqlens is int32 [B+1], cu[0] = 0, cu[b+1] = cu[b] + L_b, cu[B] = N.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream). All
 *   work is enqueued on it. Only pe_pack waits on the host (once, to read the
 *   token count); every other call is asynchronous and launches no more work
 *   than its host arguments fix, so it may be captured in a HIP graph.
 * - Host arguments are validated before anything is launched; a call that
 *   returns an error has enqueued nothing (except PE_ERR_CAPACITY and
 *   PE_ERR_LENGTHS from pe_pack, described there). PE_ERR_HIP means a HIP
 *   runtime call or launch failed.
 * - The attention calls do not validate device contents: cu_seqlens must be
 *   non-decreasing from 0 to N with every length in [1, max_seq_len], as
 *   pe_pack produces it. Anything else is undefined behaviour. With the
 *   environment variable PE_CHECK=1 (a debugging aid) every attention call
 *   first checks cu_seqlens on the device (cu[0] = 0, every length in
 *   [1, max_seq_len], cu[B] <= total_tokens) and waits for the answer: on a
 *   violation it returns PE_ERR_LENGTHS with nothing else launched. That mode
 *   synchronizes the stream (no graph capture); each call writes its answer to
 *   its own word of a ring of 256, so calls that overlap from other threads or
 *   streams do not interfere.
 * - dtype PE_FP32 computes in fp32 throughout (the GiGL page runs its kernel in
 *   fp32 because inference needs it). PE_BF16 reads and writes bf16 and
 *   accumulates in fp32; the probabilities are rounded to bf16 before they
 *   multiply V. Log-sum-exp values are always fp32.
 * - Supported head_dim: every multiple of 8 from 8 to 128 (the GiGL page's
 *   "Constraints" require a multiple of 8). Any other head_dim returns
 *   PE_ERR_UNSUPPORTED before anything is launched.
 */
#ifndef PE_H
#define PE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PE_OK = 0,
  PE_ERR_NULL = 1,        /* a required pointer is NULL */
  PE_ERR_ARG = 2,         /* a size, count, alignment or the scale is invalid */
  PE_ERR_UNSUPPORTED = 3, /* head_dim or dtype outside what the kernels support */
  PE_ERR_LENGTHS = 4,     /* pe_pack (or the PE_CHECK=1 mode) found a length outside [1, max_seq_len] */
  PE_ERR_CAPACITY = 5,    /* pe_pack: the token count exceeds `capacity` */
  PE_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required */
  PE_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed */
  PE_ERR_METADATA = 8     /* pe_flatten_*: packed metadata that is not consistent */
} pe_status;

typedef enum { PE_FP32 = 0, PE_BF16 = 1, PE_FP16 = 2 } pe_dtype;

/* Human-readable name of a status code. Never NULL. */
const char* pe_status_string(int status);

/* Tile height (packed query or key rows per work item) of the attention kernels. */
int32_t pe_attn_tile_rows(void);

/* ------------------------------------------------------------------------ pack
 * pe_pack: lengths -> cu_seqlens, flat_index and the packed rows of a grid.
 *
 * Source: GiGL module docstring, data flow diagram and "Example":
 * `pack_sequences(lengths, max_seq_len)` returns `flat_index` and the offsets;
 * `grid.flatten()[flat_index]` gathers the real tokens into a [num_tokens, dim]
 * buffer; packing needs one host read, of the total token count.
 *
 *   cu[0] = 0, cu[b+1] = cu[b] + L_b,  N = cu[B]
 *   flat_index[cu[b] + t] = b * max_seq_len + t            for t < L_b
 *   packed[r, :] = grid[flat_index[r], :]                   (rows of row_elems)
 *
 * `grid` is [num_seqs * max_seq_len, row_elems], i.e. a padded
 * [num_seqs, max_seq_len, row_elems] tensor; rows past a sequence's length are
 * never read. The copy moves bits (element size from `dtype`: 4 or 2 bytes).
 *
 * Arguments
 *   lengths      device int32 [num_seqs]; every length must lie in [1, max_seq_len]
 *   grid         device, or NULL to compute only the layout (cu_seqlens, flat_index)
 *   cu_seqlens   device int32 [num_seqs + 1], written
 *   flat_index   device int64 [capacity], or NULL; rows [0, N) written
 *   packed       device [capacity, row_elems], or NULL (must be NULL if grid is NULL)
 *   h_total_tokens  HOST int64, receives N (also on PE_ERR_CAPACITY)
 * Behaviour
 *   One device-to-host read of N and of a length-error flag; this is the only
 *   host wait in the library. If any length is outside [1, max_seq_len] it
 *   returns PE_ERR_LENGTHS after the read (cu_seqlens holds the running sum of
 *   the given values; nothing else written). If N exceeds INT32_MAX it returns
 *   PE_ERR_ARG. If N > capacity it returns PE_ERR_CAPACITY with
 *   *h_total_tokens = N: cu_seqlens is valid, flat_index and packed untouched;
 *   the caller may allocate N rows and call again.
 */
size_t pe_pack_workspace_size(int32_t num_seqs, int32_t max_seq_len, int64_t row_elems, pe_dtype dtype);
pe_status pe_pack(const int32_t* lengths, int32_t num_seqs, int32_t max_seq_len,
                  const void* grid, int64_t row_elems, pe_dtype dtype,
                  int32_t* cu_seqlens, int64_t* flat_index, void* packed, int64_t capacity,
                  int64_t* h_total_tokens, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------- pack without host read
 * pe_pack_async: pe_pack with no host read, so that a stream capture can record
 * it (the launch-bound short-batch case, where the packed-encoders README runs
 * the whole forward as one graph replay over fixed (batch, length) buckets).
 *
 * Source: as pe_pack; packed-encoders README, "CUDA graphs" (bucketed runner
 * over padded shapes, explicit batch and sequence bounds for packed graphs).
 *
 * Same layout as pe_pack. The token count stays on the device:
 *   status   device int64 [2], written: status[0] = N = sum of the lengths,
 *            status[1] = 0 (ok), 1 (a length outside [1, max_seq_len]) or
 *            2 (N > capacity)
 * On status[1] != 0 cu_seqlens is all zeros (a batch of empty sequences, which
 * every kernel queued behind reads as "no rows") and flat_index and packed are
 * untouched; nothing reads or writes out of bounds whatever the lengths.
 * `capacity` (rows of flat_index / packed) may be any value >= 0; the copy
 * kernels are sized for min(capacity, num_seqs * max_seq_len) rows and skip the
 * tail past N on the device. Asynchronous; host arguments are checked first
 * (PE_ERR_* and nothing enqueued). Workspace: pe_pack_workspace_size.
 */
pe_status pe_pack_async(const int32_t* lengths, int32_t num_seqs, int32_t max_seq_len, const void* grid,
                        int64_t row_elems, pe_dtype dtype, int32_t* cu_seqlens, int64_t* flat_index, void* packed,
                        int64_t capacity, int64_t* status, void* workspace, size_t workspace_bytes, void* stream);

/* -------------------------------------------------------------------- unpack
 * pe_unpack: packed rows -> padded grid, the inverse of the gather.
 *
 * Source: GiGL data flow diagram (the padded interface around the packed
 * buffer) and `_padded_packed_attention`, which scatters packed rows back into a
 * [num_sequences, max_seq_len] grid and fills the rest from `zeros_like`.
 *
 *   grid[b, t, :] = packed[cu[b] + t, :]   for t < L_b
 *   grid[b, t, :] = +0.0                   for L_b <= t < max_seq_len
 *
 * Arguments
 *   packed       device [total_tokens, row_elems]
 *   cu_seqlens   device int32 [num_seqs + 1]
 *   grid         device [num_seqs * max_seq_len, row_elems], every element written
 * A bit copy; no workspace; asynchronous.
 */
pe_status pe_unpack(const void* packed, const int32_t* cu_seqlens, int32_t num_seqs,
                    int32_t max_seq_len, int64_t total_tokens, int64_t row_elems, pe_dtype dtype,
                    void* grid, void* stream);

/* ----------------------------------------------------------------- work list
 * pe_worklist: cu_seqlens -> the attention kernels' work items.
 *
 * The packed rows are cut into tiles of `tile_rows` consecutive rows, so a
 * launch mixes ~30-token queries and multi-thousand-token documents (the
 * packed-encoders README, "Why packing?", on contrastive batches that mix
 * both) without padding any sequence to a tile. Item t covers rows
 * [t*R, min((t+1)*R, N)); its keys are those of every sequence the tile
 * touches. items[t] is the sequence holding row t*R (cu[b] <= t*R < cu[b+1]);
 * items[T] = num_seqs closes the list, T = ceil(N / R).
 *
 *   items   device int32 [ceil(total_tokens / tile_rows) + 1], written
 * Asynchronous. The attention calls run this themselves in their workspace;
 * it is exported so it can be checked and reused. The fp32 one-wave kernels
 * (head dims 32, 64) and the 16-bit kernels at head dims 32 and 64 (length
 * bounds above 64) build a sequence-aligned variant instead: tiles start at
 * every sequence's first row, so a tile never spans two sequences.
 */
pe_status pe_worklist(const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                      int32_t tile_rows, int32_t* items, void* stream);

/* ------------------------------------------------------------------- forward
 * pe_varlen_attn_fwd: non-causal attention within each packed sequence.
 *
 * Source: GiGL `_varlen_attention` ("query sequence i attends to key sequence
 * i"; offsets read on the device, length bounds as host ints, no host sync) and
 * `_varlen_attention_op` (output plus log-sum-exp, the latter computed only when
 * a gradient will be needed). For sequence b, head h, query row i in it:
 *
 *   s_j   = softmax_scale * <q[i,h,:], k[j,h,:]>   for j in [cu[b], cu[b+1])
 *   out[i,h,:] = sum_j exp(s_j - m) v[j,h,:] / sum_j exp(s_j - m),  m = max_j s_j
 *   lse[h, i]  = m + ln(sum_j exp(s_j - m))        (natural log, fp32)
 *
 * Arguments
 *   q, k, v      device [total_tokens, num_heads, head_dim] of `dtype`
 *   out          device [total_tokens, num_heads, head_dim] of `dtype`
 *   lse          device fp32 [num_heads, total_tokens], or NULL to skip it
 *   max_seq_len  upper bound on every length (host int, as the GiGL call takes)
 *   softmax_scale  finite and > 0; the GiGL call uses the SDPA default 1/sqrt(d)
 *   workspace    device, at least pe_attn_workspace_size(..., for_backward=0)
 *   total_tokens N = cu[B], or a capacity above it (rows of q, k, v, out and of
 *                lse's row stride); rows cu[B]..N-1 are then neither read nor
 *                written. This holds for every forward call (local, fused QKV,
 *                first-token), so a forward can follow pe_pack_async with no host read.
 */
size_t pe_attn_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                              int32_t head_dim, pe_dtype dtype, int for_backward);
pe_status pe_varlen_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                             int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len,
                             int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale,
                             void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------- first-token query
 * pe_varlen_attn_fwd_first_token: one query per sequence, its first token.
 *
 * Source: GiGL `packed_attention` with `query_is_first_token` (the caller
 * passes `query[cu_seqlens[:-1]]`; each sequence's single query attends over
 * all its keys; "all the anchor readout of the last layer needs"). The result
 * equals rows cu[:-1] of pe_varlen_attn_fwd.
 *
 *   q_first      device [num_seqs, num_heads, head_dim]
 *   k, v         device [total_tokens, num_heads, head_dim]
 *   out_first    device [num_seqs, num_heads, head_dim]
 *   lse_first    device fp32 [num_heads, num_seqs], or NULL
 * No workspace; asynchronous.
 */
pe_status pe_varlen_attn_fwd_first_token(const void* q_first, const void* k, const void* v,
                                         const int32_t* cu_seqlens, int32_t num_seqs,
                                         int64_t total_tokens, int32_t max_seq_len, int32_t num_heads,
                                         int32_t head_dim, pe_dtype dtype, float softmax_scale,
                                         void* out_first, float* lse_first, void* stream);

/* pe_varlen_attn_fwd_first_row: pe_varlen_attn_fwd_first_token with the query
 * gather fused: the query of sequence b is row cu_seqlens[b] of the packed
 * q [total_tokens, num_heads, head_dim], which GiGL's caller otherwise gathers
 * itself (`query[cu_seqlens[:-1]]`) before the call. Same outputs and errors.
 */
pe_status pe_varlen_attn_fwd_first_row(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                       int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len,
                                       int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale,
                                       void* out_first, float* lse_first, void* stream);

/* pe_varlen_attn_bwd_first_token: gradients of the first-token readout.
 *
 * Source: GiGL `packed_attention` runs the readout through its autograd-
 * registered varlen op with one query per sequence (cu_seqlens_q =
 * arange(num_seqs + 1)), so training flows through it; the backward of that op
 * (`_varlen_attention_backward`) takes the output and log-sum-exp and drops the
 * log-sum-exp's gradient. With one query per sequence, for key row j of
 * sequence b:
 *
 *   P_j = exp(s_j - lse_b)   D_b = <dout_b, out_b>   dS_j = P_j (<dout_b, v_j> - D_b)
 *   dv_j = P_j dout_b        dk_j = scale dS_j q_b   dq_b = scale sum_j dS_j k_j
 *
 * Arguments
 *   dout_first, q_first, out_first, dq_first   device [num_seqs, num_heads, head_dim] of `dtype`
 *   lse_first                                   device fp32 [num_heads, num_seqs] (required)
 *   k, v, dk, dv                                device [total_tokens, num_heads, head_dim] of `dtype`;
 *                                               every row of dk and dv is written
 * For pe_varlen_attn_fwd_first_row the gradient of the packed q is dq_first
 * placed at rows cu_seqlens[:-1] and zero elsewhere. No workspace;
 * asynchronous; deterministic (every output element has one writer).
 */
pe_status pe_varlen_attn_bwd_first_token(const void* dout_first, const void* q_first, const void* k, const void* v,
                                         const void* out_first, const float* lse_first, const int32_t* cu_seqlens,
                                         int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len,
                                         int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale,
                                         void* dq_first, void* dk, void* dv, void* stream);

/* ------------------------------------------------------------------ backward
 * pe_varlen_attn_bwd: gradients of pe_varlen_attn_fwd in q, k and v.
 *
 * Source: GiGL `_varlen_attention_backward` (gradients in query, key and value
 * from grad_output, the inputs, the output and the log-sum-exp; the gradient of
 * the log-sum-exp is dropped). Recomputes the probabilities from `lse`:
 *
 *   P_ij = exp(s_ij - lse_i)   D_i = <dout_i, out_i>   dS_ij = P_ij (<dout_i, v_j> - D_i)
 *   dv_j = sum_i P_ij dout_i   dq_i = scale sum_j dS_ij k_j   dk_j = scale sum_i dS_ij q_i
 *
 * Arguments
 *   dout, q, k, v, out   device [total_tokens, num_heads, head_dim] of `dtype`
 *   lse                  device fp32 [num_heads, total_tokens] from the forward
 *   dq, dk, dv           device [total_tokens, num_heads, head_dim] of `dtype`, written
 *   workspace            at least pe_attn_workspace_size(..., for_backward=1); with
 *                        pe_attn_bwd_workspace_size(...) bytes (more for fp32 at head dims
 *                        32 and 64 with max_seq_len <= 256) the fp32 global-attention path
 *                        passes the blocks of dS
 *                        from its dK/dV pass to its dQ pass through the workspace instead of
 *                        recomputing S and dP for dQ. Both sizes give gradients within the
 *                        same tolerances; each is deterministic.
 * Deterministic: no floating-point atomics; the same inputs give the same bits.
 */
/* The workspace size of the fastest backward path: pe_attn_workspace_size(..., 1), plus for
 * fp32 at head dims 32 and 64 with max_seq_len <= 256 one 32x32 fp32 block per (32-row query
 * tile, 32-row key block) of a sequence of max_seq_len rows, per head:
 * num_heads * (total_tokens / 32 + num_seqs) * ceil(max_seq_len / 32) * 4096 bytes (about
 * 4.1 GB for 368,449 tokens in 4096 sequences of up to 256 rows and 8 heads; a caller that
 * passes only the smaller workspace gets the path that recomputes S and dP instead).
 * Returns 0 for invalid sizes. */
size_t pe_attn_bwd_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len,
                                  int32_t num_heads, int32_t head_dim, pe_dtype dtype);
pe_status pe_varlen_attn_bwd(const void* dout, const void* q, const void* k, const void* v,
                             const void* out, const float* lse, const int32_t* cu_seqlens,
                             int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len,
                             int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale,
                             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                             void* stream);

/* ---------------------------------------------------------- local attention
 * pe_varlen_attn_fwd_local / pe_varlen_attn_bwd_local: pe_varlen_attn_fwd and
 * pe_varlen_attn_bwd with each query row i seeing only the keys j of its own
 * sequence with |i - j| <= window (sliding-window, non-causal).
 *
 * Source: the packed-encoders README, backend table: its short-sequence kernel
 * serves "global or local" attention (a "local-64" variant) and its
 * FlashAttention backend prunes by sliding window. The README does not say how
 * 64 maps to a radius; `window` is the radius itself (a window of 64 keys
 * centred on the query is window = 32). Key tiles outside every row's band are
 * skipped, so the cost falls with the window.
 *
 * Arguments as for the global calls, plus
 *   window   >= 0 (PE_ERR_ARG otherwise); window >= max_seq_len - 1 is global
 *            attention. The backward must be given the window of its forward.
 */
pe_status pe_varlen_attn_fwd_local(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                   int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len,
                                   int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale,
                                   int32_t window, void* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream);
pe_status pe_varlen_attn_bwd_local(const void* dout, const void* q, const void* k, const void* v,
                                   const void* out, const float* lse, const int32_t* cu_seqlens,
                                   int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len,
                                   int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale,
                                   int32_t window, void* dq, void* dk, void* dv, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ---------------------------------------------- forward without allocation
 * pe_varlen_attn_fwd_noalloc: pe_varlen_attn_fwd with no workspace argument, for
 * callers that cannot allocate device memory or pass a workspace (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Its work list lives in a fixed scratch array the library holds in device
 * memory (pe_noalloc_scratch_size() bytes, 1 MiB, one copy on each GPU it is
 * called on, kept until the process ends); the call itself allocates nothing.
 *
 * Arguments, layouts, results and errors as pe_varlen_attn_fwd, except:
 *   - a batch whose work list would not fit the scratch array, i.e.
 *     pe_attn_workspace_size(num_seqs, total_tokens, num_heads, head_dim,
 *     dtype, 0) > pe_noalloc_scratch_size() (about total_tokens / 32 + num_seqs
 *     + 1 int32 entries, so up to ~8 million tokens), returns PE_ERR_WORKSPACE
 *     before anything is launched;
 *   - every call on one GPU shares that GPU's array: calls that overlap on one
 *     GPU (concurrent streams, or host threads) race and are not allowed. Each
 *     call rewrites the whole list before its kernel reads it, so nothing in it
 *     needs to start at zero.
 * The first call on a device looks the array's address up on that device (the
 * device current at the call).
 */
size_t pe_noalloc_scratch_size(void);
pe_status pe_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                     int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len,
                                     int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale,
                                     void* out, float* lse, void* stream);

/* ---------------------------------------------------------------- fused QKV
 * pe_varlen_attn_fwd_qkv / pe_varlen_attn_bwd_qkv: the attention calls on a
 * fused projection buffer qkv [total_tokens, 3, num_heads, head_dim] (Q, K and V
 * of a token side by side in one row, the layout of a fused QKV projection),
 * read in place through a row stride of 3 * num_heads * head_dim elements; the
 * backward writes dqkv in the same fused layout.
 *
 * Source: the packed-encoders README (its kernels consume the Hugging Face
 * weight layout as is, nothing re-packed; ModernBERT projects Q, K and V with
 * one fused matrix).
 *
 *   window   -1 for global attention, or the local radius as in
 *            pe_varlen_attn_fwd_local (window >= 0)
 *   out, dout   device [total_tokens, num_heads, head_dim] (dense); lse fp32 [H, N]
 * Everything else as pe_varlen_attn_fwd / pe_varlen_attn_bwd (same workspace).
 */
pe_status pe_varlen_attn_fwd_qkv(const void* qkv, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                 int32_t max_seq_len, int32_t num_heads, int32_t head_dim, pe_dtype dtype,
                                 float softmax_scale, int32_t window, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);
pe_status pe_varlen_attn_bwd_qkv(const void* dout, const void* qkv, const void* out, const float* lse,
                                 const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                 int32_t max_seq_len, int32_t num_heads, int32_t head_dim, pe_dtype dtype,
                                 float softmax_scale, int32_t window, void* dqkv, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------- captured bucket forward
 * pe_forward_graph_create / pe_graph_launch / pe_graph_destroy: the whole padded
 * forward of one fixed bucket (num_seqs sequence slots, max_seq_len) recorded
 * once as a HIP graph and replayed with one launch.
 *
 * Source: packed-encoders README, "CUDA graphs": short-sequence inference is
 * bound by host launches; a bucketed runner collapses the forward to a single
 * replay; packed graphs take explicit batch and sequence bounds; graphs serve
 * only gradient-free calls.
 *
 * One replay computes, on the buffers given here, what these calls would:
 *   pe_pack_async(lengths, qkv_grid -> cu_seqlens, qkv_packed; capacity C = num_seqs * max_seq_len)
 *   pe_varlen_attn_fwd_qkv(qkv_packed, total_tokens = C, window -> out_packed, lse)
 *   pe_unpack(out_packed -> out_grid)
 * bit for bit. For buckets of up to ~16k work-list entries (about C / pack rows per
 * tile + C / 128) the scan and both work lists run as one single-workgroup kernel,
 * so a replay is four dependent kernels instead of six.
 * Buffers (device, caller-owned, fixed for the life of the graph)
 *   lengths     int32 [num_seqs]; the caller writes the batch before each replay.
 *               A batch of fewer sequences fills the unused slots with length 1:
 *               sequences never interact, so those slots change no real output.
 *   qkv_grid    [num_seqs, max_seq_len, 3, num_heads, head_dim] of dtype (fused Q, K, V)
 *   cu_seqlens  int32 [num_seqs + 1];  qkv_packed [C, 3, H, d];  out_packed [C, H, d]
 *   lse         fp32 [H, C], or NULL;  out_grid [num_seqs, max_seq_len, H, d]
 *   status      int64 [2] as in pe_pack_async (on an error out_grid is all +0.0)
 *   workspace   at least pe_forward_graph_workspace_size(...) bytes
 * Rows of out_packed and lse past the replay's N are not written. *graph is
 * NULL on any error. Creation captures on a stream of its own and enqueues
 * nothing; pe_graph_launch enqueues one replay on `stream` (asynchronous);
 * replays on one graph must not overlap (they share every buffer).
 */
typedef struct pe_graph_s* pe_graph;
size_t pe_forward_graph_workspace_size(int32_t num_seqs, int32_t max_seq_len, int32_t num_heads, int32_t head_dim,
                                       pe_dtype dtype);
pe_status pe_forward_graph_create(const int32_t* lengths, int32_t num_seqs, int32_t max_seq_len, const void* qkv_grid,
                                  int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale,
                                  int32_t window, int32_t* cu_seqlens, void* qkv_packed, void* out_packed, float* lse,
                                  void* out_grid, int64_t* status, void* workspace, size_t workspace_bytes,
                                  pe_graph* graph);
pe_status pe_graph_launch(pe_graph graph, void* stream);
pe_status pe_graph_destroy(pe_graph graph);

/* ---------------------------------------------------------- packing metadata
 * pe_position_ids / pe_document_ids: per packed token, its position inside its
 * own sequence (int64, position_ids[r] = r - cu[b]) and the 1-based index of its
 * sequence (int32, document_ids[r] = b + 1).
 *
 * Sources: the packed-encoders README's direct packed entry takes position ids
 * built as the concatenation of arange(L_b); NeMo's indexed packing mask marks
 * document i (1-based) with i (padding 0), which for a stream without padding is
 * document_ids. Either output may be NULL. Asynchronous; no workspace.
 */
pe_status pe_position_ids(const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                          int64_t* position_ids, int32_t* document_ids, void* stream);

/* pe_flatten_packed_metadata / pe_flatten_document_mask: NeMo's batch-major
 * packed metadata to one token stream.
 *
 * Source: NeMo `flatten_packed_sequence_metadata` (token indices [batch,
 * sequence] row-local with -1 padding, cumulative lengths [batch, max_documents
 * + 1] row-local with -1 padding, flattened to flat token indices into the padded
 * [batch, sequence] grid; inconsistent layouts, boundaries or token counts are
 * errors) and NeMo's indexed packing mask ([batch, sequence]; document i of a
 * row marked i, padding 0).
 *
 *   token_index    device int32 [rows, width]: a strictly increasing prefix of
 *                  indices in [0, width), then only -1
 *   cu_local       device int32 [rows, max_docs + 1]: 0, then strictly increasing
 *                  ends, then only -1; the last end equals the row's token count
 *                  (a row without documents is all -1 or 0 then -1)
 *   document_mask  device int32 [rows, width]: 1, then ids equal to or one above
 *                  their predecessor, then only 0
 * Outputs (rows in order, each row's tokens in order):
 *   flat_index     device int64 [capacity] or NULL: r * width + the token's index
 *   cu_seqlens     device int32 [doc_capacity + 1]: 0 and the end of every document
 *                  in the stream (usable as the attention calls' cu_seqlens)
 *   *h_total_tokens, *h_num_docs   host: the stream's token and document counts
 * One host read (counts and the validity flag), as pe_pack. PE_ERR_METADATA if
 * any row breaks the rules (outputs untouched); PE_ERR_CAPACITY if the counts
 * exceed capacity / doc_capacity (counts still reported, outputs untouched).
 * workspace: pe_flatten_workspace_size(rows) bytes.
 */
size_t pe_flatten_workspace_size(int32_t rows);
pe_status pe_flatten_packed_metadata(const int32_t* token_index, const int32_t* cu_local, int32_t rows, int32_t width,
                                     int32_t max_docs, int64_t* flat_index, int32_t* cu_seqlens, int64_t capacity,
                                     int64_t doc_capacity, int64_t* h_total_tokens, int64_t* h_num_docs,
                                     void* workspace, size_t workspace_bytes, void* stream);
pe_status pe_flatten_document_mask(const int32_t* document_mask, int32_t rows, int32_t width, int64_t* flat_index,
                                   int32_t* cu_seqlens, int64_t capacity, int64_t doc_capacity,
                                   int64_t* h_total_tokens, int64_t* h_num_docs, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* pe_gather_rows / pe_scatter_rows: the row copies of pack and unpack for any
 * flat index (e.g. one from pe_flatten_*): dst[r] = src[flat_index[r]] for
 * r < n, and dst[flat_index[r]] = src[r] with every other row of dst zero
 * (+0.0). Source: GiGL's `grid.flatten()[flat_index]` gather and its scatter
 * back into zeros (the data flow of the packed path).
 *   src, dst         device, rows of row_elems elements of `dtype`
 *   src_rows         rows of src (gather) / dst_rows rows of dst (scatter);
 *                    index entries outside them give a zero row (gather) or are
 *                    skipped (scatter)
 * Bit copies; asynchronous; no workspace.
 */
pe_status pe_gather_rows(const void* src, int64_t src_rows, const int64_t* flat_index, int64_t n, int64_t row_elems,
                         pe_dtype dtype, void* dst, void* stream);
pe_status pe_scatter_rows(const void* src, const int64_t* flat_index, int64_t n, int64_t row_elems, pe_dtype dtype,
                          void* dst, int64_t dst_rows, void* stream);

/* ------------------------------------------------------------- kernel timing
 * Measurement support, not part of the computation. While enabled, every
 * kernel the library launches is bracketed by two HIP events recorded on the
 * launch's stream (the events come from a pool the library creates on first
 * use; no device memory is allocated). pe_timing_read waits for the recorded
 * events and writes, in launch order, the kernel name (NUL-terminated, at most
 * 31 characters, into `names` + 32*i; `names` may be NULL) and its duration in
 * milliseconds (`ms`, may be NULL; -1 if unavailable) of up to `max_records`
 * kernels launched since the previous read, forgets all records, and returns
 * how many it wrote. At most 4096 kernels are recorded between reads. Disabled
 * by default; disabling drops unread records. Not thread-safe.
 */
pe_status pe_timing_enable(int on);
int pe_timing_read(char* names, float* ms, int max_records);

#ifdef __cplusplus
}
#endif

#endif /* PE_H */
