// C ABI of the packed-attention library: argument validation, workspace
// layout, and the launch sequence of every call. See include/pe.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "kernels.h"
#include "pe.h"

namespace {

// Checked mode: with PE_CHECK=1 in the environment, every attention call first
// checks cu_seqlens on the device and waits for the answer; on a violation it
// returns PE_ERR_LENGTHS with nothing else launched. A debugging aid: it
// synchronizes the stream (so it cannot be captured in a graph). Each call takes
// the next of kCheckSlots answer words in turn, so calls that overlap (from other
// threads, on other streams) write different words.
constexpr uint32_t kCheckSlots = 256;
__device__ int32_t g_check_flags[kCheckSlots];
std::atomic<uint32_t> g_check_next{0};

bool check_mode() {
  const char* e = std::getenv("PE_CHECK");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

pe_status check_cu(const int32_t* cu, int32_t B, int64_t N, int32_t S, hipStream_t st) {
  if (!check_mode()) return PE_OK;
  int32_t* flags = nullptr;
  if (hipGetSymbolAddress(reinterpret_cast<void**>(&flags), HIP_SYMBOL(g_check_flags)) != hipSuccess)
    return PE_ERR_HIP;
  int32_t* flag = flags + g_check_next.fetch_add(1, std::memory_order_relaxed) % kCheckSlots;
  if (pe::launch_check_cu(cu, B, N, S, flag, st) != hipSuccess) return PE_ERR_HIP;
  int32_t h = 0;
  if (hipMemcpyAsync(&h, flag, sizeof h, hipMemcpyDeviceToHost, st) != hipSuccess) return PE_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return PE_ERR_HIP;
  return h ? PE_ERR_LENGTHS : PE_OK;
}

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_head_dim(int32_t d) { return pe::head_dim_supported(d); }

bool valid_dtype(int dt) { return dt == PE_FP32 || dt == PE_BF16 || dt == PE_FP16; }

int64_t elem_bytes(pe_dtype dt) { return dt == PE_FP32 ? 4 : 2; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

pe_status hip_status(hipError_t e) { return e == hipSuccess ? PE_OK : PE_ERR_HIP; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A work list of any tiling the kernels use: the sequence-aligned one of kAttnWaveRows rows
// (N / 32 + B + 1 entries) is the longest.
size_t items_bytes(int32_t num_seqs, int64_t total_tokens) {
  return round_up(static_cast<size_t>(total_tokens / pe::kAttnWaveRows + num_seqs + 1) * sizeof(int32_t));
}

// Elements between rows of separate [N, H, d] tensors.
int64_t dense_ld(int32_t num_heads, int32_t head_dim) { return static_cast<int64_t>(num_heads) * head_dim; }

// The fp32 backward's dS hand-off: one 32x32 fp32 block per (query tile, key block) of every
// sequence and head, [H][N/32 + B][nb_max][1024] floats (nb_max: 32-row blocks of a sequence of
// max_seq_len rows). The region reserves nb_max blocks for every query tile, so it is offered
// only for length bounds up to kDsMaxSeqLen (8 blocks per tile; the blocks used are the
// sum over sequences of ceil(L/32)^2 per head).
constexpr int32_t kDsMaxSeqLen = 256;
int32_t nb_max(int32_t max_seq_len) { return (max_seq_len + pe::kAttnWaveRows - 1) / pe::kAttnWaveRows; }
bool ds_handoff(pe_dtype dtype, int32_t head_dim, int32_t num_heads, int32_t max_seq_len) {
  return dtype == PE_FP32 && max_seq_len <= kDsMaxSeqLen &&
         pe::attn_f32_wave_supported(head_dim, dense_ld(num_heads, head_dim), num_heads);
}
size_t ds_bytes(int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len, int32_t num_heads) {
  return round_up(static_cast<size_t>(num_heads) *
                  static_cast<size_t>(total_tokens / pe::kAttnWaveRows + num_seqs) *
                  static_cast<size_t>(nb_max(max_seq_len)) * 1024 * sizeof(float));
}

// Checks shared by the attention calls.
pe_status check_attn_args(int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len, int32_t num_heads,
                          int32_t head_dim, int dtype, float scale) {
  if (num_seqs < 1 || max_seq_len < 1 || num_heads < 1) return PE_ERR_ARG;
  if (total_tokens < num_seqs || total_tokens > INT32_MAX) return PE_ERR_ARG;
  if (total_tokens > static_cast<int64_t>(num_seqs) * max_seq_len) return PE_ERR_ARG;
  if (!valid_dtype(dtype) || !supported_head_dim(head_dim)) return PE_ERR_UNSUPPORTED;
  if (!(std::isfinite(scale) && scale > 0.f)) return PE_ERR_ARG;
  if (ceil_div(total_tokens, pe::kAttnTileRows) * num_heads > INT32_MAX) return PE_ERR_ARG;
  if (static_cast<int64_t>(num_heads) * head_dim > (1 << 16)) return PE_ERR_UNSUPPORTED;
  return PE_OK;
}

}  // namespace

extern "C" {

const char* pe_status_string(int status) {
  switch (status) {
    case PE_OK: return "PE_OK";
    case PE_ERR_NULL: return "PE_ERR_NULL: a required pointer is NULL";
    case PE_ERR_ARG: return "PE_ERR_ARG: invalid size, count, alignment or scale";
    case PE_ERR_UNSUPPORTED: return "PE_ERR_UNSUPPORTED: head_dim or dtype not supported";
    case PE_ERR_LENGTHS: return "PE_ERR_LENGTHS: a sequence length lies outside [1, max_seq_len]";
    case PE_ERR_CAPACITY: return "PE_ERR_CAPACITY: token count exceeds the output capacity";
    case PE_ERR_WORKSPACE: return "PE_ERR_WORKSPACE: workspace missing or too small";
    case PE_ERR_METADATA: return "PE_ERR_METADATA: inconsistent packed metadata (indices, boundaries or counts)";
    case PE_ERR_HIP: return "PE_ERR_HIP: a HIP runtime call or kernel launch failed";
    default: return "unknown pe_status";
  }
}

int32_t pe_attn_tile_rows(void) { return pe::kAttnTileRows; }

// ------------------------------------------------------------------------ pack

}  // extern "C"

namespace {
// Bytes of the copy work list a pack call may build: tiles of pack_tile_rows(row bytes)
// rows when it copies rows, of pack_tile_rows(64) rows when it writes flat_index only
// (the list for the smaller tiles is the longer one).
size_t pack_items_bytes(int32_t num_seqs, int32_t max_seq_len, int64_t row_elems, pe_dtype dtype) {
  const int64_t rowbytes = (row_elems > 0 ? row_elems : 1) * elem_bytes(dtype);
  const int64_t R = std::min(pe::pack_tile_rows(rowbytes), pe::pack_tile_rows(64));
  const int64_t max_rows = static_cast<int64_t>(num_seqs) * max_seq_len;
  return round_up(static_cast<size_t>(ceil_div(max_rows, R) + 1) * sizeof(int32_t));
}
// The scan's scratch in a pack workspace: after the result words and the copy work list.
int64_t* scan_part(void* workspace, int32_t num_seqs, int32_t max_seq_len, int64_t row_elems, pe_dtype dtype) {
  if (pe::scan_scratch_bytes(num_seqs) == 0) return nullptr;
  return reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + kAlign +
                                    pack_items_bytes(num_seqs, max_seq_len, row_elems, dtype));
}
}  // namespace

extern "C" {

size_t pe_pack_workspace_size(int32_t num_seqs, int32_t max_seq_len, int64_t row_elems, pe_dtype dtype) {
  if (num_seqs < 1 || max_seq_len < 1) return 0;
  return kAlign + pack_items_bytes(num_seqs, max_seq_len, row_elems, dtype) +
         round_up(static_cast<size_t>(pe::scan_scratch_bytes(num_seqs)));
}

pe_status pe_pack(const int32_t* lengths, int32_t num_seqs, int32_t max_seq_len, const void* grid,
                  int64_t row_elems, pe_dtype dtype, int32_t* cu_seqlens, int64_t* flat_index,
                  void* packed, int64_t capacity, int64_t* h_total_tokens, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (!lengths || !cu_seqlens || !h_total_tokens) return PE_ERR_NULL;
  if (grid && !packed) return PE_ERR_NULL;
  if (!grid && packed) return PE_ERR_ARG;
  if (num_seqs < 1 || max_seq_len < 1 || capacity < 0) return PE_ERR_ARG;
  if (!valid_dtype(dtype)) return PE_ERR_UNSUPPORTED;
  if (grid && row_elems < 1) return PE_ERR_ARG;
  for (const void* p : {static_cast<const void*>(lengths), static_cast<const void*>(cu_seqlens),
                        static_cast<const void*>(flat_index), grid, static_cast<const void*>(packed),
                        static_cast<const void*>(workspace)})
    if (p && !aligned16(p)) return PE_ERR_ARG;
  if (!workspace || workspace_bytes < pe_pack_workspace_size(num_seqs, max_seq_len, row_elems, dtype))
    return PE_ERR_WORKSPACE;

  hipStream_t st = as_stream(stream);
  int64_t* result = static_cast<int64_t*>(workspace);
  int32_t* items = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + kAlign);
  hipError_t e = pe::launch_scan(lengths, num_seqs, max_seq_len, -1, cu_seqlens, result,
                                 scan_part(workspace, num_seqs, max_seq_len, row_elems, dtype), st);
  if (e != hipSuccess) return PE_ERR_HIP;
  // The one host read of the library: the token count and the length-error flag.
  int64_t host[2] = {0, 0};
  e = hipMemcpyAsync(host, result, sizeof(host), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return PE_ERR_HIP;
  *h_total_tokens = host[0];
  if (host[1] != 0) return PE_ERR_LENGTHS;
  const int64_t N = host[0];
  if (N > INT32_MAX) return PE_ERR_ARG;
  if (!flat_index && !packed) return PE_OK;
  if (N > capacity) return PE_ERR_CAPACITY;
  const int64_t rowbytes = (packed ? row_elems : 1) * elem_bytes(dtype);
  const int32_t R = pe::pack_tile_rows(packed ? rowbytes : 64);
  e = pe::launch_worklist(cu_seqlens, num_seqs, N, R, items, st);
  if (e != hipSuccess) return PE_ERR_HIP;
  e = pe::launch_pack_rows(grid, packed, flat_index, cu_seqlens, items, num_seqs, max_seq_len, rowbytes, N,
                           R, st);
  return hip_status(e);
}

// -------------------------------------------------------------------- unpack

pe_status pe_unpack(const void* packed, const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seq_len,
                    int64_t total_tokens, int64_t row_elems, pe_dtype dtype, void* grid, void* stream) {
  if (!packed || !cu_seqlens || !grid) return PE_ERR_NULL;
  if (num_seqs < 1 || max_seq_len < 1 || row_elems < 1) return PE_ERR_ARG;
  if (total_tokens < num_seqs || total_tokens > INT32_MAX ||
      total_tokens > static_cast<int64_t>(num_seqs) * max_seq_len)
    return PE_ERR_ARG;
  if (!valid_dtype(dtype)) return PE_ERR_UNSUPPORTED;
  if (!aligned16(packed) || !aligned16(cu_seqlens) || !aligned16(grid)) return PE_ERR_ARG;
  return hip_status(pe::launch_unpack_rows(packed, grid, cu_seqlens, num_seqs, max_seq_len,
                                           row_elems * elem_bytes(dtype), as_stream(stream)));
}

// ----------------------------------------------------------------- work list

pe_status pe_worklist(const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens, int32_t tile_rows,
                      int32_t* items, void* stream) {
  if (!cu_seqlens || !items) return PE_ERR_NULL;
  if (num_seqs < 1 || tile_rows < 1 || total_tokens < num_seqs || total_tokens > INT32_MAX) return PE_ERR_ARG;
  return hip_status(pe::launch_worklist(cu_seqlens, num_seqs, total_tokens, tile_rows, items,
                                        as_stream(stream)));
}

// ------------------------------------------------------------------- forward

size_t pe_attn_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t head_dim,
                              pe_dtype dtype, int for_backward) {
  (void)head_dim;
  (void)dtype;
  if (num_seqs < 1 || total_tokens < 0 || num_heads < 1) return 0;
  size_t s = items_bytes(num_seqs, total_tokens);
  if (for_backward)  // a second list and two [H, N] float arrays
    s += items_bytes(num_seqs, total_tokens) +
         2 * round_up(static_cast<size_t>(total_tokens) * num_heads * sizeof(float));
  return s;
}

size_t pe_attn_bwd_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len, int32_t num_heads,
                                  int32_t head_dim, pe_dtype dtype) {
  if (num_seqs < 1 || total_tokens < 0 || num_heads < 1 || max_seq_len < 1) return 0;
  size_t s = pe_attn_workspace_size(num_seqs, total_tokens, num_heads, head_dim, dtype, 1);
  if (ds_handoff(dtype, head_dim, num_heads, max_seq_len)) s += ds_bytes(num_seqs, total_tokens, max_seq_len, num_heads);
  return s;
}

}  // extern "C"

namespace {

// The work list of a forward (the one pe::attn_fwd_list names), built on `st`.
hipError_t build_fwd_list(pe::FwdList kind, const int32_t* cu, int32_t B, int64_t N, int32_t* items, hipStream_t st) {
  switch (kind) {
    case pe::kFwdListSeq32: return pe::launch_seq_worklist(cu, B, N, pe::kAttnWaveRows, items, st);
    case pe::kFwdListSeq128: return pe::launch_seq_worklist(cu, B, N, pe::kAttnTileRows, items, st);
    case pe::kFwdListNone: return hipSuccess;
    default: return pe::launch_worklist(cu, B, N, pe::kAttnTileRows, items, st);
  }
}

// The forward for every entry point: win is the local-attention radius, or -1.

pe_status fwd_impl(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, int32_t num_seqs,
                   int64_t total_tokens, int32_t max_seq_len, int32_t num_heads, int32_t head_dim, pe_dtype dtype,
                   float softmax_scale, int32_t win, int64_t ld, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !cu_seqlens || !out) return PE_ERR_NULL;
  const pe_status s =
      check_attn_args(num_seqs, total_tokens, max_seq_len, num_heads, head_dim, dtype, softmax_scale);
  if (s != PE_OK) return s;
  for (const void* p : {q, k, v, static_cast<const void*>(cu_seqlens), static_cast<const void*>(out),
                        static_cast<const void*>(lse), static_cast<const void*>(workspace)})
    if (p && !aligned16(p)) return PE_ERR_ARG;
  if (!workspace || workspace_bytes < pe_attn_workspace_size(num_seqs, total_tokens, num_heads, head_dim, dtype, 0))
    return PE_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  if (const pe_status c = check_cu(cu_seqlens, num_seqs, total_tokens, max_seq_len, st); c != PE_OK) return c;
  int32_t* items = static_cast<int32_t*>(workspace);
  hipError_t e = build_fwd_list(pe::attn_fwd_list(dtype, head_dim, max_seq_len, ld, num_heads), cu_seqlens,
                                num_seqs, total_tokens, items, st);
  if (e != hipSuccess) return PE_ERR_HIP;
  e = pe::launch_attn_fwd(dtype, head_dim, q, k, v, cu_seqlens, items, num_seqs,
                          static_cast<int32_t>(total_tokens), num_heads, max_seq_len, win, ld, softmax_scale, out,
                          lse, st);
  return hip_status(e);
}


// A window at least max_seq_len - 1 keeps every key of every sequence: global attention.
int32_t effective_window(int32_t window, int32_t max_seq_len) { return window >= max_seq_len - 1 ? -1 : window; }

}  // namespace

extern "C" {

pe_status pe_varlen_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                             int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len, int32_t num_heads,
                             int32_t head_dim, pe_dtype dtype, float softmax_scale, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, cu_seqlens, num_seqs, total_tokens, max_seq_len, num_heads, head_dim, dtype,
                  softmax_scale, -1, dense_ld(num_heads, head_dim), out, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------ forward without allocation

namespace {

// The work list of pe_varlen_attn_fwd_noalloc, in device memory the library holds
// for the process's lifetime (one copy per GPU it runs on). kNoAllocScratchBytes
// bounds the batch: the list takes pe_attn_workspace_size(..., 0) bytes.
constexpr size_t kNoAllocScratchBytes = size_t{1} << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on each GPU, looked up once per device with that
// device current (the host-side name is not a device address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

pe_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return PE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PE_OK;
}

}  // namespace

extern "C" {

size_t pe_noalloc_scratch_size(void) { return kNoAllocScratchBytes; }

pe_status pe_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                     int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len, int32_t num_heads,
                                     int32_t head_dim, pe_dtype dtype, float softmax_scale, void* out, float* lse,
                                     void* stream) {
  // sizes first: a batch whose work list exceeds the built-in scratch is rejected before
  // the device is touched
  if (num_seqs >= 1 && total_tokens >= 0 && num_heads >= 1 &&
      pe_attn_workspace_size(num_seqs, total_tokens, num_heads, head_dim, dtype, 0) > kNoAllocScratchBytes)
    return PE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (const pe_status s = scratch_on_current_device(&ws); s != PE_OK) return s;
  return fwd_impl(q, k, v, cu_seqlens, num_seqs, total_tokens, max_seq_len, num_heads, head_dim, dtype,
                  softmax_scale, -1, dense_ld(num_heads, head_dim), out, lse, ws, kNoAllocScratchBytes, stream);
}

pe_status pe_varlen_attn_fwd_local(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                   int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len, int32_t num_heads,
                                   int32_t head_dim, pe_dtype dtype, float softmax_scale, int32_t window, void* out,
                                   float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (window < 0) return PE_ERR_ARG;
  return fwd_impl(q, k, v, cu_seqlens, num_seqs, total_tokens, max_seq_len, num_heads, head_dim, dtype,
                  softmax_scale, effective_window(window, max_seq_len), dense_ld(num_heads, head_dim), out, lse,
                  workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

pe_status first_impl(const void* q, int32_t gather, const void* k, const void* v, const int32_t* cu_seqlens,
                     int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len, int32_t num_heads, int32_t head_dim,
                     pe_dtype dtype, float softmax_scale, void* out_first, float* lse_first, void* stream) {
  if (!q || !k || !v || !cu_seqlens || !out_first) return PE_ERR_NULL;
  const pe_status s =
      check_attn_args(num_seqs, total_tokens, max_seq_len, num_heads, head_dim, dtype, softmax_scale);
  if (s != PE_OK) return s;
  for (const void* p : {q, k, v, static_cast<const void*>(cu_seqlens), static_cast<const void*>(out_first),
                        static_cast<const void*>(lse_first)})
    if (p && !aligned16(p)) return PE_ERR_ARG;
  if (const pe_status c = check_cu(cu_seqlens, num_seqs, total_tokens, max_seq_len, as_stream(stream)); c != PE_OK)
    return c;
  return hip_status(pe::launch_attn_fwd_first(dtype, head_dim, q, k, v, cu_seqlens, num_seqs,
                                              static_cast<int32_t>(total_tokens), num_heads, max_seq_len, gather,
                                              static_cast<int64_t>(num_heads) * head_dim, softmax_scale, out_first,
                                              lse_first, as_stream(stream)));
}

}  // namespace

extern "C" {

pe_status pe_varlen_attn_fwd_first_token(const void* q_first, const void* k, const void* v,
                                         const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                         int32_t max_seq_len, int32_t num_heads, int32_t head_dim,
                                         pe_dtype dtype, float softmax_scale, void* out_first, float* lse_first,
                                         void* stream) {
  return first_impl(q_first, 0, k, v, cu_seqlens, num_seqs, total_tokens, max_seq_len, num_heads, head_dim, dtype,
                    softmax_scale, out_first, lse_first, stream);
}

pe_status pe_varlen_attn_fwd_first_row(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                       int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len,
                                       int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale,
                                       void* out_first, float* lse_first, void* stream) {
  return first_impl(q, 1, k, v, cu_seqlens, num_seqs, total_tokens, max_seq_len, num_heads, head_dim, dtype,
                    softmax_scale, out_first, lse_first, stream);
}

pe_status pe_varlen_attn_bwd_first_token(const void* dout_first, const void* q_first, const void* k, const void* v,
                                         const void* out_first, const float* lse_first, const int32_t* cu_seqlens,
                                         int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len,
                                         int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale,
                                         void* dq_first, void* dk, void* dv, void* stream) {
  if (!dout_first || !q_first || !k || !v || !out_first || !lse_first || !cu_seqlens || !dq_first || !dk || !dv)
    return PE_ERR_NULL;
  const pe_status s =
      check_attn_args(num_seqs, total_tokens, max_seq_len, num_heads, head_dim, dtype, softmax_scale);
  if (s != PE_OK) return s;
  for (const void* p : {dout_first, q_first, k, v, out_first, static_cast<const void*>(lse_first),
                        static_cast<const void*>(cu_seqlens), static_cast<const void*>(dq_first),
                        static_cast<const void*>(dk), static_cast<const void*>(dv)})
    if (!aligned16(p)) return PE_ERR_ARG;
  if (const pe_status c = check_cu(cu_seqlens, num_seqs, total_tokens, max_seq_len, as_stream(stream)); c != PE_OK)
    return c;
  return hip_status(pe::launch_attn_bwd_first(dtype, head_dim, dout_first, q_first, k, v, out_first,
                                              lse_first, cu_seqlens, num_seqs, static_cast<int32_t>(total_tokens),
                                              num_heads, max_seq_len, static_cast<int64_t>(num_heads) * head_dim,
                                              softmax_scale,
                                              dq_first, dk, dv, as_stream(stream)));
}

// ------------------------------------------------------------------ backward

}  // extern "C"

namespace {

// The backward for every entry point: win is the local-attention radius, or -1.
pe_status bwd_impl(const void* dout, const void* q, const void* k, const void* v, const void* out, const float* lse,
                   const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens, int32_t max_seq_len,
                   int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale, int32_t win, int64_t ld,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dout || !q || !k || !v || !out || !lse || !cu_seqlens || !dq || !dk || !dv) return PE_ERR_NULL;
  const pe_status s =
      check_attn_args(num_seqs, total_tokens, max_seq_len, num_heads, head_dim, dtype, softmax_scale);
  if (s != PE_OK) return s;
  for (const void* p : {dout, q, k, v, out, static_cast<const void*>(lse), static_cast<const void*>(cu_seqlens),
                        static_cast<const void*>(dq), static_cast<const void*>(dk), static_cast<const void*>(dv),
                        static_cast<const void*>(workspace)})
    if (p && !aligned16(p)) return PE_ERR_ARG;
  if (!workspace || workspace_bytes < pe_attn_workspace_size(num_seqs, total_tokens, num_heads, head_dim, dtype, 1))
    return PE_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  if (const pe_status c = check_cu(cu_seqlens, num_seqs, total_tokens, max_seq_len, st); c != PE_OK) return c;
  int32_t* items = static_cast<int32_t*>(workspace);
  const size_t ib = items_bytes(num_seqs, total_tokens);
  int32_t* items32 = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + ib);
  float* delta = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * ib);
  if (pe::attn_bwd_short_supported(dtype, head_dim, max_seq_len, ld, num_heads))
    return hip_status(pe::launch_attn_bwd_short(dtype, head_dim, dout, q, k, v, out, lse, cu_seqlens, num_seqs,
                                                static_cast<int32_t>(total_tokens), num_heads, max_seq_len, win, ld,
                                                softmax_scale, dq, dk, dv, st));
  if (pe::attn_bwd_seq_supported(dtype, head_dim, win, total_tokens, num_heads, ld)) {
    float* nd = reinterpret_cast<float*>(reinterpret_cast<char*>(delta) +
                                         round_up(static_cast<size_t>(total_tokens) * num_heads * sizeof(float)));
    hipError_t e = pe::launch_seq_worklist(cu_seqlens, num_seqs, total_tokens, pe::kAttnTileRows, items, st);
    if (e != hipSuccess) return PE_ERR_HIP;
    return hip_status(pe::launch_attn_bwd_seq(dtype, head_dim, dout, q, k, v, out, lse, cu_seqlens, items, num_seqs,
                                              static_cast<int32_t>(total_tokens), num_heads, win, ld, softmax_scale,
                                              dq, dk, dv, delta, nd, st));
  }
  // the fp32 one-wave kernels take the sequence-aligned list, every other kernel the 128-row one
  const bool wave = dtype == PE_FP32 && pe::attn_f32_wave_supported(head_dim, ld, num_heads);
  // fp32 global attention with a workspace of pe_attn_bwd_workspace_size: the dK/dV pass hands
  // its dS blocks to the dQ pass through the rest of the workspace
  float* ds = nullptr;
  if (wave && win < 0 && max_seq_len <= kDsMaxSeqLen) {
    const size_t base = pe_attn_workspace_size(num_seqs, total_tokens, num_heads, head_dim, dtype, 1);
    if (workspace_bytes >= base + ds_bytes(num_seqs, total_tokens, max_seq_len, num_heads))
      ds = reinterpret_cast<float*>(static_cast<char*>(workspace) + base);
  }
  hipError_t e = wave ? pe::launch_seq_worklist(cu_seqlens, num_seqs, total_tokens, pe::kAttnWaveRows, items32, st)
                      : pe::launch_worklist(cu_seqlens, num_seqs, total_tokens, pe::kAttnTileRows, items, st);
  if (e != hipSuccess) return PE_ERR_HIP;
  e = pe::launch_attn_bwd(dtype, head_dim, dout, q, k, v, out, lse, cu_seqlens, wave ? nullptr : items,
                          wave ? items32 : nullptr, num_seqs, static_cast<int32_t>(total_tokens), num_heads, win, ld,
                          softmax_scale, dq, dk, dv, delta, ds, nb_max(max_seq_len), st);
  if (e == hipErrorNotSupported) return PE_ERR_UNSUPPORTED;
  return hip_status(e);
}

}  // namespace

extern "C" {

pe_status pe_varlen_attn_bwd(const void* dout, const void* q, const void* k, const void* v, const void* out,
                             const float* lse, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                             int32_t max_seq_len, int32_t num_heads, int32_t head_dim, pe_dtype dtype,
                             float softmax_scale, void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return bwd_impl(dout, q, k, v, out, lse, cu_seqlens, num_seqs, total_tokens, max_seq_len, num_heads, head_dim,
                  dtype, softmax_scale, -1, dense_ld(num_heads, head_dim), dq, dk, dv, workspace, workspace_bytes,
                  stream);
}

pe_status pe_varlen_attn_bwd_local(const void* dout, const void* q, const void* k, const void* v, const void* out,
                                   const float* lse, const int32_t* cu_seqlens, int32_t num_seqs,
                                   int64_t total_tokens, int32_t max_seq_len, int32_t num_heads, int32_t head_dim,
                                   pe_dtype dtype, float softmax_scale, int32_t window, void* dq, void* dk, void* dv,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (window < 0) return PE_ERR_ARG;
  return bwd_impl(dout, q, k, v, out, lse, cu_seqlens, num_seqs, total_tokens, max_seq_len, num_heads, head_dim,
                  dtype, softmax_scale, effective_window(window, max_seq_len), dense_ld(num_heads, head_dim), dq, dk,
                  dv, workspace, workspace_bytes, stream);
}

pe_status pe_varlen_attn_fwd_qkv(const void* qkv, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                 int32_t max_seq_len, int32_t num_heads, int32_t head_dim, pe_dtype dtype,
                                 float softmax_scale, int32_t window, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!qkv) return PE_ERR_NULL;
  if (window < -1) return PE_ERR_ARG;
  const int64_t hd = dense_ld(num_heads, head_dim);
  const char* base = static_cast<const char*>(qkv);
  const size_t step = static_cast<size_t>(hd) * elem_bytes(dtype);
  return fwd_impl(base, base + step, base + 2 * step, cu_seqlens, num_seqs, total_tokens, max_seq_len, num_heads,
                  head_dim, dtype, softmax_scale, window < 0 ? -1 : effective_window(window, max_seq_len), 3 * hd,
                  out, lse, workspace, workspace_bytes, stream);
}

pe_status pe_varlen_attn_bwd_qkv(const void* dout, const void* qkv, const void* out, const float* lse,
                                 const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                 int32_t max_seq_len, int32_t num_heads, int32_t head_dim, pe_dtype dtype,
                                 float softmax_scale, int32_t window, void* dqkv, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!qkv || !dqkv) return PE_ERR_NULL;
  if (window < -1) return PE_ERR_ARG;
  const int64_t hd = dense_ld(num_heads, head_dim);
  const char* base = static_cast<const char*>(qkv);
  char* dbase = static_cast<char*>(dqkv);
  const size_t step = static_cast<size_t>(hd) * elem_bytes(dtype);
  return bwd_impl(dout, base, base + step, base + 2 * step, out, lse, cu_seqlens, num_seqs, total_tokens,
                  max_seq_len, num_heads, head_dim, dtype, softmax_scale,
                  window < 0 ? -1 : effective_window(window, max_seq_len), 3 * hd, dbase, dbase + step,
                  dbase + 2 * step, workspace, workspace_bytes, stream);
}

pe_status pe_position_ids(const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                          int64_t* position_ids, int32_t* document_ids, void* stream) {
  if (!cu_seqlens) return PE_ERR_NULL;
  if (num_seqs < 1 || total_tokens < 0 || total_tokens > INT32_MAX) return PE_ERR_ARG;
  for (const void* p : {static_cast<const void*>(cu_seqlens), static_cast<const void*>(position_ids),
                        static_cast<const void*>(document_ids)})
    if (p && !aligned16(p)) return PE_ERR_ARG;
  if (!position_ids && !document_ids) return PE_OK;
  return hip_status(pe::launch_ids(cu_seqlens, num_seqs, total_tokens, position_ids, document_ids, as_stream(stream)));
}

size_t pe_flatten_workspace_size(int32_t rows) { return rows < 1 ? 0 : pe::flatten_workspace_bytes(rows); }

}  // extern "C"

namespace {

pe_status flatten_impl(int form, const int32_t* a, const int32_t* cl, int32_t rows, int32_t width, int32_t ld,
                       int64_t* flat_index, int32_t* cu_seqlens, int64_t capacity, int64_t doc_capacity,
                       int64_t* h_total_tokens, int64_t* h_num_docs, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!a || (form == 0 && !cl) || !cu_seqlens || !h_total_tokens || !h_num_docs) return PE_ERR_NULL;
  if (rows < 1 || width < 1 || ld < 1 || capacity < 0 || doc_capacity < 0) return PE_ERR_ARG;
  if (static_cast<int64_t>(rows) * width > INT32_MAX) return PE_ERR_ARG;
  for (const void* p : {static_cast<const void*>(a), static_cast<const void*>(cl),
                        static_cast<const void*>(flat_index), static_cast<const void*>(cu_seqlens),
                        static_cast<const void*>(workspace)})
    if (p && !aligned16(p)) return PE_ERR_ARG;
  if (!workspace || workspace_bytes < pe_flatten_workspace_size(rows)) return PE_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  hipError_t e = pe::launch_flatten_counts(form, a, cl, rows, width, ld, workspace, st);
  if (e != hipSuccess) return PE_ERR_HIP;
  int64_t host[3] = {0, 0, 0};  // tokens, documents, error flag: the one host read
  e = hipMemcpyAsync(host, workspace, sizeof(host), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return PE_ERR_HIP;
  *h_total_tokens = host[0];
  *h_num_docs = host[1];
  if (host[2] != 0) return PE_ERR_METADATA;
  if (host[0] > capacity || host[1] > doc_capacity) return PE_ERR_CAPACITY;
  return hip_status(pe::launch_flatten_write(form, a, cl, rows, width, ld, workspace, flat_index, cu_seqlens, st));
}

}  // namespace

extern "C" {

pe_status pe_flatten_packed_metadata(const int32_t* token_index, const int32_t* cu_local, int32_t rows, int32_t width,
                                     int32_t max_docs, int64_t* flat_index, int32_t* cu_seqlens, int64_t capacity,
                                     int64_t doc_capacity, int64_t* h_total_tokens, int64_t* h_num_docs,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (max_docs < 0) return PE_ERR_ARG;
  return flatten_impl(0, token_index, cu_local, rows, width, max_docs + 1, flat_index, cu_seqlens, capacity,
                      doc_capacity, h_total_tokens, h_num_docs, workspace, workspace_bytes, stream);
}

pe_status pe_flatten_document_mask(const int32_t* document_mask, int32_t rows, int32_t width, int64_t* flat_index,
                                   int32_t* cu_seqlens, int64_t capacity, int64_t doc_capacity,
                                   int64_t* h_total_tokens, int64_t* h_num_docs, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return flatten_impl(1, document_mask, nullptr, rows, width, 1, flat_index, cu_seqlens, capacity, doc_capacity,
                      h_total_tokens, h_num_docs, workspace, workspace_bytes, stream);
}

pe_status pe_gather_rows(const void* src, int64_t src_rows, const int64_t* flat_index, int64_t n, int64_t row_elems,
                         pe_dtype dtype, void* dst, void* stream) {
  if (!src || !flat_index || !dst) return PE_ERR_NULL;
  if (src_rows < 0 || n < 0 || row_elems < 1) return PE_ERR_ARG;
  if (!valid_dtype(dtype)) return PE_ERR_UNSUPPORTED;
  return hip_status(pe::launch_gather_rows(src, src_rows, flat_index, n, row_elems * elem_bytes(dtype), dst,
                                           as_stream(stream)));
}

pe_status pe_scatter_rows(const void* src, const int64_t* flat_index, int64_t n, int64_t row_elems, pe_dtype dtype,
                          void* dst, int64_t dst_rows, void* stream) {
  if (!src || !flat_index || !dst) return PE_ERR_NULL;
  if (dst_rows < 0 || n < 0 || row_elems < 1) return PE_ERR_ARG;
  if (!valid_dtype(dtype)) return PE_ERR_UNSUPPORTED;
  return hip_status(pe::launch_scatter_rows(src, flat_index, n, row_elems * elem_bytes(dtype), dst, dst_rows,
                                            as_stream(stream)));
}

}  // extern "C"

// ------------------------------------------------------- pack without host read

extern "C" {

pe_status pe_pack_async(const int32_t* lengths, int32_t num_seqs, int32_t max_seq_len, const void* grid,
                        int64_t row_elems, pe_dtype dtype, int32_t* cu_seqlens, int64_t* flat_index, void* packed,
                        int64_t capacity, int64_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  if (!lengths || !cu_seqlens || !status) return PE_ERR_NULL;
  if (grid && !packed) return PE_ERR_NULL;
  if (!grid && packed) return PE_ERR_ARG;
  if (num_seqs < 1 || max_seq_len < 1 || capacity < 0) return PE_ERR_ARG;
  if (static_cast<int64_t>(num_seqs) * max_seq_len > INT32_MAX) return PE_ERR_ARG;
  if (!valid_dtype(dtype)) return PE_ERR_UNSUPPORTED;
  if (grid && row_elems < 1) return PE_ERR_ARG;
  for (const void* p : {static_cast<const void*>(lengths), static_cast<const void*>(cu_seqlens),
                        static_cast<const void*>(flat_index), grid, static_cast<const void*>(packed),
                        static_cast<const void*>(status), static_cast<const void*>(workspace)})
    if (p && !aligned16(p)) return PE_ERR_ARG;
  if (!workspace || workspace_bytes < pe_pack_workspace_size(num_seqs, max_seq_len, row_elems, dtype))
    return PE_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  // no valid batch holds more than num_seqs * max_seq_len rows
  const int64_t cap = std::min(capacity, static_cast<int64_t>(num_seqs) * max_seq_len);
  hipError_t e = pe::launch_scan(lengths, num_seqs, max_seq_len, cap, cu_seqlens, status,
                                 scan_part(workspace, num_seqs, max_seq_len, row_elems, dtype), st);
  if (e != hipSuccess) return PE_ERR_HIP;
  if ((!flat_index && !packed) || cap == 0) return PE_OK;
  int32_t* items = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + kAlign);
  const int64_t rowbytes = (packed ? row_elems : 1) * elem_bytes(dtype);
  const int32_t R = pe::pack_tile_rows(packed ? rowbytes : 64);
  e = pe::launch_worklist(cu_seqlens, num_seqs, cap, R, items, st);
  if (e != hipSuccess) return PE_ERR_HIP;
  return hip_status(pe::launch_pack_rows(grid, packed, flat_index, cu_seqlens, items, num_seqs, max_seq_len,
                                         rowbytes, cap, R, st));
}

// ----------------------------------------------------- captured bucket forward

struct pe_graph_s {
  hipGraphExec_t exec;
};

namespace {

// Work-list entries the single-workgroup plan kernel writes for a bucket; above
// kPlanMaxEntries the separate multi-block kernels are faster than one workgroup
// (measured per replay: 2-3 us gained up to ~8k entries, even at ~16k, 4.5 us lost at ~33k).
constexpr int64_t kPlanMaxEntries = 1 << 14;
int64_t plan_entries(int32_t num_seqs, int64_t cap, int64_t rowbytes, bool wave, bool w64) {
  const int64_t np = std::max(ceil_div(cap, pe::pack_tile_rows(rowbytes)), static_cast<int64_t>(num_seqs));
  const int64_t na = wave  ? cap / pe::kAttnWaveRows + num_seqs
                     : w64 ? cap / pe::kAttnTileRows + num_seqs
                           : std::max(ceil_div(cap, pe::kAttnTileRows), static_cast<int64_t>(num_seqs));
  return np + na;
}

}  // namespace

size_t pe_forward_graph_workspace_size(int32_t num_seqs, int32_t max_seq_len, int32_t num_heads, int32_t head_dim,
                                       pe_dtype dtype) {
  if (num_seqs < 1 || max_seq_len < 1 || num_heads < 1 || head_dim < 1) return 0;
  const int64_t cap = static_cast<int64_t>(num_seqs) * max_seq_len;
  return round_up(pe_pack_workspace_size(num_seqs, max_seq_len, 3 * dense_ld(num_heads, head_dim), dtype)) +
         pe_attn_workspace_size(num_seqs, cap, num_heads, head_dim, dtype, 0);
}

pe_status pe_forward_graph_create(const int32_t* lengths, int32_t num_seqs, int32_t max_seq_len, const void* qkv_grid,
                                  int32_t num_heads, int32_t head_dim, pe_dtype dtype, float softmax_scale,
                                  int32_t window, int32_t* cu_seqlens, void* qkv_packed, void* out_packed, float* lse,
                                  void* out_grid, int64_t* status, void* workspace, size_t workspace_bytes,
                                  pe_graph* graph) {
  if (!graph) return PE_ERR_NULL;
  *graph = nullptr;
  if (!lengths || !qkv_grid || !cu_seqlens || !qkv_packed || !out_packed || !out_grid || !status || !workspace)
    return PE_ERR_NULL;
  if (num_seqs < 1 || max_seq_len < 1 || window < -1) return PE_ERR_ARG;
  for (const void* p : {static_cast<const void*>(lengths), qkv_grid, static_cast<const void*>(cu_seqlens),
                        static_cast<const void*>(qkv_packed), static_cast<const void*>(out_packed),
                        static_cast<const void*>(lse), static_cast<const void*>(out_grid),
                        static_cast<const void*>(status), static_cast<const void*>(workspace)})
    if (p && !aligned16(p)) return PE_ERR_ARG;
  const int64_t cap = static_cast<int64_t>(num_seqs) * max_seq_len;
  const pe_status chk = check_attn_args(num_seqs, cap, max_seq_len, num_heads, head_dim, dtype, softmax_scale);
  if (chk != PE_OK) return chk;
  if (workspace_bytes < pe_forward_graph_workspace_size(num_seqs, max_seq_len, num_heads, head_dim, dtype))
    return PE_ERR_WORKSPACE;
  const int64_t hd = dense_ld(num_heads, head_dim);
  const size_t pack_ws = round_up(pe_pack_workspace_size(num_seqs, max_seq_len, 3 * hd, dtype));
  void* attn_ws = static_cast<char*>(workspace) + pack_ws;
  const size_t attn_wsb = workspace_bytes - pack_ws;

  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return PE_ERR_HIP;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return PE_ERR_HIP;
  }
  pe_status s = PE_OK;
  const pe::FwdList list = pe::attn_fwd_list(dtype, head_dim, max_seq_len, 3 * hd, num_heads);
  const bool wave = list == pe::kFwdListSeq32;
  const bool w64 = list == pe::kFwdListSeq128;
  const int64_t rowbytes = 3 * hd * elem_bytes(dtype);
  if (plan_entries(num_seqs, cap, rowbytes, wave, w64) <= kPlanMaxEntries) {
    // Four kernels: plan (scan + both work lists), pack, attention, unpack. The work lists sit
    // where pe_pack_async and the attention calls put them in the same workspace.
    const int32_t rp = pe::pack_tile_rows(rowbytes);
    int32_t* items_p = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + kAlign);
    int32_t* items_a = static_cast<int32_t*>(attn_ws);
    const char* base = static_cast<const char*>(qkv_packed);
    const size_t step = static_cast<size_t>(hd) * elem_bytes(dtype);
    const int32_t win = window < 0 ? -1 : effective_window(window, max_seq_len);
    const int32_t n = static_cast<int32_t>(cap);
    hipError_t e = pe::launch_plan(lengths, num_seqs, max_seq_len, cap, cu_seqlens, status, rp, items_p,
                                   wave ? pe::kAttnWaveRows : pe::kAttnTileRows, wave || w64, items_a, cs);
    if (e == hipSuccess)
      e = pe::launch_pack_rows(qkv_grid, qkv_packed, nullptr, cu_seqlens, items_p, num_seqs, max_seq_len, rowbytes,
                               cap, rp, cs);
    if (e == hipSuccess)
      e = pe::launch_attn_fwd(dtype, head_dim, base, base + step, base + 2 * step, cu_seqlens, items_a, num_seqs, n,
                              num_heads, max_seq_len, win, 3 * hd, softmax_scale, out_packed, lse, cs);
    if (e == hipSuccess)
      e = pe::launch_unpack_rows(out_packed, out_grid, cu_seqlens, num_seqs, max_seq_len, hd * elem_bytes(dtype), cs);
    s = hip_status(e);
  } else {
    s = pe_pack_async(lengths, num_seqs, max_seq_len, qkv_grid, 3 * hd, dtype, cu_seqlens, nullptr, qkv_packed, cap,
                      status, workspace, pack_ws, cs);
    if (s == PE_OK)
      s = pe_varlen_attn_fwd_qkv(qkv_packed, cu_seqlens, num_seqs, cap, max_seq_len, num_heads, head_dim, dtype,
                                 softmax_scale, window, out_packed, lse, attn_ws, attn_wsb, cs);
    if (s == PE_OK) s = pe_unpack(out_packed, cu_seqlens, num_seqs, max_seq_len, cap, hd, dtype, out_grid, cs);
  }
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(cs, &g);
  if (s == PE_OK && e != hipSuccess) s = PE_ERR_HIP;
  hipGraphExec_t exec = nullptr;
  if (s == PE_OK && hipGraphInstantiate(&exec, g, nullptr, nullptr, 0) != hipSuccess) s = PE_ERR_HIP;
  if (g) (void)hipGraphDestroy(g);
  (void)hipStreamDestroy(cs);
  if (s != PE_OK) return s;
  *graph = new pe_graph_s{exec};
  return PE_OK;
}

pe_status pe_graph_launch(pe_graph graph, void* stream) {
  if (!graph) return PE_ERR_NULL;
  return hip_status(hipGraphLaunch(graph->exec, as_stream(stream)));
}

pe_status pe_graph_destroy(pe_graph graph) {
  if (!graph) return PE_OK;
  const hipError_t e = hipGraphExecDestroy(graph->exec);
  delete graph;
  return hip_status(e);
}

}  // extern "C"
