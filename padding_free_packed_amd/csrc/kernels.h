// Internal launch functions of the HIP kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pe {

// Per-kernel timing hooks (no-ops unless pe_timing_enable(1) was called).
hipEvent_t timing_start(hipStream_t stream);
void timing_stop(const char* name, hipEvent_t start, hipStream_t stream);

// element type codes of the attention launchers (the pe_dtype values)
constexpr int kDtF32 = 0;
constexpr int kDtBF16 = 1;
constexpr int kDtF16 = 2;

// Every head dim the attention kernels are built for: the multiples of 8 up to 128.
#define PE_HEAD_DIMS(X) \
  X(8) X(16) X(24) X(32) X(40) X(48) X(56) X(64) X(72) X(80) X(88) X(96) X(104) X(112) X(120) X(128)
constexpr bool head_dim_supported(int d) { return d >= 8 && d <= 128 && d % 8 == 0; }

// packed query (or key) rows per attention work item
constexpr int kAttnTileRows = 128;
// packed rows per work item of the one-wave fp32 kernels
constexpr int kAttnWaveRows = 32;

// cap < 0: no capacity check, cu keeps the running sum even on a length error;
// cap >= 0: a length error or a total above cap zeroes cu (see scan_lengths_kernel).
// part: scan_scratch_bytes(B) bytes of device scratch (16-byte aligned) for the
// multi-workgroup scan of large batches; nullptr (or a small batch) takes one workgroup.
int64_t scan_scratch_bytes(int32_t B);
hipError_t launch_scan(const int32_t* lengths, int32_t B, int32_t S, int64_t cap, int32_t* cu, int64_t* result,
                       int64_t* part, hipStream_t stream);
// N may exceed cu[B] (a capacity): tiles from ceil(cu[B] / R) on get item B
hipError_t launch_worklist(const int32_t* cu, int32_t B, int64_t N, int32_t R, int32_t* items,
                           hipStream_t stream);
// Tiles of R rows aligned to each sequence's first row: N / R + B slots, items[N / R + B] = B
// (see seq_worklist_kernel for the slot layout)
hipError_t launch_seq_worklist(const int32_t* cu, int32_t B, int64_t N, int32_t R, int32_t* items,
                               hipStream_t stream);
// One workgroup: launch_scan (with cap = N) followed by launch_worklist(cu, B, N, Rp, items_p) and
// the attention list of tile height Ra (launch_seq_worklist if aligned, else launch_worklist).
hipError_t launch_plan(const int32_t* lengths, int32_t B, int32_t S, int64_t N, int32_t* cu, int64_t* result,
                       int32_t Rp, int32_t* items_p, int32_t Ra, bool aligned, int32_t* items_a, hipStream_t stream);
int32_t pack_tile_rows(int64_t rowbytes);
hipError_t launch_pack_rows(const void* grid, void* packed, int64_t* flat_index, const int32_t* cu,
                            const int32_t* items, int32_t B, int32_t S, int64_t rowbytes, int64_t N,
                            int32_t R, hipStream_t stream);
hipError_t launch_unpack_rows(const void* packed, void* grid, const int32_t* cu, int32_t B, int32_t S,
                              int64_t rowbytes, hipStream_t stream);

// The work list a forward reads, decided from host-visible arguments only. The
// entry points build the list this names, and launch_attn_fwd picks its kernel
// from the same answer, so list and kernel cannot disagree:
//   kFwdListPacked128: tiles of kAttnTileRows consecutive packed rows (launch_worklist);
//   kFwdListSeq128:    sequence-aligned tiles of kAttnTileRows rows (launch_seq_worklist),
//                      the 16-bit kernel of attn_fwd_w64b.hip;
//   kFwdListSeq32:     sequence-aligned tiles of kAttnWaveRows rows, the fp32 one-wave kernel;
//   kFwdListNone:      no list, the 16-bit short-sequence kernel (one wave per sequence and head).
enum FwdList { kFwdListPacked128 = 0, kFwdListSeq128 = 1, kFwdListSeq32 = 2, kFwdListNone = 3 };
FwdList attn_fwd_list(int dt, int D, int max_seq_len, int64_t ld, int32_t H);
// The forward of every entry point; items is the list attn_fwd_list names for the same
// arguments. dt: kDtF32, kDtBF16 or kDtF16 (every attention launcher takes it).
hipError_t launch_attn_fwd(int dt, int D, const void* q, const void* k, const void* v,
                           const int32_t* cu, const int32_t* items, int32_t B, int32_t N, int32_t H,
                           int32_t max_seq_len, int32_t win, int64_t ld, float scale, void* out, float* lse,
                           hipStream_t stream);

// 16-bit forward for lengths up to 64 at head dims 32 and 64: one wave per (sequence,
// head), K and Q rows loaded as operands, V by LDS DMA; global or windowed attention.
bool attn_fwd_short_supported(int dt, int D, int max_seq_len);
hipError_t launch_attn_fwd_short(bool f16, int D, const void* q, const void* k, const void* v, const int32_t* cu,
                                 int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* out,
                                 float* lse, hipStream_t stream);
// 16-bit forward with LDS-DMA staging (head dims 32, 64, 128); f16 selects fp16 over bf16.
bool attn_fwd_bf16_supported(int D, int max_seq_len);
// global or windowed attention over sequence-aligned 128-row tiles (head dims 32, 64): four
// waves of 32 query rows at d = 64, two of 64 rows at d = 32
bool attn_fwd_w64b_supported(int D);
hipError_t launch_attn_fwd_w64b(bool f16, int D, const void* q, const void* k, const void* v, const int32_t* cu,
                                const int32_t* items, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld,
                                float scale, void* out, float* lse, hipStream_t stream);
hipError_t launch_attn_fwd_bf16(bool f16, int D, const void* q, const void* k, const void* v, const int32_t* cu,
                                const int32_t* items, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld,
                                float scale, void* out, float* lse, hipStream_t stream);

// fp32 forward, one independent wave per 32 query rows of one sequence (head dims 32, 64);
// items32 is the sequence-aligned work list (launch_seq_worklist) with tile height kAttnWaveRows.
bool attn_f32_wave_supported(int D, int64_t ld, int32_t H);  // forward and backward alike
hipError_t launch_attn_fwd_f32_wave(int D, const void* q, const void* k, const void* v, const int32_t* cu,
                                    const int32_t* items32, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld,
                                    float scale, void* out, float* lse, hipStream_t stream);

// fp32 dK/dV and dQ, one independent wave per 32 key (query) rows of one sequence (head dims 32, 64;
// items32 as for the fp32 forward). With ds non-NULL (global attention only) the dK/dV pass also
// stores every 32x32 block of dS to ds, [H][T][nb_max][1024] floats (T = N/32 + B slots,
// nb_max >= the 32-row blocks of the longest sequence), for launch_bwd_dq_ds_f32_wave.
hipError_t launch_bwd_dkdv_f32_wave(int D, const void* dout, const void* q, const void* k, const void* v,
                                    const float* lse, const float* delta, const int32_t* cu, const int32_t* items32,
                                    int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* dk,
                                    void* dv, float* ds, int32_t nb_max, hipStream_t stream);
// dQ from the dS blocks of launch_bwd_dkdv_f32_wave (no recomputation of S and dP)
hipError_t launch_bwd_dq_ds_f32_wave(int D, const void* k, const float* ds, int32_t nb_max, const int32_t* cu,
                                     const int32_t* items32, int32_t B, int32_t N, int32_t H, int64_t ld, float scale,
                                     void* dq, hipStream_t stream);
// The dQ pass also computes D = rowsum(dO * O) (O dense [N, H, D]) and stores it to delta for
// the dK/dV pass, which therefore runs after it.
hipError_t launch_bwd_dq_f32_wave(int D, const void* dout, const void* q, const void* k, const void* v,
                                  const void* out, const float* lse, float* delta, const int32_t* cu,
                                  const int32_t* items32, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld,
                                  float scale, void* dq, hipStream_t stream);

// gather = 0: q_first is [B, H, D]; gather = 1: the query of sequence b is row cu[b] of a packed [N, H, D]
// max_seq_len (the host length bound) sets the key slots per block of both first-token kernels.
int first_token_slots(int max_seq_len);
hipError_t launch_attn_fwd_first(int dt, int D, const void* q_first, const void* k, const void* v,
                                 const int32_t* cu, int32_t B, int32_t N, int32_t H, int32_t max_seq_len,
                                 int32_t gather, int64_t ld, float scale, void* out_first, float* lse_first,
                                 hipStream_t stream);
// backward of the first-token readout: dq_first [B, H, D], dk and dv [N, H, D] (every row written)
hipError_t launch_attn_bwd_first(int dt, int D, const void* dout_first, const void* q_first, const void* k,
                                 const void* v, const void* out_first, const float* lse_first, const int32_t* cu,
                                 int32_t B, int32_t N, int32_t H, int32_t max_seq_len, int64_t ld, float scale,
                                 void* dq_first, void* dk, void* dv, hipStream_t stream);

// Backward: D = rowsum(dO * O) per (head, row), then dK/dV over key tiles, then dQ over query tiles.
// items32: the sequence-aligned list with kAttnWaveRows, given exactly when fp32 and
// attn_f32_wave_supported (the one-wave kernels run); otherwise NULL and items is the work
// list with tile height kAttnTileRows.
// win: local attention radius (keys with |i - j| <= win), or -1 for global attention;
// ld: elements between consecutive rows of Q, K, V (and of dQ, dK, dV): num_heads * D for
// separate [N, H, D] tensors, 3 * num_heads * D for a fused [N, 3, H, D] buffer. O, dO,
// LSE and D keep their own dense layouts. Every attention launcher takes both.
// ds, nb_max: the dS hand-off buffer of the fp32 one-wave path (launch_bwd_dkdv_f32_wave), or
// NULL; used for global attention only (then: delta pass, dK/dV storing dS, dQ from dS).
hipError_t launch_attn_bwd(int dt, int D, const void* dout, const void* q, const void* k,
                           const void* v, const void* out, const float* lse, const int32_t* cu,
                           const int32_t* items, const int32_t* items32, int32_t B, int32_t N, int32_t H,
                           int32_t win, int64_t ld, float scale, void* dq, void* dk, void* dv, float* delta,
                           float* ds, int32_t nb_max,
                           hipStream_t stream);

// The 16-bit backward of global or local attention over sequence-aligned tiles
// (attn_bwd_seq.hip): bf16 or fp16, head dims 32 and 64. items: the sequence-aligned list of kAttnTileRows
// rows (launch_seq_worklist); nl, nd: [H, N] floats each, nd after nl within 4 GiB of it
// (scratch of the call). Same layouts and ld as launch_attn_bwd.
bool attn_bwd_seq_supported(int dt, int D, int32_t win, int64_t N, int32_t H, int64_t ld);
hipError_t launch_attn_bwd_seq(int dt, int D, const void* dout, const void* q, const void* k, const void* v,
                               const void* out, const float* lse, const int32_t* cu, const int32_t* items, int32_t B,
                               int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* dq, void* dk, void* dv,
                               float* nl, float* nd, hipStream_t stream);

// The 16-bit backward for lengths up to 64 (attn_bwd_seq.hip): bf16 or fp16, head dims 32
// and 64, global or local; one workgroup of two waves per (sequence, head), dQ, dK and dV in one pass, no work
// list and no scratch. Same layouts and ld as launch_attn_bwd.
bool attn_bwd_short_supported(int dt, int D, int32_t max_seq_len, int64_t ld, int32_t H);
hipError_t launch_attn_bwd_short(int dt, int D, const void* dout, const void* q, const void* k, const void* v,
                                 const void* out, const float* lse, const int32_t* cu, int32_t B, int32_t N,
                                 int32_t H, int32_t max_seq_len, int32_t win, int64_t ld, float scale, void* dq,
                                 void* dk, void* dv, hipStream_t stream);

// checked mode (meta.hip): flag[0] = 1 if cu[0] != 0, a length is outside [1, S] or cu[B] > N
hipError_t launch_check_cu(const int32_t* cu, int32_t B, int64_t N, int32_t S, int32_t* flag, hipStream_t stream);

// packing metadata (meta.hip)
hipError_t launch_ids(const int32_t* cu, int32_t B, int64_t N, int64_t* pos, int32_t* doc, hipStream_t stream);
size_t flatten_workspace_bytes(int32_t rows);
// form 0: token_index + cu_local (ld = max_docs + 1); form 1: document mask. Writes the
// totals and the error flag to the first 24 bytes of ws (int64 x 3).
hipError_t launch_flatten_counts(int form, const int32_t* a, const int32_t* cl, int32_t rows, int32_t width,
                                 int32_t ld, void* ws, hipStream_t stream);
hipError_t launch_flatten_write(int form, const int32_t* a, const int32_t* cl, int32_t rows, int32_t width,
                                int32_t ld, const void* ws, int64_t* flat, int32_t* cu_out, hipStream_t stream);
hipError_t launch_gather_rows(const void* src, int64_t src_rows, const int64_t* flat, int64_t n, int64_t rowbytes,
                              void* dst, hipStream_t stream);
hipError_t launch_scatter_rows(const void* src, const int64_t* flat, int64_t n, int64_t rowbytes, void* dst,
                               int64_t dst_rows, hipStream_t stream);

}  // namespace pe
