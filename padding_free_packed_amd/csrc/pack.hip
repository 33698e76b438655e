// Packing kernels: lengths -> offsets (one workgroup scan), the tile work list,
// the row gather from the padded grid into the packed buffer (with flat_index),
// and the scatter back to the padded grid with zero fill.
//
// The gather of sequence b is one contiguous byte range in both buffers
// (grid rows b*S .. b*S+L_b-1 go to packed rows cu[b] .. cu[b+1]-1), so both
// copies are streams of contiguous segments. Work is split by bytes of the
// OUTPUT, evenly, so that one 8192-token document and many 30-token queries
// cost the same per byte.
#include "common.h"
#include "kernels.h"

namespace pe {

// ---------------------------------------------------------------- scan
// One workgroup of 1024 threads; each pass scans 32768 lengths, thread i taking
// the 32 consecutive lengths from 32 i (eight 16-byte loads, eight 16-byte stores
// of their exclusive prefixes), and carries the running total in int64. Writes
// cu[0..B], result[0] = total token count (int64), result[1] = 1 if any length
// lies outside [1, S], else 2 if cap >= 0 and the total exceeds cap, else 0. With
// cap >= 0 a nonzero result[1] also rewrites cu[0..B] as zeros, so that kernels
// queued behind the scan without a host check see no rows at all.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 32;

__device__ __forceinline__ void scan_lengths_block(const int32_t* __restrict__ lengths, int32_t B, int32_t S,
                                                   int64_t cap, int32_t* __restrict__ cu,
                                                   int64_t* __restrict__ result) {
  __shared__ int64_t wsum[kScanThreads / 64];
  __shared__ int bad_any;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) bad_any = 0;
  int bad = 0;
  int64_t carry = 0;
  for (int64_t base = 0; base < B; base += kScanThreads * kScanPer) {
    const int64_t i0 = base + static_cast<int64_t>(tid) * kScanPer;
    const bool whole = i0 + kScanPer <= B;  // the thread's lengths all exist
    int32_t L[kScanPer];
    if (whole) {
#pragma unroll
      for (int v = 0; v < kScanPer / 4; ++v) {
        const int4 x = *reinterpret_cast<const int4*>(lengths + i0 + 4 * v);
        L[4 * v] = x.x; L[4 * v + 1] = x.y; L[4 * v + 2] = x.z; L[4 * v + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kScanPer; ++j) L[j] = i0 + j < B ? lengths[i0 + j] : 0;
    }
    int64_t local = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      if (i0 + j < B) bad |= (L[j] < 1) | (L[j] > S);
      local += L[j];
    }
    // inclusive scan of `local` across the wave
    int64_t incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t up = __shfl_up(incl, o);
      if (lane >= o) incl += up;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int64_t wprefix = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) {
      const int64_t s = wsum[w];
      if (w < wv) wprefix += s;
      total += s;
    }
    int64_t run = carry + wprefix + incl - local;  // rows before the thread's first sequence
    int32_t E[kScanPer];                            // exclusive prefixes = cu[i0 + j]
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      E[j] = static_cast<int32_t>(run);
      run += L[j];
    }
    if (whole) {
#pragma unroll
      for (int v = 0; v < kScanPer / 4; ++v)
        *reinterpret_cast<int4*>(cu + i0 + 4 * v) = make_int4(E[4 * v], E[4 * v + 1], E[4 * v + 2], E[4 * v + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < kScanPer; ++j)
        if (i0 + j < B) cu[i0 + j] = E[j];
    }
    carry += total;
    __syncthreads();  // wsum is rewritten by the next pass
  }
  if (bad) atomicOr(&bad_any, 1);
  __syncthreads();
  const int64_t code = bad_any ? 1 : (cap >= 0 && carry > cap ? 2 : 0);
  const bool clear = cap >= 0 && code != 0;
  if (tid == 0) {
    result[0] = carry;
    result[1] = code;
    if (!clear) cu[B] = static_cast<int32_t>(carry);
  }
  if (clear)
    for (int64_t i = tid; i <= B; i += kScanThreads) cu[i] = 0;
}

__global__ __launch_bounds__(kScanThreads) void scan_lengths_kernel(
    const int32_t* __restrict__ lengths, int32_t B, int32_t S, int64_t cap, int32_t* __restrict__ cu,
    int64_t* __restrict__ result) {
  scan_lengths_block(lengths, B, S, cap, cu, result);
}

// The same scan over many workgroups, for batches of at least kScanMbMin sequences, in two
// launches (no workgroup waits for another): the first writes each workgroup's length sum
// and length-error flag (part[2 g], part[2 g + 1]); the second has every workgroup add up
// the partials before its own (its offset), all of them (the total and the flags, so each
// knows whether the batch is rejected) and rescan its 4096 lengths into cu.
constexpr int kScanMbThreads = 256;
constexpr int kScanMbPer = 16;  // lengths per thread
constexpr int kScanMbRows = kScanMbThreads * kScanMbPer;
constexpr int32_t kScanMbMin = 8192;

// the lengths of one thread: [i0, i0 + kScanMbPer), zeros past B
__device__ __forceinline__ void scan_mb_load(const int32_t* __restrict__ lengths, int64_t i0, int32_t B,
                                             int32_t (&L)[kScanMbPer]) {
  if (i0 + kScanMbPer <= B) {
#pragma unroll
    for (int v = 0; v < kScanMbPer / 4; ++v) {
      const int4 x = *reinterpret_cast<const int4*>(lengths + i0 + 4 * v);
      L[4 * v] = x.x; L[4 * v + 1] = x.y; L[4 * v + 2] = x.z; L[4 * v + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kScanMbPer; ++j) L[j] = i0 + j < B ? lengths[i0 + j] : 0;
  }
}

// sum over the workgroup (every thread gets it)
__device__ __forceinline__ int64_t scan_mb_sum(int64_t x, int64_t* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  const int wv = threadIdx.x >> 6;
  __syncthreads();  // red may hold an earlier sum
  if ((threadIdx.x & 63) == 0) red[wv] = x;
  __syncthreads();
  int64_t t = 0;
#pragma unroll
  for (int w = 0; w < kScanMbThreads / 64; ++w) t += red[w];
  return t;
}

__global__ __launch_bounds__(kScanMbThreads) void scan_part_kernel(const int32_t* __restrict__ lengths, int32_t B,
                                                                   int32_t S, int64_t* __restrict__ part) {
  __shared__ int64_t red[kScanMbThreads / 64];
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kScanMbRows + threadIdx.x * kScanMbPer;
  int32_t L[kScanMbPer];
  scan_mb_load(lengths, i0, B, L);
  int64_t local = 0;
  int bad = 0;
#pragma unroll
  for (int j = 0; j < kScanMbPer; ++j) {
    if (i0 + j < B) bad |= (L[j] < 1) | (L[j] > S);
    local += L[j];
  }
  const int64_t sum = scan_mb_sum(local, red);
  const int64_t nbad = scan_mb_sum(bad, red);
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = sum;
    part[2 * blockIdx.x + 1] = nbad != 0;
  }
}

__global__ __launch_bounds__(kScanMbThreads) void scan_fin_kernel(const int32_t* __restrict__ lengths, int32_t B,
                                                                  int64_t cap, const int64_t* __restrict__ part,
                                                                  int32_t G, int32_t* __restrict__ cu,
                                                                  int64_t* __restrict__ result) {
  __shared__ int64_t red[kScanMbThreads / 64];
  __shared__ int64_t wsum[kScanMbThreads / 64];
  const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t pre = 0, tot = 0, bad = 0;
  for (int i = tid; i < G; i += kScanMbThreads) {
    const int64_t x = part[2 * i];
    if (i < g) pre += x;
    tot += x;
    bad |= part[2 * i + 1];
  }
  pre = scan_mb_sum(pre, red);
  tot = scan_mb_sum(tot, red);
  bad = scan_mb_sum(bad, red);
  const int64_t code = bad ? 1 : (cap >= 0 && tot > cap ? 2 : 0);
  const bool clear = cap >= 0 && code != 0;
  const int64_t i0 = static_cast<int64_t>(g) * kScanMbRows + tid * kScanMbPer;
  if (clear) {  // a rejected batch: every offset 0 (no rows for the kernels queued behind)
    for (int j = 0; j < kScanMbPer; ++j)
      if (i0 + j < B) cu[i0 + j] = 0;
  } else {
    int32_t L[kScanMbPer];
    scan_mb_load(lengths, i0, B, L);
    int64_t local = 0;
#pragma unroll
    for (int j = 0; j < kScanMbPer; ++j) local += L[j];
    int64_t incl = local;  // inclusive scan of `local` across the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t up = __shfl_up(incl, o);
      if (lane >= o) incl += up;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int64_t run = pre + incl - local;
#pragma unroll
    for (int w = 0; w < kScanMbThreads / 64; ++w)
      if (w < wv) run += wsum[w];
    int32_t E[kScanMbPer];
#pragma unroll
    for (int j = 0; j < kScanMbPer; ++j) {
      E[j] = static_cast<int32_t>(run);
      run += L[j];
    }
    if (i0 + kScanMbPer <= B) {
#pragma unroll
      for (int v = 0; v < kScanMbPer / 4; ++v)
        *reinterpret_cast<int4*>(cu + i0 + 4 * v) = make_int4(E[4 * v], E[4 * v + 1], E[4 * v + 2], E[4 * v + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < kScanMbPer; ++j)
        if (i0 + j < B) cu[i0 + j] = E[j];
    }
  }
  if (tid == 0 && g == G - 1) cu[B] = clear ? 0 : static_cast<int32_t>(tot);
  if (tid == 0 && g == 0) {
    result[0] = tot;
    result[1] = code;
  }
}

// ---------------------------------------------------------------- work list
// items[t] = b with cu[b] <= t*R < cu[b+1]; items[T] = B, T = ceil(N / R).
// Thread b writes the entries of the tiles that start inside sequence b. N may
// be a capacity above cu[B]: thread i then also marks tile i, if it starts at
// or after cu[B], with B (a tile of no sequence).
// cu_B = cu[B], read once by the caller.
__device__ __forceinline__ void worklist_entry(const int32_t* __restrict__ cu, int64_t cu_B, int32_t B, int64_t N,
                                               int32_t R, int32_t* __restrict__ items, int64_t i) {
  const int64_t T = (N + R - 1) / R;
  if (i == 0) items[T] = B;
  if (i < T && i >= (cu_B + R - 1) / R) items[i] = B;
  if (i >= B) return;
  const int64_t c0 = cu[i], c1 = cu[i + 1];
  int64_t t = (c0 + R - 1) / R;
  const int64_t tend = min((c1 + R - 1) / R, T);
  for (; t < tend; ++t) items[t] = static_cast<int32_t>(i);
}

__global__ void worklist_kernel(const int32_t* __restrict__ cu, int32_t B, int64_t N, int32_t R,
                                int32_t* __restrict__ items) {
  worklist_entry(cu, cu[B], B, N, R, items, static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
}

// ---------------------------------------------------------------- sequence-aligned work list
// Tiles of R rows that start at each sequence's first row, so no tile holds two
// sequences. Sequence b owns the slots [s_b, s_{b+1}) with s_b = cu[b]/R + b:
// its ceil(L_b/R) tiles fit there because floor(cu/R) + ceil(L/R) <= floor((cu + L)/R) + 1,
// so the slots need no prefix sum over tile counts, at the price of at most one
// empty slot per sequence. items[s] = b for every slot of sequence b (slot s holds
// tile s - s_b, empty when that tile starts at or past cu[b+1]); slots before s_0
// and from s_B to T = N/R + B are marked B; items[T] = B. One thread per slot or
// sequence, whichever is more.
// cu_0 = cu[0] and cu_B = cu[B], read once by the caller.
__device__ __forceinline__ void seq_worklist_entry(const int32_t* __restrict__ cu, int64_t cu_0, int64_t cu_B,
                                                   int32_t B, int64_t N, int32_t R, int32_t* __restrict__ items,
                                                   int64_t i) {
  const int64_t T = N / R + B;
  if (i == 0) items[T] = B;
  if (i < T && (i < cu_0 / R || i >= cu_B / R + B)) items[i] = B;
  if (i >= B) return;
  // clamped to [0, T): offsets outside [0, N] (a broken precondition) never write past the list
  const int64_t s0 = max(static_cast<int64_t>(cu[i]) / R + i, static_cast<int64_t>(0));
  const int64_t s1 = min(static_cast<int64_t>(cu[i + 1]) / R + i + 1, T);
  for (int64_t s = s0; s < s1; ++s) items[s] = static_cast<int32_t>(i);
}

__global__ void seq_worklist_kernel(const int32_t* __restrict__ cu, int32_t B, int64_t N, int32_t R,
                                    int32_t* __restrict__ items) {
  seq_worklist_entry(cu, cu[0], cu[B], B, N, R, items,
                     static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
}

// ---------------------------------------------------------------- plan (scan + both work lists)
// One workgroup: the scan above, then from the offsets it has just written the
// work list of the packing copy (tile height Rp over N rows) and that of the
// attention (tile height Ra; sequence-aligned when `aligned`). The three kernels
// of the pack -> attention path in one launch, for short batches whose captured
// replay is a chain of dependent launches.
__global__ __launch_bounds__(kScanThreads) void plan_kernel(
    const int32_t* __restrict__ lengths, int32_t B, int32_t S, int64_t N, int32_t* __restrict__ cu,
    int64_t* __restrict__ result, int32_t Rp, int32_t* __restrict__ items_p, int32_t Ra, int aligned,
    int32_t* __restrict__ items_a) {
  scan_lengths_block(lengths, B, S, N, cu, result);
  __syncthreads();  // the offsets this workgroup wrote are visible to all of it
  const int64_t cu_0 = cu[0], cu_B = cu[B];
  const int64_t np = max((N + Rp - 1) / Rp, static_cast<int64_t>(B));
  for (int64_t i = threadIdx.x; i < np; i += kScanThreads) worklist_entry(cu, cu_B, B, N, Rp, items_p, i);
  if (aligned) {
    const int64_t na = N / Ra + B;
    for (int64_t i = threadIdx.x; i < na; i += kScanThreads)
      seq_worklist_entry(cu, cu_0, cu_B, B, N, Ra, items_a, i);
  } else {
    const int64_t na = max((N + Ra - 1) / Ra, static_cast<int64_t>(B));
    for (int64_t i = threadIdx.x; i < na; i += kScanThreads) worklist_entry(cu, cu_B, B, N, Ra, items_a, i);
  }
}

// ---------------------------------------------------------------- segment copy
template <typename U>
__device__ __forceinline__ void copy_units(const U* __restrict__ src, U* __restrict__ dst, int64_t n) {
  int64_t i = threadIdx.x;
  constexpr int BS = 256;
  for (; i + 3 * BS < n; i += 4 * BS) {
    const U a = src[i], b = src[i + BS], c = src[i + 2 * BS], d = src[i + 3 * BS];
    st_nt(dst + i, a);
    st_nt(dst + i + BS, b);
    st_nt(dst + i + 2 * BS, c);
    st_nt(dst + i + 3 * BS, d);
  }
  for (; i < n; i += BS) st_nt(dst + i, src[i]);
}

template <typename U>
__device__ __forceinline__ void zero_units(U* __restrict__ dst, int64_t n) {
  U z;
  __builtin_memset(&z, 0, sizeof(U));
  for (int64_t i = threadIdx.x; i < n; i += 256) st_nt(dst + i, z);
}

// Block w packs rows [w*R, min((w+1)*R, N)) of the packed buffer. items[w] is
// the sequence of its first row (work list with tile height R).
template <typename U>
__global__ __launch_bounds__(256) void pack_rows_kernel(
    const char* __restrict__ grid, char* __restrict__ packed, int64_t* __restrict__ flat_index,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t S,
    int64_t rowbytes, int64_t N, int32_t R) {
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * R;
  const int64_t r1 = min(r0 + R, N);
  int b = items[blockIdx.x];
  while (b < B) {
    const int64_t c0 = cu[b], c1 = cu[b + 1];
    const int64_t s0 = max(c0, r0), s1 = min(c1, r1);
    if (s0 < s1) {
      if (flat_index) {
        const int64_t base = static_cast<int64_t>(b) * S - c0;
        for (int64_t r = s0 + threadIdx.x; r < s1; r += 256) flat_index[r] = base + r;
      }
      if (packed) {
        const char* src = grid + (static_cast<int64_t>(b) * S + (s0 - c0)) * rowbytes;
        char* dst = packed + s0 * rowbytes;
        copy_units(reinterpret_cast<const U*>(src), reinterpret_cast<U*>(dst),
                   (s1 - s0) * rowbytes / static_cast<int64_t>(sizeof(U)));
      }
    }
    if (c1 >= r1) break;
    ++b;
  }
}

// Block w writes grid rows [w*R, min((w+1)*R, B*S)).
template <typename U>
__global__ __launch_bounds__(256) void unpack_rows_kernel(
    const char* __restrict__ packed, char* __restrict__ grid, const int32_t* __restrict__ cu,
    int32_t B, int32_t S, int64_t rowbytes, int64_t R) {
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * R;
  const int64_t g1 = min(g0 + R, static_cast<int64_t>(B) * S);
  for (int64_t b = g0 / S; b < B && b * S < g1; ++b) {
    const int64_t base = b * S;
    const int64_t c0 = cu[b];
    const int64_t L = cu[b + 1] - c0;
    const int64_t t0 = max(g0 - base, int64_t(0)), t1 = min(g1 - base, static_cast<int64_t>(S));
    const int64_t tc = min(t1, L);
    constexpr int64_t us = sizeof(U);
    if (t0 < tc)
      copy_units(reinterpret_cast<const U*>(packed + (c0 + t0) * rowbytes),
                 reinterpret_cast<U*>(grid + (base + t0) * rowbytes), (tc - t0) * rowbytes / us);
    const int64_t tz = max(t0, L);
    if (tz < t1) zero_units(reinterpret_cast<U*>(grid + (base + tz) * rowbytes), (t1 - tz) * rowbytes / us);
  }
}

// ---------------------------------------------------------------- launchers

int64_t scan_scratch_bytes(int32_t B) {
  return B >= kScanMbMin ? 16 * ((static_cast<int64_t>(B) + kScanMbRows - 1) / kScanMbRows) : 0;
}

hipError_t launch_scan(const int32_t* lengths, int32_t B, int32_t S, int64_t cap, int32_t* cu, int64_t* result,
                       int64_t* part, hipStream_t stream) {
  hipEvent_t ev = timing_start(stream);
  if (B >= kScanMbMin && part != nullptr) {
    const int32_t G = static_cast<int32_t>((static_cast<int64_t>(B) + kScanMbRows - 1) / kScanMbRows);
    hipLaunchKernelGGL(scan_part_kernel, dim3(G), dim3(kScanMbThreads), 0, stream, lengths, B, S, part);
    hipLaunchKernelGGL(scan_fin_kernel, dim3(G), dim3(kScanMbThreads), 0, stream, lengths, B, cap, part, G, cu,
                       result);
  } else {
    hipLaunchKernelGGL(scan_lengths_kernel, dim3(1), dim3(kScanThreads), 0, stream, lengths, B, S, cap, cu, result);
  }
  timing_stop("scan", ev, stream);
  return hipGetLastError();
}

hipError_t launch_worklist(const int32_t* cu, int32_t B, int64_t N, int32_t R, int32_t* items,
                           hipStream_t stream) {
  const int threads = 256;
  const int64_t T = (N + R - 1) / R;
  const int64_t n = T > B ? T : static_cast<int64_t>(B);
  const int blocks = static_cast<int>((n + threads - 1) / threads);
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL(worklist_kernel, dim3(blocks), dim3(threads), 0, stream, cu, B, N, R, items);
  timing_stop("worklist", ev, stream);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* lengths, int32_t B, int32_t S, int64_t N, int32_t* cu, int64_t* result,
                       int32_t Rp, int32_t* items_p, int32_t Ra, bool aligned, int32_t* items_a, hipStream_t stream) {
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kScanThreads), 0, stream, lengths, B, S, N, cu, result, Rp, items_p,
                     Ra, aligned ? 1 : 0, items_a);
  timing_stop("plan", ev, stream);
  return hipGetLastError();
}

hipError_t launch_seq_worklist(const int32_t* cu, int32_t B, int64_t N, int32_t R, int32_t* items,
                               hipStream_t stream) {
  const int threads = 256;
  const int64_t T = N / R + B;
  const int blocks = static_cast<int>((T + threads - 1) / threads);  // T >= B
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL(seq_worklist_kernel, dim3(blocks), dim3(threads), 0, stream, cu, B, N, R, items);
  timing_stop("worklist", ev, stream);
  return hipGetLastError();
}

// Rows per copy block: about 8 KiB of output per block (the best of 2-128 KiB measured).
int32_t pack_tile_rows(int64_t rowbytes) {
  const int64_t r = (8 * 1024) / (rowbytes > 0 ? rowbytes : 1);
  return static_cast<int32_t>(r < 1 ? 1 : (r > (1 << 20) ? (1 << 20) : r));
}

static int unit_bytes(int64_t rowbytes, const void* a, const void* b) {
  const uintptr_t m = reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b);
  for (int u = 16; u > 1; u >>= 1)
    if (rowbytes % u == 0 && (m % u) == 0) return u;
  return 1;
}

template <typename U>
static void pack_rows_typed(const char* g, char* p, int64_t* flat_index, const int32_t* cu, const int32_t* items,
                            int32_t B, int32_t S, int64_t rowbytes, int64_t N, int32_t R, unsigned blocks,
                            hipStream_t stream) {
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL(pack_rows_kernel<U>, dim3(blocks), dim3(256), 0, stream, g, p, flat_index, cu, items, B, S,
                     rowbytes, N, R);
  timing_stop("pack_rows", ev, stream);
}

hipError_t launch_pack_rows(const void* grid, void* packed, int64_t* flat_index, const int32_t* cu,
                            const int32_t* items, int32_t B, int32_t S, int64_t rowbytes, int64_t N,
                            int32_t R, hipStream_t stream) {
  const int64_t blocks = (N + R - 1) / R;
  if (blocks == 0) return hipSuccess;
  const char* g = static_cast<const char*>(grid);
  char* p = static_cast<char*>(packed);
  const int u = packed ? unit_bytes(rowbytes, grid, packed) : 16;
  const unsigned nb = static_cast<unsigned>(blocks);
  switch (u) {
    case 16: pack_rows_typed<uint4>(g, p, flat_index, cu, items, B, S, rowbytes, N, R, nb, stream); break;
    case 8: pack_rows_typed<uint2>(g, p, flat_index, cu, items, B, S, rowbytes, N, R, nb, stream); break;
    case 4: pack_rows_typed<uint32_t>(g, p, flat_index, cu, items, B, S, rowbytes, N, R, nb, stream); break;
    case 2: pack_rows_typed<uint16_t>(g, p, flat_index, cu, items, B, S, rowbytes, N, R, nb, stream); break;
    default: pack_rows_typed<uint8_t>(g, p, flat_index, cu, items, B, S, rowbytes, N, R, nb, stream); break;
  }
  return hipGetLastError();
}

template <typename U>
static void unpack_rows_typed(const char* p, char* g, const int32_t* cu, int32_t B, int32_t S, int64_t rowbytes,
                              int64_t R, unsigned blocks, hipStream_t stream) {
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL(unpack_rows_kernel<U>, dim3(blocks), dim3(256), 0, stream, p, g, cu, B, S, rowbytes, R);
  timing_stop("unpack_rows", ev, stream);
}

hipError_t launch_unpack_rows(const void* packed, void* grid, const int32_t* cu, int32_t B, int32_t S,
                              int64_t rowbytes, hipStream_t stream) {
  const int64_t R = pack_tile_rows(rowbytes);
  const int64_t rows = static_cast<int64_t>(B) * S;
  const int64_t blocks = (rows + R - 1) / R;
  if (blocks == 0) return hipSuccess;
  const char* p = static_cast<const char*>(packed);
  char* g = static_cast<char*>(grid);
  const int u = unit_bytes(rowbytes, packed, grid);
  const unsigned nb = static_cast<unsigned>(blocks);
  switch (u) {
    case 16: unpack_rows_typed<uint4>(p, g, cu, B, S, rowbytes, R, nb, stream); break;
    case 8: unpack_rows_typed<uint2>(p, g, cu, B, S, rowbytes, R, nb, stream); break;
    case 4: unpack_rows_typed<uint32_t>(p, g, cu, B, S, rowbytes, R, nb, stream); break;
    case 2: unpack_rows_typed<uint16_t>(p, g, cu, B, S, rowbytes, R, nb, stream); break;
    default: unpack_rows_typed<uint8_t>(p, g, cu, B, S, rowbytes, R, nb, stream); break;
  }
  return hipGetLastError();
}

}  // namespace pe
