// Packing metadata: per-token position and document ids from cu_seqlens, the
// flattening of NeMo's batch-major metadata (row-local token indices with
// row-local cumulative lengths, or an indexed document mask) into one packed
// token stream with global cu_seqlens, and row gather / scatter by flat index.
// Integer work; every kernel reads and writes each element once.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace pe {

// ---------------------------------------------------------------- checked mode
// One workgroup: flag[0] = 1 unless cu[0] == 0, every length cu[b+1] - cu[b] lies
// in [1, S] and cu[B] <= N (the contract the attention kernels assume), else 0.
// Reads cu[0..B] only; the flag is one vector store by thread 0.
__global__ __launch_bounds__(1024) void check_cu_kernel(const int32_t* __restrict__ cu, int32_t B, int64_t N,
                                                        int32_t S, int32_t* __restrict__ flag) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = (cu[0] != 0 || static_cast<int64_t>(cu[B]) > N) ? 1 : 0;
  __syncthreads();
  int mine = 0;
  for (int64_t i = threadIdx.x; i < B; i += blockDim.x) {
    const int32_t L = cu[i + 1] - cu[i];
    mine |= (L < 1) | (L > S);
  }
  if (mine) bad = 1;  // every writer stores the same value
  __syncthreads();
  if (threadIdx.x == 0) flag[0] = bad;
}

hipError_t launch_check_cu(const int32_t* cu, int32_t B, int64_t N, int32_t S, int32_t* flag, hipStream_t stream) {
  hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(1024), 0, stream, cu, B, N, S, flag);
  return hipGetLastError();
}


namespace {

// ---------------------------------------------------------------- position / document ids
__global__ __launch_bounds__(256) void ids_kernel(const int32_t* __restrict__ cu, int32_t B, int64_t N,
                                                  int64_t* __restrict__ pos, int32_t* __restrict__ doc) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (r >= N) return;
  int lo = 0, hi = B - 1;  // the sequence b with cu[b] <= r < cu[b+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= r) lo = mid; else hi = mid - 1;
  }
  if (pos) pos[r] = r - cu[lo];
  if (doc) doc[r] = lo + 1;
}

// ---------------------------------------------------------------- metadata flattening
// One wave per row. FORM 0: token_index [rows, width] + cu_local [rows, ld];
// FORM 1: an indexed document mask [rows, width] (ld unused).
constexpr int kFlatWave = 64;

template <int FORM>
__global__ __launch_bounds__(kFlatWave) void flatten_count_kernel(const int32_t* __restrict__ a,
                                                                  const int32_t* __restrict__ cl, int32_t rows,
                                                                  int32_t width, int32_t ld,
                                                                  int32_t* __restrict__ ntok,
                                                                  int32_t* __restrict__ ndoc,
                                                                  int32_t* __restrict__ bad) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int32_t* row = a + static_cast<int64_t>(r) * width;
  // the valid prefix: entries >= 0 (FORM 0) or > 0 (FORM 1)
  int first_pad = width;
  for (int t = lane; t < width; t += kFlatWave) {
    const int32_t x = row[t];
    if (FORM == 0 ? x < 0 : x <= 0) first_pad = min(first_pad, t);
  }
  const int n = wave_min_i(first_pad);
  int err = 0;
  for (int t = lane; t < width; t += kFlatWave) {
    const int32_t x = row[t];
    if (t >= n) {
      err |= FORM == 0 ? (x != -1) : (x != 0);
    } else if (FORM == 0) {
      err |= (x >= width) | (t + 1 < n && row[t + 1] <= x);
    } else {
      const int32_t prev = t == 0 ? 0 : row[t - 1];
      err |= (x != prev) & (x != prev + 1);
    }
  }
  int docs = 0;
  if (FORM == 0) {
    const int32_t* crow = cl + static_cast<int64_t>(r) * ld;
    int cfirst = ld;
    for (int i = lane; i < ld; i += kFlatWave)
      if (crow[i] < 0) cfirst = min(cfirst, i);
    const int m = wave_min_i(cfirst);
    for (int i = lane; i < ld; i += kFlatWave) {
      const int32_t x = crow[i];
      if (i >= m) err |= x != -1;
      else err |= (i == 0 && x != 0) | (i + 1 < m && crow[i + 1] <= x) | (i == m - 1 && x != n);
    }
    if (m == 0) err |= n != 0;
    docs = m > 0 ? m - 1 : 0;
  } else {
    docs = n > 0 ? row[n - 1] : 0;
  }
  err = wave_max_i(err);
  if (lane == 0) {
    ntok[r] = n;
    ndoc[r] = docs;
    if (err) atomicOr(bad, 1);
  }
}

// Exclusive scans of the per-row token and document counts (one block); writes
// the totals and the error flag to result[0..2].
constexpr int kFlatScan = 1024;

__global__ __launch_bounds__(kFlatScan) void flatten_scan_kernel(const int32_t* __restrict__ ntok,
                                                                 const int32_t* __restrict__ ndoc, int32_t rows,
                                                                 const int32_t* __restrict__ bad,
                                                                 int64_t* __restrict__ otok,
                                                                 int64_t* __restrict__ odoc,
                                                                 int64_t* __restrict__ result) {
  __shared__ int64_t wt[kFlatScan / 64], wd[kFlatScan / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t ct = 0, cd = 0;  // carries of the chunks before
  for (int base = 0; base < rows; base += kFlatScan) {
    const int i = base + tid;
    const int64_t xt = i < rows ? ntok[i] : 0, xd = i < rows ? ndoc[i] : 0;
    // inclusive scan within the wave
    int64_t st = xt, sd = xd;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t yt = __shfl_up(st, o), yd = __shfl_up(sd, o);
      if (lane >= o) {
        st += yt;
        sd += yd;
      }
    }
    if (lane == 63) {
      wt[wv] = st;
      wd[wv] = sd;
    }
    __syncthreads();
    int64_t pt = 0, pd = 0, tt = 0, td = 0;
    for (int w = 0; w < kFlatScan / 64; ++w) {
      if (w < wv) {
        pt += wt[w];
        pd += wd[w];
      }
      tt += wt[w];
      td += wd[w];
    }
    if (i < rows) {
      otok[i] = ct + pt + st - xt;
      odoc[i] = cd + pd + sd - xd;
    }
    ct += tt;
    cd += td;
    __syncthreads();
  }
  if (tid == 0) {
    result[0] = ct;
    result[1] = cd;
    result[2] = *bad;
  }
}

template <int FORM>
__global__ __launch_bounds__(kFlatWave) void flatten_write_kernel(const int32_t* __restrict__ a,
                                                                  const int32_t* __restrict__ cl, int32_t width,
                                                                  int32_t ld, const int32_t* __restrict__ ntok,
                                                                  const int32_t* __restrict__ ndoc,
                                                                  const int64_t* __restrict__ otok,
                                                                  const int64_t* __restrict__ odoc,
                                                                  int64_t* __restrict__ flat,
                                                                  int32_t* __restrict__ cu_out) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int32_t* row = a + static_cast<int64_t>(r) * width;
  const int n = ntok[r];
  const int64_t ot = otok[r], od = odoc[r];
  const int64_t rb = static_cast<int64_t>(r) * width;
  if (r == 0 && lane == 0) cu_out[0] = 0;
  for (int t = lane; t < n; t += kFlatWave) {
    if (flat) flat[ot + t] = rb + (FORM == 0 ? row[t] : t);
    if (FORM == 1 && (t == n - 1 || row[t + 1] != row[t]))  // the end of document row[t]
      cu_out[1 + od + row[t] - 1] = static_cast<int32_t>(ot + t + 1);
  }
  if (FORM == 0) {
    const int32_t* crow = cl + static_cast<int64_t>(r) * ld;
    for (int i = lane; i < ndoc[r]; i += kFlatWave) cu_out[1 + od + i] = static_cast<int32_t>(ot + crow[i + 1]);
  }
}

// ---------------------------------------------------------------- row gather / scatter
template <typename U>
__global__ __launch_bounds__(256) void gather_rows_kernel(const U* __restrict__ src, int64_t src_rows,
                                                          const int64_t* __restrict__ flat, int64_t n, int64_t upr,
                                                          U* __restrict__ dst) {
  const int64_t total = n * upr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = i / upr, u = i - row * upr;
    const int64_t s = flat[row];
    st_nt(dst + i, (s >= 0 && s < src_rows) ? src[s * upr + u] : U{});
  }
}

template <typename U>
__global__ __launch_bounds__(256) void fill_zero_kernel(U* __restrict__ dst, int64_t total) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256)
    st_nt(dst + i, U{});
}

template <typename U>
__global__ __launch_bounds__(256) void scatter_rows_kernel(const U* __restrict__ src,
                                                           const int64_t* __restrict__ flat, int64_t n, int64_t upr,
                                                           U* __restrict__ dst, int64_t dst_rows) {
  const int64_t total = n * upr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = i / upr, u = i - row * upr;
    const int64_t d = flat[row];
    if (d >= 0 && d < dst_rows) st_nt(dst + d * upr + u, src[i]);
  }
}

unsigned grid_for(int64_t total) {
  const int64_t want = (total + 255) / 256;
  return static_cast<unsigned>(want < 1 ? 1 : (want > 65536 ? 65536 : want));
}

template <typename U>
hipError_t gather_as(const void* src, int64_t src_rows, const int64_t* flat, int64_t n, int64_t rowbytes, void* dst,
                     hipStream_t stream) {
  const int64_t upr = rowbytes / static_cast<int64_t>(sizeof(U));
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL((gather_rows_kernel<U>), dim3(grid_for(n * upr)), dim3(256), 0, stream,
                     static_cast<const U*>(src), src_rows, flat, n, upr, static_cast<U*>(dst));
  timing_stop("gather_rows", ev, stream);
  return hipGetLastError();
}

template <typename U>
hipError_t scatter_as(const void* src, const int64_t* flat, int64_t n, int64_t rowbytes, void* dst, int64_t dst_rows,
                      hipStream_t stream) {
  const int64_t upr = rowbytes / static_cast<int64_t>(sizeof(U));
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL((fill_zero_kernel<U>), dim3(grid_for(dst_rows * upr)), dim3(256), 0, stream,
                     static_cast<U*>(dst), dst_rows * upr);
  hipLaunchKernelGGL((scatter_rows_kernel<U>), dim3(grid_for(n * upr)), dim3(256), 0, stream,
                     static_cast<const U*>(src), flat, n, upr, static_cast<U*>(dst), dst_rows);
  timing_stop("scatter_rows", ev, stream);
  return hipGetLastError();
}

int unit_for(const void* a, const void* b, int64_t rowbytes) {
  const uintptr_t m = reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) | static_cast<uintptr_t>(rowbytes);
  return (m & 15) == 0 ? 16 : (m & 7) == 0 ? 8 : (m & 3) == 0 ? 4 : 2;
}

}  // namespace

hipError_t launch_ids(const int32_t* cu, int32_t B, int64_t N, int64_t* pos, int32_t* doc, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL(ids_kernel, dim3(static_cast<unsigned>((N + 255) / 256)), dim3(256), 0, stream, cu, B, N, pos,
                     doc);
  timing_stop("ids", ev, stream);
  return hipGetLastError();
}

size_t flatten_workspace_bytes(int32_t rows) {
  const size_t r = static_cast<size_t>(rows < 0 ? 0 : rows);
  return 256 + ((r * 8 + 255) / 256) * 256 + ((r * 16 + 255) / 256) * 256;
}

hipError_t launch_flatten_counts(int form, const int32_t* a, const int32_t* cl, int32_t rows, int32_t width,
                                 int32_t ld, void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  int64_t* result = reinterpret_cast<int64_t*>(w);                 // [0..2] totals and flag, [3] error word
  int32_t* bad = reinterpret_cast<int32_t*>(w + 24);
  int32_t* ntok = reinterpret_cast<int32_t*>(w + 256);
  int32_t* ndoc = ntok + rows;
  int64_t* otok = reinterpret_cast<int64_t*>(w + 256 + ((static_cast<size_t>(rows) * 8 + 255) / 256) * 256);
  int64_t* odoc = otok + rows;
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL(fill_zero_kernel<int64_t>, dim3(1), dim3(256), 0, stream, result, int64_t(4));
  if (form == 0)
    hipLaunchKernelGGL(flatten_count_kernel<0>, dim3(static_cast<unsigned>(rows)), dim3(kFlatWave), 0, stream, a, cl,
                       rows, width, ld, ntok, ndoc, bad);
  else
    hipLaunchKernelGGL(flatten_count_kernel<1>, dim3(static_cast<unsigned>(rows)), dim3(kFlatWave), 0, stream, a, cl,
                       rows, width, ld, ntok, ndoc, bad);
  hipLaunchKernelGGL(flatten_scan_kernel, dim3(1), dim3(kFlatScan), 0, stream, ntok, ndoc, rows, bad, otok, odoc,
                     result);
  timing_stop("flatten_count", ev, stream);
  return hipGetLastError();
}

hipError_t launch_flatten_write(int form, const int32_t* a, const int32_t* cl, int32_t rows, int32_t width,
                                int32_t ld, const void* ws, int64_t* flat, int32_t* cu_out, hipStream_t stream) {
  const char* w = static_cast<const char*>(ws);
  const int32_t* ntok = reinterpret_cast<const int32_t*>(w + 256);
  const int32_t* ndoc = ntok + rows;
  const int64_t* otok =
      reinterpret_cast<const int64_t*>(w + 256 + ((static_cast<size_t>(rows) * 8 + 255) / 256) * 256);
  const int64_t* odoc = otok + rows;
  hipEvent_t ev = timing_start(stream);
  if (form == 0)
    hipLaunchKernelGGL(flatten_write_kernel<0>, dim3(static_cast<unsigned>(rows)), dim3(kFlatWave), 0, stream, a, cl,
                       width, ld, ntok, ndoc, otok, odoc, flat, cu_out);
  else
    hipLaunchKernelGGL(flatten_write_kernel<1>, dim3(static_cast<unsigned>(rows)), dim3(kFlatWave), 0, stream, a, cl,
                       width, ld, ntok, ndoc, otok, odoc, flat, cu_out);
  timing_stop("flatten_write", ev, stream);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, int64_t src_rows, const int64_t* flat, int64_t n, int64_t rowbytes,
                              void* dst, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  switch (unit_for(src, dst, rowbytes)) {
    case 16: return gather_as<uint4>(src, src_rows, flat, n, rowbytes, dst, stream);
    case 8: return gather_as<uint2>(src, src_rows, flat, n, rowbytes, dst, stream);
    case 4: return gather_as<uint32_t>(src, src_rows, flat, n, rowbytes, dst, stream);
    default: return gather_as<uint16_t>(src, src_rows, flat, n, rowbytes, dst, stream);
  }
}

hipError_t launch_scatter_rows(const void* src, const int64_t* flat, int64_t n, int64_t rowbytes, void* dst,
                               int64_t dst_rows, hipStream_t stream) {
  if (dst_rows == 0) return hipSuccess;
  switch (unit_for(src, dst, rowbytes)) {
    case 16: return scatter_as<uint4>(src, flat, n, rowbytes, dst, dst_rows, stream);
    case 8: return scatter_as<uint2>(src, flat, n, rowbytes, dst, dst_rows, stream);
    case 4: return scatter_as<uint32_t>(src, flat, n, rowbytes, dst, dst_rows, stream);
    default: return scatter_as<uint16_t>(src, flat, n, rowbytes, dst, dst_rows, stream);
  }
}

}  // namespace pe
