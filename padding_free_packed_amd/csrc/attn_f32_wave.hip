// fp32 attention kernels with one independent wave per 32 rows of one sequence: the
// forward, and the dQ and dK/dV passes of the backward. Tiles start at each
// sequence's first row (the sequence-aligned work list), so a wave's rows share one
// key range and the 32x32 products only overhang at a sequence's last tile; there
// the forward and the dK/dV pass skip the products of whole 8-row groups past the
// range (in the dQ pass that measured no faster).
//
// On fp32 the MFMA operands of every product are one element per lane per step, so
// the transposed operands load straight from global memory (L2-resident: neighbouring
// waves read the same sequences) and the waves share no LDS tile and no barrier: a
// wave whose rows cover short sequences never waits for one covering long ones. All
// block loads go through buffer resources bounded at the walk's end (rows past it
// read 0), with wave-uniform row offsets, so no lane computes addresses per load.
// The forward loads each step's operands one step ahead; the dQ and dK/dV passes load
// at use and rely on their second wave per SIMD to cover the latency (measured faster
// than prefetching with the registers that takes).
//
// Backward of global attention given the larger workspace: the dK/dV pass also stores
// every 32x32 dS block of a sequence, and a dQ pass computes dQ = dS K from those blocks
// (transposed through LDS) instead of recomputing S and dP; with a window or the smaller
// workspace the dQ pass recomputes them (and forms D = <dO, O> of its rows itself).
//
// fp32 forward, one wave per (head, 32 query rows), over its key span in 32-key steps:
//   S^T (32 keys x 32 queries) += K Q^T   v_mfma_f32_32x32x2f32, 32 steps of 2 over d=64
//   O^T (d x 32 queries)       += V^T P^T 16 steps per 32-row d block
#include <climits>

#include "attn_common.h"

namespace pe {

namespace {

constexpr int kRows = 32;  // query rows per wave

// Slot t of the sequence-aligned work list (tiles of kRows rows starting at each
// sequence's first row, sequence b in slots cu[b]/kRows + b onwards): rows
// [r0, rend) of sequence b = items[t], which spans rows [lo, hi). False for an
// empty slot (past a sequence's last tile, or past cu[B]).
struct SeqTile {
  int r0, rend, lo, hi;
};
__device__ __forceinline__ bool seq_tile(const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int t,
                                         int B, SeqTile& sp) {
  const int b = items[t];
  if (b >= B) return false;
  sp.lo = cu[b];
  sp.hi = cu[b + 1];
  sp.r0 = sp.lo + (t - (sp.lo / kRows + b)) * kRows;
  sp.rend = min(sp.r0 + kRows, sp.hi);
  return sp.r0 < sp.hi;
}

// The lane's index in the wave, computed where it is used: an opaque instruction, so the
// compiler neither hoists it out of a loop nor keeps it live in a register across one.
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Buffer resource over `rows` rows of `stride` floats from `base`: a load at a byte
// offset at or past rows * stride * 4 returns 0 and touches no memory, so rows past a
// block's end need neither clamping nor per-lane address arithmetic. rows <= 32 here,
// so the byte count fits the 32-bit record count for any row stride below 2^24.
constexpr int kBufferFlags = 0x00020000;  // dword 3 of a raw buffer resource on CDNA
constexpr int kNonTemporal = 2;           // cache policy operand of a buffer access: streamed
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const float* base, int rows, uint32_t stride) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0,
                                           static_cast<int>(static_cast<uint32_t>(rows) * stride * 4u), kBufferFlags);
}
__device__ __forceinline__ float buf_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), static_cast<int>(soff), 0));
}
__device__ __forceinline__ float4 buf_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff),
                                                                          static_cast<int>(soff), 0));
}

template <int D>
struct F32Ops {
  static constexpr int HALF = D / 2;  // head-dim elements per lane half (MFMA steps of S)
  static constexpr int DB = D / 32;   // 32-row blocks of O^T
  float k[HALF];                      // K[key][g*HALF + st], key = kb + lane%32
  float v[16][DB];                    // V[kb + 8(st/4) + 4g + st%4][db*32 + lane%32]
};

// The operands of one 32-key step, through buffer resources over rows
// [kb, min(kb + 32, kend)) of head h: rows past kend read 0 (kb < kend).
template <int D>
__device__ __forceinline__ void load_ops_buf(F32Ops<D>& ops, const float* __restrict__ kp,
                                             const float* __restrict__ vp, int kb, int kend, uint32_t LD,
                                             int64_t hoff, int ql, int g) {
  using O = F32Ops<D>;
  const int n = min(32, kend - kb);
  const int64_t off = static_cast<int64_t>(kb) * LD + hoff;
  const auto rk = rows_rsrc(kp + off, n, LD), rv = rows_rsrc(vp + off, n, LD);
  const uint32_t vrow = (static_cast<uint32_t>(ql) * LD + g * O::HALF) * 4u;
#pragma unroll
  for (int j = 0; j < O::HALF / 4; ++j) {
    const float4 x = buf_f32x4(rk, vrow + 16u * j, 0);
    ops.k[4 * j] = x.x, ops.k[4 * j + 1] = x.y, ops.k[4 * j + 2] = x.z, ops.k[4 * j + 3] = x.w;
  }
  const uint32_t vtr = (static_cast<uint32_t>(4 * g) * LD + ql) * 4u;
#pragma unroll
  for (int st = 0; st < 16; ++st)
#pragma unroll
    for (int db = 0; db < O::DB; ++db)
      ops.v[st][db] = buf_f32(rv, vtr + 128u * db, (8u * (st >> 2) + (st & 3)) * LD * 4u);
}

template <int D>
__global__ __launch_bounds__(64, 2) void attn_fwd_f32_kernel(
    const float* __restrict__ qp, const float* __restrict__ kp, const float* __restrict__ vp,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N, int32_t H, int32_t T,
    int32_t win, int64_t ld, float c, float* __restrict__ op, float* __restrict__ lse) {
  using O = F32Ops<D>;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lin / T, t = lin - h * T;
  const int lane = threadIdx.x, ql = lane & 31, g = lane >> 5;

  SeqTile sp;
  if (!seq_tile(cu, items, t, B, sp)) return;
  const int r0 = sp.r0;
  const int qrow = r0 + ql;
  const bool qvalid = qrow < sp.rend;
  int qk0 = 0, qk1 = 0;
  if (qvalid) {
    qk0 = sp.lo;
    qk1 = sp.hi;
    band_limit(qrow, win, qk0, qk1);
  }
  const int wk0 = __builtin_amdgcn_readfirstlane(wave_min_i(qvalid ? qk0 : INT_MAX));
  const int wk1 = __builtin_amdgcn_readfirstlane(wave_max_i(qvalid ? qk1 : INT_MIN));
  const int mk0 = __builtin_amdgcn_readfirstlane(wave_max_i(qvalid ? qk0 : INT_MIN));
  const int mk1 = __builtin_amdgcn_readfirstlane(wave_min_i(qvalid ? qk1 : INT_MAX));

  float qf[O::HALF];
  {
    const float4* src =
        reinterpret_cast<const float4*>(qp + static_cast<int64_t>(qvalid ? qrow : r0) * ld + h * D + g * O::HALF);
#pragma unroll
    for (int j = 0; j < O::HALF / 4; ++j) {
      const float4 x = src[j];
      qf[4 * j + 0] = qvalid ? x.x : 0.f;
      qf[4 * j + 1] = qvalid ? x.y : 0.f;
      qf[4 * j + 2] = qvalid ? x.z : 0.f;
      qf[4 * j + 3] = qvalid ? x.w : 0.f;
    }
  }

  floatx16 o[O::DB];
#pragma unroll
  for (int db = 0; db < O::DB; ++db) o[db] = floatx16{};
  float m = kNegBig, l = 0.f;

  auto block = [&](const O& ops, int kb) __attribute__((always_inline)) {
    floatx16 s = floatx16{};
#pragma unroll
    for (int st = 0; st < O::HALF; ++st) s = __builtin_amdgcn_mfma_f32_32x32x2f32(ops.k[st], qf[st], s, 0, 0, 0);
    if (!(kb >= mk0 && kb + 32 <= mk1)) {
      const int base = kb + 4 * g;
      mask_block(s, qk0 - base, qk1 - base);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = xhalf_max(mx);
    const float mnew = fmaxf(m, mx * c);
    if (__any(mnew > m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < O::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m = mnew;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m));
      s[i] = p;
      l += p;
    }
    // keys 8j .. 8j+7 of the block (steps 4j .. 4j+3) at or past wk1 have P = 0 for every
    // query of the wave: their products would add nothing, so they are skipped
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j > 0 && kb + 8 * j >= wk1) break;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int db = 0; db < O::DB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(ops.v[4 * j + e][db], s[4 * j + e], o[db], 0, 0, 0);
    }
  };

  // keys [wk0, wk1) in steps of 32; operands of the next step load while this one computes
  if (wk0 < wk1) {
    const int klast = wk1 - 1;
    O a, b;
    const uint32_t LDu = static_cast<uint32_t>(ld);
    const int64_t hoff = static_cast<int64_t>(h) * D;
    const int kl = wk0 + (klast - wk0) / 32 * 32;  // first row of the last block
    load_ops_buf<D>(a, kp, vp, wk0, wk1, LDu, hoff, ql, g);
    for (int kb = wk0; kb < wk1; kb += 64) {
      // Unconditional (a step past the end reloads the last block): a load under a branch
      // makes the wait counts at the join assume the worst path and wait for the younger
      // loads too. The empty asm keeps each load group where it is written.
      load_ops_buf<D>(b, kp, vp, min(kb + 32, kl), wk1, LDu, hoff, ql, g);
      asm volatile("" ::: "memory");
      block(a, kb);
      if (kb + 32 >= wk1) break;
      load_ops_buf<D>(a, kp, vp, min(kb + 64, kl), wk1, LDu, hoff, ql, g);
      asm volatile("" ::: "memory");
      block(b, kb + 32);
    }
  }

  const float lt = xhalf_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qvalid) {
    store_acc_row<float, D>(op, (static_cast<int64_t>(qrow) * H + h) * D, o, inv, g);
    if (lse != nullptr && g == 0) lse[static_cast<int64_t>(h) * N + qrow] = (m + log2f(lt)) * kLn2;
  }
}

template <int D>
hipError_t dispatch(const void* q, const void* k, const void* v, const int32_t* cu, const int32_t* items,
                    int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* out, float* lse,
                    hipStream_t stream) {
  const int T = N / kRows + B;  // slots of the sequence-aligned work list
  const int64_t blocks = static_cast<int64_t>(T) * H;
  if (blocks == 0) return hipSuccess;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D>), dim3(static_cast<unsigned>(blocks)), dim3(64), 0, stream,
                     static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v), cu,
                     items, B, N, H, T, win, ld, c, static_cast<float*>(out), lse);
  timing_stop("attn_fwd", ev, stream);
  return hipGetLastError();
}

}  // namespace

// Head dims 32 and 64; the buffer offsets are 32-bit, so row strides (ld, and H * D for
// O and dO) stay below 2^24 elements.
bool attn_f32_wave_supported(int D, int64_t ld, int32_t H) {
  return (D == 32 || D == 64) && ld < (int64_t{1} << 24) && static_cast<int64_t>(H) * D < (int64_t{1} << 24);
}

hipError_t launch_attn_fwd_f32_wave(int D, const void* q, const void* k, const void* v, const int32_t* cu,
                                    const int32_t* items32, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld,
                                    float scale, void* out, float* lse, hipStream_t stream) {
  switch (D) {
    case 32: return dispatch<32>(q, k, v, cu, items32, B, N, H, win, ld, scale, out, lse, stream);
    case 64: return dispatch<64>(q, k, v, cu, items32, B, N, H, win, ld, scale, out, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pe

// ---------------------------------------------------------------- fp32 dQ, one wave per 32 query rows
// Same walk as the forward: per 32-key step
//   S^T = K Q^T, dP^T = V dO^T          (K and V row chunks as A operands)
//   dS^T = P^T (dP^T - D), P^T = exp(scale S^T - lse)
//   dQ^T += K^T dS^T                    (K scalars K[key(st)][d] as A operands)
namespace pe {
namespace {

// Row loads relative to a wave-uniform base (row `r`, head h) with 32-bit
// element offsets, so one scalar base and one offset register serve many loads.
template <int D>
__device__ __forceinline__ void load_rows(float (&r)[D / 2], const float* __restrict__ base, uint32_t rel, uint32_t HD,
                                          int g) {
  const float4* src = reinterpret_cast<const float4*>(base + (rel * HD + static_cast<uint32_t>(g * (D / 2))));
#pragma unroll
  for (int j = 0; j < D / 8; ++j) {
    const float4 x = src[j];
    r[4 * j + 0] = x.x;
    r[4 * j + 1] = x.y;
    r[4 * j + 2] = x.z;
    r[4 * j + 3] = x.w;
  }
}

template <int D>
__global__ __launch_bounds__(64, 2) void bwd_dq_f32_kernel(
    const float* __restrict__ dop, const float* __restrict__ qp, const float* __restrict__ kp,
    const float* __restrict__ vp, const float* __restrict__ op, const float* __restrict__ lse,
    float* __restrict__ delta, const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B,
    int32_t N, int32_t H, int32_t T, int32_t win, int64_t ld, float c, float scale, float* __restrict__ dqp) {
  constexpr int HALF = D / 2, DB = D / 32;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lin / T, t = lin - h * T;
  const int lane = threadIdx.x, ql = lane & 31, g = lane >> 5;

  SeqTile sp;
  if (!seq_tile(cu, items, t, B, sp)) return;
  const int r0 = sp.r0;
  const int qrow = r0 + ql;
  const bool qvalid = qrow < sp.rend;
  int qk0 = 0, qk1 = 0;
  if (qvalid) {
    qk0 = sp.lo;
    qk1 = sp.hi;
    band_limit(qrow, win, qk0, qk1);
  }
  const int wk0 = __builtin_amdgcn_readfirstlane(wave_min_i(qvalid ? qk0 : INT_MAX));
  const int wk1 = __builtin_amdgcn_readfirstlane(wave_max_i(qvalid ? qk1 : INT_MIN));
  const int mk0 = __builtin_amdgcn_readfirstlane(wave_max_i(qvalid ? qk0 : INT_MIN));
  const int mk1 = __builtin_amdgcn_readfirstlane(wave_min_i(qvalid ? qk1 : INT_MAX));

  float qf[HALF], df[HALF];
  const int qsafe = qvalid ? qrow : r0;
  const uint32_t HD = static_cast<uint32_t>(H) * D;  // rows of dO
  const uint32_t LD = static_cast<uint32_t>(ld);     // rows of Q, K, V and dQ
  const int64_t hoff = static_cast<int64_t>(h) * D;
  auto at = [&](const float* p, int row, uint32_t stride) { return p + (static_cast<int64_t>(row) * stride + hoff); };
  load_rows<D>(qf, at(qp, r0, LD), qsafe - r0, LD, g);
  load_rows<D>(df, at(dop, r0, HD), qsafe - r0, HD, g);
  if (!qvalid) {
#pragma unroll
    for (int i = 0; i < HALF; ++i) qf[i] = df[i] = 0.f;
  }
  const float lse2 = qvalid ? lse[static_cast<int64_t>(h) * N + qrow] * kLog2e : 0.f;
  // D = <dO, O> of the lane's row (each half of the wave holds half of the row), stored
  // for the dK/dV pass that follows: every row of every sequence is one wave's, per head
  float dlq;
  {
    float of[HALF];
    load_rows<D>(of, at(op, r0, HD), qsafe - r0, HD, g);
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < HALF; ++i) part = fmaf(df[i], of[i], part);
    dlq = qvalid ? xhalf_sum(part) : 0.f;
    if (qvalid && g == 0) delta[static_cast<int64_t>(h) * N + qrow] = dlq;
  }

  floatx16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = floatx16{};

  if (wk0 < wk1) {
    // key blocks through buffer resources over their rows inside [wk0, wk1): rows past wk1 read 0
    const uint32_t vrow = (static_cast<uint32_t>(ql) * LD + g * HALF) * 4u;
    const uint32_t vtr = (static_cast<uint32_t>(4 * g) * LD + ql) * 4u;
    float kr[HALF], vr[HALF], kt[16][DB];
    auto load_kv = [&](int kb) {
      const int n = min(32, wk1 - kb);
      const auto rk = rows_rsrc(at(kp, kb, LD), n, LD), rv = rows_rsrc(at(vp, kb, LD), n, LD);
#pragma unroll
      for (int j = 0; j < HALF / 4; ++j) {
        const float4 x = buf_f32x4(rk, vrow + 16u * j, 0), y = buf_f32x4(rv, vrow + 16u * j, 0);
        kr[4 * j] = x.x, kr[4 * j + 1] = x.y, kr[4 * j + 2] = x.z, kr[4 * j + 3] = x.w;
        vr[4 * j] = y.x, vr[4 * j + 1] = y.y, vr[4 * j + 2] = y.z, vr[4 * j + 3] = y.w;
      }
    };
    auto load_kt = [&](int kb) {
      const auto rk = rows_rsrc(at(kp, kb, LD), min(32, wk1 - kb), LD);
#pragma unroll
      for (int st = 0; st < 16; ++st)
#pragma unroll
        for (int db = 0; db < DB; ++db) kt[st][db] = buf_f32(rk, vtr + 128u * db, (8u * (st >> 2) + (st & 3)) * LD * 4u);
    };
    for (int kb = wk0; kb < wk1; kb += 32) {
      load_kv(kb);
      floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
      for (int st = 0; st < HALF; ++st) {
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[st], qf[st], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[st], df[st], dp, 0, 0, 0);
      }
      load_kt(kb);
      if (!(kb >= mk0 && kb + 32 <= mk1)) {
        const int base = kb + 4 * g;
        mask_block(s, qk0 - base, qk1 - base);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c, -lse2));
        dp[i] = p * (dp[i] - dlq);
      }
#pragma unroll
      for (int st = 0; st < 16; ++st)
#pragma unroll
        for (int db = 0; db < DB; ++db) dq[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(kt[st][db], dp[st], dq[db], 0, 0, 0);
    }
  }
  if (qvalid) store_acc_row<float, D>(dqp, static_cast<int64_t>(qrow) * ld + hoff, dq, scale, g);
}

// dQ from the dS blocks the dK/dV pass stored (global attention): per 32-key block of the
// wave's sequence, dQ^T += K^T dS^T with the K scalars as A operands, 32 MFMAs per block at
// d = 64 instead of the 96 that recompute S and dP. A block arrives in the dK/dV
// accumulator layout (lane = key, chunk-major); the B operands want lane = query, so each block passes
// through 4 KB of LDS: written as the wave's 16-byte chunks, read back as single floats.
// Rows are placed so that both sides are free of bank conflicts: row L of the block
// (the 16 floats of stored lane L) sits at row prow(L) = L ^ bit2(L) ^ 2 bit5(L), its
// chunk c at chunk c ^ ((L >> 2) & 3).
template <int D>
__global__ __launch_bounds__(64, 2) void bwd_dq_ds_f32_kernel(const float* __restrict__ kp, const float* __restrict__ dsp,
                                                            const int32_t* __restrict__ cu,
                                                            const int32_t* __restrict__ items, int32_t B, int32_t H,
                                                            int32_t T, int32_t NB, int64_t ld, float scale,
                                                            float* __restrict__ dqp) {
  constexpr int DB = D / 32;
  __shared__ __align__(16) float tile[1024];
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lin / T, t = lin - h * T;
  const int lane = threadIdx.x, ql = lane & 31, g = lane >> 5;

  SeqTile sp;
  if (!seq_tile(cu, items, t, B, sp)) return;
  const int qrow = sp.r0 + ql;
  const bool qvalid = qrow < sp.rend;
  const uint32_t LD = static_cast<uint32_t>(ld);
  const int64_t hoff = static_cast<int64_t>(h) * D;
  const int sb = sp.lo / kRows + items[t];  // slot of the sequence's first tile
  const float* row = dsp + (static_cast<int64_t>(h) * T + sb + (sp.r0 - sp.lo) / kRows) * NB * 1024;
  const uint32_t vtr = (static_cast<uint32_t>(4 * g) * LD + ql) * 4u;

  // write side: float index of this lane's chunk c4
  int wr[4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4)
    wr[c4] = 16 * (lane ^ ((lane >> 2) & 1) ^ (((lane >> 5) & 1) << 1)) + 4 * (c4 ^ ((lane >> 2) & 3));
  // read side: at step st = 8 u + 4 a + b the lane takes dS[ql][key], key = 8 (st/4) + 4 g + b,
  // element 4 (ql/8) + ql%4 of stored lane key + 32 gq (gq = bit 2 of ql); its float index
  // is rd[a][b] + 256 u
  const int gq = (ql >> 2) & 1;
  int rd[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int prow = 8 * a + (b ^ (g | (gq << 1))) + 4 * g + 32 * gq;
      rd[a][b] = 16 * prow + 4 * ((ql >> 3) ^ ((2 * a + g) & 3)) + (ql & 3);
    }

  floatx16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = floatx16{};
  const int nb = min(NB, (sp.hi - sp.lo + kRows - 1) / kRows);  // blocks the dK/dV pass stored
  // Two register sets: block j + 1 is fetched into one while block j's MFMAs read the
  // other (buffer loads for dS: plain loads here are merged into a single load at the
  // loop's head, which waits for it at once)
  struct Blk {
    floatx4 x[4];
    float k[16][DB];
  };
  Blk b0, b1;
  const auto rds = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, nb * 4096, kBufferFlags);
  const int vl = lane * 16;  // byte offset of the lane's float4 in each 1 KB chunk
  auto fetch = [&](int j, Blk& bk) {
    const int o = j * 4096;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
      bk.x[c4] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rds, vl + 1024 * c4, o, kNonTemporal));
    // K[key(st)][d] for the key order of the dS operands; rows past the sequence read 0
    const int kb = sp.lo + j * kRows;
    const auto rk = rows_rsrc(kp + (static_cast<int64_t>(kb) * LD + hoff), min(kRows, sp.hi - kb), LD);
#pragma unroll
    for (int st = 0; st < 16; ++st)
#pragma unroll
      for (int db = 0; db < DB; ++db) bk.k[st][db] = buf_f32(rk, vtr + 128u * db, (8u * (st >> 2) + (st & 3)) * LD * 4u);
  };
  auto consume = [&](const Blk& bk) {
    __syncthreads();  // the previous block's reads are done
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) *reinterpret_cast<floatx4*>(&tile[wr[c4]]) = bk.x[c4];
    __syncthreads();
    float ds[16];
#pragma unroll
    for (int st = 0; st < 16; ++st) ds[st] = tile[rd[(st >> 2) & 1][st & 3] + 256 * (st >> 3)];
#pragma unroll
    for (int st = 0; st < 16; ++st)
#pragma unroll
      for (int db = 0; db < DB; ++db) dq[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(bk.k[st][db], ds[st], dq[db], 0, 0, 0);
  };
  if (nb > 0) fetch(0, b0);
  for (int j = 0; j < nb; j += 2) {
    if (j + 1 < nb) fetch(j + 1, b1);
    consume(b0);
    if (j + 1 >= nb) break;
    if (j + 2 < nb) fetch(j + 2, b0);
    consume(b1);
  }
  if (qvalid) store_acc_row<float, D>(dqp, static_cast<int64_t>(qrow) * ld + hoff, dq, scale, g);
}

}  // namespace

hipError_t launch_bwd_dq_f32_wave(int D, const void* dout, const void* q, const void* k, const void* v,
                                  const void* out, const float* lse, float* delta, const int32_t* cu,
                                  const int32_t* items32,
                                  int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* dq,
                                  hipStream_t stream) {
  const int T = N / kRows + B;  // slots of the sequence-aligned work list
  const int64_t blocks = static_cast<int64_t>(T) * H;
  if (blocks == 0) return hipSuccess;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  const dim3 gd(static_cast<unsigned>(blocks)), bd(64);
  hipEvent_t ev = timing_start(stream);
  if (D == 32)
    hipLaunchKernelGGL((bwd_dq_f32_kernel<32>), gd, bd, 0, stream, static_cast<const float*>(dout),
                       static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                       static_cast<const float*>(out), lse, delta, cu, items32, B, N, H, T, win, ld, c, scale,
                       static_cast<float*>(dq));
  else if (D == 64)
    hipLaunchKernelGGL((bwd_dq_f32_kernel<64>), gd, bd, 0, stream, static_cast<const float*>(dout),
                       static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                       static_cast<const float*>(out), lse, delta, cu, items32, B, N, H, T, win, ld, c, scale,
                       static_cast<float*>(dq));
  else
    return hipErrorInvalidValue;
  timing_stop("bwd_dq", ev, stream);
  return hipGetLastError();
}

}  // namespace pe

// ---------------------------------------------------------------- fp32 dK/dV, one wave per 32 key rows
// The mirror of the dQ walk, over the query span of the wave's 32 keys:
//   S = Q K^T, dP = dO V^T                  (Q and dO row chunks as A operands,
//                                            K and V rows held for the whole walk)
//   P = exp2(c S - lse2), dS = P (dP - D)   (row statistics per query = per register)
//   dV^T += dO^T P, dK^T += Q^T dS          (dO and Q scalars as A operands)
// The per-query statistics arrive one per lane (query = lane%32) and are
// turned into the per-register layout through a 32-float LDS slot.
namespace pe {
namespace {

template <int D, bool kDs>
__global__ __launch_bounds__(64, 2) void bwd_dkdv_f32_kernel(
    const float* __restrict__ dop, const float* __restrict__ qp, const float* __restrict__ kp,
    const float* __restrict__ vp, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N, int32_t H, int32_t T,
    int32_t win, int64_t ld, float c, float scale, float* __restrict__ dkp, float* __restrict__ dvp,
    float* __restrict__ dsp, int32_t NB) {
  constexpr int HALF = D / 2, DB = D / 32;
  __shared__ __align__(16) float stat[2][kRows];
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lin / T, t = lin - h * T;
  const int lane = threadIdx.x, ql = lane & 31, g = lane >> 5;

  SeqTile sp;
  if (!seq_tile(cu, items, t, B, sp)) return;
  const int r0 = sp.r0;
  const int krow = r0 + ql;
  const bool kvalid = krow < sp.rend;
  int kq0 = 0, kq1 = 0;
  if (kvalid) {  // the queries that attend to this key
    kq0 = sp.lo;
    kq1 = sp.hi;
    band_limit(krow, win, kq0, kq1);
  }
  const int wq0 = __builtin_amdgcn_readfirstlane(wave_min_i(kvalid ? kq0 : INT_MAX));
  const int wq1 = __builtin_amdgcn_readfirstlane(wave_max_i(kvalid ? kq1 : INT_MIN));
  const int mq0 = __builtin_amdgcn_readfirstlane(wave_max_i(kvalid ? kq0 : INT_MIN));
  const int mq1 = __builtin_amdgcn_readfirstlane(wave_min_i(kvalid ? kq1 : INT_MAX));

  float kr[HALF], vr[HALF];
  const int ksafe = kvalid ? krow : r0;
  const uint32_t HD = static_cast<uint32_t>(H) * D;  // rows of dO
  const uint32_t LD = static_cast<uint32_t>(ld);     // rows of Q, K, V, dK and dV
  const int64_t hoff = static_cast<int64_t>(h) * D;
  auto at = [&](const float* p, int row, uint32_t stride) { return p + (static_cast<int64_t>(row) * stride + hoff); };
  load_rows<D>(kr, at(kp, r0, LD), ksafe - r0, LD, g);
  load_rows<D>(vr, at(vp, r0, LD), ksafe - r0, LD, g);

  floatx16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = floatx16{};

  const float* lse_h = lse + static_cast<int64_t>(h) * N;
  const float* del_h = delta + static_cast<int64_t>(h) * N;
  // Query blocks load through buffer resources over their rows inside [wq0, wq1), so rows
  // past wq1 read 0 and no lane computes an address per load. Two waves share a SIMD
  // (256 registers each), one computing while the other waits for its loads; a
  // one-wave kernel prefetching a block ahead (360 registers) ran 1.2x slower.
  const uint32_t vrow_q = (static_cast<uint32_t>(ql) * LD + g * HALF) * 4u;
  const uint32_t vrow_d = (static_cast<uint32_t>(ql) * HD + g * HALF) * 4u;
  const uint32_t vtr_q = (static_cast<uint32_t>(4 * g) * LD + ql) * 4u;
  const uint32_t vtr_d = (static_cast<uint32_t>(4 * g) * HD + ql) * 4u;
  float qr[HALF], dr[HALF];
  float lse_r = 0.f, del_r = 0.f;
  auto load_rows_blk = [&](int qb) {
    const int n = min(32, wq1 - qb);
    const auto rq = rows_rsrc(at(qp, qb, LD), n, LD), rd = rows_rsrc(at(dop, qb, HD), n, HD);
#pragma unroll
    for (int j = 0; j < HALF / 4; ++j) {
      const float4 x = buf_f32x4(rq, vrow_q + 16u * j, 0), y = buf_f32x4(rd, vrow_d + 16u * j, 0);
      qr[4 * j] = x.x, qr[4 * j + 1] = x.y, qr[4 * j + 2] = x.z, qr[4 * j + 3] = x.w;
      dr[4 * j] = y.x, dr[4 * j + 1] = y.y, dr[4 * j + 2] = y.z, dr[4 * j + 3] = y.w;
    }
    lse_r = buf_f32(rows_rsrc(lse_h + qb, n, 1), ql * 4u, 0);
    del_r = buf_f32(rows_rsrc(del_h + qb, n, 1), ql * 4u, 0);
  };
  // dS hand-off (global attention: the walk covers the sequence's query blocks from lo):
  // block (query block (qb - lo)/32, key block (r0 - lo)/32) of the sequence, one block of
  // NB * 1024 floats further per query block; a key block at or past NB (a length above
  // the stated maximum) writes nothing
  float* dsw = nullptr;
  if constexpr (kDs) {
    const int sb = sp.lo / kRows + items[t];  // slot of the sequence's first tile
    if (r0 - sp.lo < NB * kRows)
      dsw = dsp + ((static_cast<int64_t>(h) * T + sb + (wq0 - sp.lo) / kRows) * NB + (r0 - sp.lo) / kRows) * 1024;
  }
  for (int qb = wq0; qb < wq1; qb += 32) {
    load_rows_blk(qb);
    if (g == 0) {
      stat[0][ql] = lse_r * kLog2e;
      stat[1][ql] = del_r;
    }
    floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
    for (int st = 0; st < HALF; ++st) {
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(qr[st], kr[st], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x2f32(dr[st], vr[st], dp, 0, 0, 0);
    }
    float qt[16][DB], dt[16][DB];
    {
      const int n = min(32, wq1 - qb);
      const auto rq = rows_rsrc(at(qp, qb, LD), n, LD), rd = rows_rsrc(at(dop, qb, HD), n, HD);
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const uint32_t r = 8 * (st >> 2) + (st & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          qt[st][db] = buf_f32(rq, vtr_q + 128u * db, r * LD * 4u);
          dt[st][db] = buf_f32(rd, vtr_d + 128u * db, r * HD * 4u);
        }
      }
    }
    if (!(qb >= mq0 && qb + 32 <= mq1)) {
      const int base = qb + 4 * g;
      mask_block(s, kq0 - base, kq1 - base);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 l4 = *reinterpret_cast<const float4*>(&stat[0][8 * j + 4 * g]);
      const float4 d4 = *reinterpret_cast<const float4*>(&stat[1][8 * j + 4 * g]);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * j + e;
        const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c, -lv[e]));
        s[i] = p;
        dp[i] = p * (dp[i] - dl[e]);
      }
    }
    __syncthreads();
    if constexpr (kDs) {
      // stored in the accumulator layout, chunk-major: the lane's c-th four values
      // (queries 8 c + 4 g + 0..3 of key ql) go to float4 c * 64 + lane, so each of the
      // four stores writes 1 KB contiguous. Keys past the sequence store finite values that
      // meet zero K rows in the dQ pass. The lane offset is recomputed here (not kept across
      // the loop, where it would take a register the loop cannot spare).
      if (dsw != nullptr) {
        floatx4* dst = reinterpret_cast<floatx4*>(dsw) + lane_now();
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)  // streamed: read once by the dQ pass
          __builtin_nontemporal_store(floatx4{dp[4 * c4], dp[4 * c4 + 1], dp[4 * c4 + 2], dp[4 * c4 + 3]},
                                      dst + 64 * c4);
        dsw += static_cast<int64_t>(NB) * 1024;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j > 0 && qb + 8 * j >= wq1) break;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(dt[4 * j + e][db], s[4 * j + e], dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(qt[4 * j + e][db], dp[4 * j + e], dk[db], 0, 0, 0);
        }
    }
  }
  if (kvalid) {
    const int64_t off = static_cast<int64_t>(krow) * ld + hoff;
    store_acc_row<float, D>(dkp, off, dk, scale, g);
    store_acc_row<float, D>(dvp, off, dv, 1.0f, g);
  }
}

}  // namespace

hipError_t launch_bwd_dkdv_f32_wave(int D, const void* dout, const void* q, const void* k, const void* v,
                                    const float* lse, const float* delta, const int32_t* cu, const int32_t* items32,
                                    int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* dk,
                                    void* dv, float* ds, int32_t nb_max, hipStream_t stream) {
  const int T = N / kRows + B;  // slots of the sequence-aligned work list
  const int64_t blocks = static_cast<int64_t>(T) * H;
  if (blocks == 0) return hipSuccess;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  const dim3 gd(static_cast<unsigned>(blocks)), bd(64);
  hipEvent_t ev = timing_start(stream);
  if (D == 32)
    hipLaunchKernelGGL((ds != nullptr ? bwd_dkdv_f32_kernel<32, true> : bwd_dkdv_f32_kernel<32, false>), gd, bd, 0,
                       stream, static_cast<const float*>(dout), static_cast<const float*>(q),
                       static_cast<const float*>(k), static_cast<const float*>(v), lse, delta, cu, items32, B, N, H, T,
                       win, ld, c, scale, static_cast<float*>(dk), static_cast<float*>(dv), ds, nb_max);
  else if (D == 64)
    hipLaunchKernelGGL((ds != nullptr ? bwd_dkdv_f32_kernel<64, true> : bwd_dkdv_f32_kernel<64, false>), gd, bd, 0,
                       stream, static_cast<const float*>(dout), static_cast<const float*>(q),
                       static_cast<const float*>(k), static_cast<const float*>(v), lse, delta, cu, items32, B, N, H, T,
                       win, ld, c, scale, static_cast<float*>(dk), static_cast<float*>(dv), ds, nb_max);
  else
    return hipErrorInvalidValue;
  timing_stop("bwd_dkdv", ev, stream);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_ds_f32_wave(int D, const void* k, const float* ds, int32_t nb_max, const int32_t* cu,
                                     const int32_t* items32, int32_t B, int32_t N, int32_t H, int64_t ld, float scale,
                                     void* dq, hipStream_t stream) {
  const int T = N / kRows + B;  // slots of the sequence-aligned work list
  const int64_t blocks = static_cast<int64_t>(T) * H;
  if (blocks == 0) return hipSuccess;
  const dim3 gd(static_cast<unsigned>(blocks)), bd(64);
  hipEvent_t ev = timing_start(stream);
  if (D == 32)
    hipLaunchKernelGGL((bwd_dq_ds_f32_kernel<32>), gd, bd, 0, stream, static_cast<const float*>(k), ds, cu, items32, B,
                       H, T, nb_max, ld, scale, static_cast<float*>(dq));
  else if (D == 64)
    hipLaunchKernelGGL((bwd_dq_ds_f32_kernel<64>), gd, bd, 0, stream, static_cast<const float*>(k), ds, cu, items32, B,
                       H, T, nb_max, ld, scale, static_cast<float*>(dq));
  else
    return hipErrorInvalidValue;
  timing_stop("bwd_dq", ev, stream);
  return hipGetLastError();
}

}  // namespace pe
