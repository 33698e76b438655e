// fp32 attention kernels with one independent wave per 32 rows of one sequence: the
// forward, and the dQ and dK/dV passes of the backward. Tiles start at each
// sequence's first row (the sequence-aligned work list), so a wave's rows share one
// key range and the 32x32 products only overhang at a sequence's last tile; there
// the forward and the dK/dV pass skip the products of whole 8-row groups past the
// range (in the dQ pass that measured no faster).
//
// fp32 forward, one independent wave per (head, 32 query rows).
//
// On fp32 the MFMA operands of both products are one element per lane per
// step, so no operand ever needs a transposed copy and the waves need not share
// an LDS tile. Each wave therefore walks only the key span of its own 32 rows,
// in 32-key steps starting exactly at the first key it needs, with K and V
// operands loaded straight from global memory (L2-resident: neighbouring waves
// read the same sequences) one step ahead of their use. There are no LDS tiles
// and no barriers, so a wave whose rows cover short sequences never waits for
// one covering long ones.
//
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

template <int D>
struct F32Ops {
  static constexpr int HALF = D / 2;  // head-dim elements per lane half (MFMA steps of S)
  static constexpr int DB = D / 32;   // 32-row blocks of O^T
  float k[HALF];                      // K[key][g*HALF + st], key = kb + lane%32
  float v[16][DB];                    // V[kb + 8(st/4) + 4g + st%4][db*32 + lane%32]
};

template <int D>
__device__ __forceinline__ void load_ops(F32Ops<D>& ops, const float* __restrict__ kp, const float* __restrict__ vp,
                                         int kb, int klast, int64_t ld, int h, int ql, int g) {
  using O = F32Ops<D>;
  {
    const int key = min(kb + ql, klast);
    const float4* src = reinterpret_cast<const float4*>(kp + static_cast<int64_t>(key) * ld + h * D + g * O::HALF);
#pragma unroll
    for (int j = 0; j < O::HALF / 4; ++j) {
      const float4 x = src[j];
      ops.k[4 * j + 0] = x.x;
      ops.k[4 * j + 1] = x.y;
      ops.k[4 * j + 2] = x.z;
      ops.k[4 * j + 3] = x.w;
    }
  }
#pragma unroll
  for (int st = 0; st < 16; ++st) {
    const int key = min(kb + 8 * (st >> 2) + 4 * g + (st & 3), klast);
    const float* row = vp + static_cast<int64_t>(key) * ld + h * D;
#pragma unroll
    for (int db = 0; db < O::DB; ++db) ops.v[st][db] = row[db * 32 + ql];
  }
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
    load_ops<D>(a, kp, vp, wk0, klast, ld, h, ql, g);
    for (int kb = wk0; kb < wk1; kb += 64) {
      // Unconditional (rows clamp to klast, so a step past the end reloads the last rows): a
      // load under a branch makes the wait counts at the join assume the worst path and wait
      // for the younger loads too. The empty asm keeps each load group where it is written.
      load_ops<D>(b, kp, vp, kb + 32, klast, ld, h, ql, g);
      asm volatile("" ::: "memory");
      block(a, kb);
      if (kb + 32 >= wk1) break;
      load_ops<D>(a, kp, vp, kb + 64, klast, ld, h, ql, g);
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

bool attn_fwd_f32_wave_supported(int D) { return D == 32 || D == 64; }

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

// t[st][db] = X[row 8(st/4) + 4g + st%4 (clamped to `last`)][db*32 + lane%32], rows relative to `base`.
template <int D>
__device__ __forceinline__ void load_tr(float (&t)[16][D / 32], const float* __restrict__ base, int last, uint32_t HD,
                                        int ql, int g) {
#pragma unroll
  for (int st = 0; st < 16; ++st) {
    const uint32_t rel = static_cast<uint32_t>(min(8 * (st >> 2) + 4 * g + (st & 3), last));
    const float* row = base + (rel * HD + static_cast<uint32_t>(ql));
#pragma unroll
    for (int db = 0; db < D / 32; ++db) t[st][db] = row[db * 32];
  }
}

template <int D>
__global__ __launch_bounds__(64, 2) void bwd_dq_f32_kernel(
    const float* __restrict__ dop, const float* __restrict__ qp, const float* __restrict__ kp,
    const float* __restrict__ vp, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N, int32_t H, int32_t T,
    int32_t win, int64_t ld, float c, float scale, float* __restrict__ dqp) {
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
  const float dlq = qvalid ? delta[static_cast<int64_t>(h) * N + qrow] : 0.f;

  floatx16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = floatx16{};

  if (wk0 < wk1) {
    const int klast = wk1 - 1;
    float kr[HALF], vr[HALF], kt[16][DB];
    load_rows<D>(kr, at(kp, wk0, LD), min(ql, klast - wk0), LD, g);
    load_rows<D>(vr, at(vp, wk0, LD), min(ql, klast - wk0), LD, g);
    load_tr<D>(kt, at(kp, wk0, LD), klast - wk0, LD, ql, g);
    for (int kb = wk0; kb < wk1; kb += 32) {
      const bool more = kb + 32 < wk1;
      floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
      for (int st = 0; st < HALF; ++st) {
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[st], qf[st], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[st], df[st], dp, 0, 0, 0);
      }
      {
        const int nb = more ? kb + 32 : kb;
        load_rows<D>(kr, at(kp, nb, LD), min(ql, klast - nb), LD, g);
        load_rows<D>(vr, at(vp, nb, LD), min(ql, klast - nb), LD, g);
        asm volatile("" ::: "memory");
      }
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
      {
        const int nb = more ? kb + 32 : kb;
        load_tr<D>(kt, at(kp, nb, LD), klast - nb, LD, ql, g);
        asm volatile("" ::: "memory");
      }
    }
  }
  if (qvalid) store_acc_row<float, D>(dqp, static_cast<int64_t>(qrow) * ld + hoff, dq, scale, g);
}

}  // namespace

hipError_t launch_bwd_dq_f32_wave(int D, const void* dout, const void* q, const void* k, const void* v,
                                  const float* lse, const float* delta, const int32_t* cu, const int32_t* items32,
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
                       static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v), lse,
                       delta, cu, items32, B, N, H, T, win, ld, c, scale, static_cast<float*>(dq));
  else if (D == 64)
    hipLaunchKernelGGL((bwd_dq_f32_kernel<64>), gd, bd, 0, stream, static_cast<const float*>(dout),
                       static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v), lse,
                       delta, cu, items32, B, N, H, T, win, ld, c, scale, static_cast<float*>(dq));
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

template <int D>
__global__ __launch_bounds__(64, D > 32 ? 1 : 2) void bwd_dkdv_f32_kernel(
    const float* __restrict__ dop, const float* __restrict__ qp, const float* __restrict__ kp,
    const float* __restrict__ vp, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N, int32_t H, int32_t T,
    int32_t win, int64_t ld, float c, float scale, float* __restrict__ dkp, float* __restrict__ dvp) {
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
  // The rows of the next query block (and their statistics) load under this block's dV/dK
  // products; the transposed operands of a block load under its own S/dP products.
  const int qlast = wq1 - 1;
  float qr[HALF], dr[HALF];
  float lse_r = 0.f, del_r = 0.f;
  auto load_rows_blk = [&](int qb) {
    const int qrow = min(qb + ql, qlast);
    load_rows<D>(qr, at(qp, qb, LD), qrow - qb, LD, g);
    load_rows<D>(dr, at(dop, qb, HD), qrow - qb, HD, g);
    lse_r = lse_h[qrow];
    del_r = del_h[qrow];
  };
  if (wq0 < wq1) load_rows_blk(wq0);
  for (int qb = wq0; qb < wq1; qb += 32) {
    float qt[16][DB], dt[16][DB];
    load_tr<D>(qt, at(qp, qb, LD), qlast - qb, LD, ql, g);
    load_tr<D>(dt, at(dop, qb, HD), qlast - qb, HD, ql, g);
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
    // rows of this block are queries qb + 8(i/4) + 4g + i%4; keep those inside the key's own sequence
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
    // unconditional (the last block reloads itself), so no branch splits the wait counts; the
    // empty asm keeps these loads here instead of letting them merge with the next iteration's use
    load_rows_blk(qb + 32 < wq1 ? qb + 32 : qb);
    asm volatile("" ::: "memory");
    // queries at or past wq1 have P = dS = 0 for every key of the wave: skip their steps
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
                                    void* dv, hipStream_t stream) {
  const int T = N / kRows + B;  // slots of the sequence-aligned work list
  const int64_t blocks = static_cast<int64_t>(T) * H;
  if (blocks == 0) return hipSuccess;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  const dim3 gd(static_cast<unsigned>(blocks)), bd(64);
  hipEvent_t ev = timing_start(stream);
  if (D == 32)
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<32>), gd, bd, 0, stream, static_cast<const float*>(dout),
                       static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v), lse,
                       delta, cu, items32, B, N, H, T, win, ld, c, scale, static_cast<float*>(dk),
                       static_cast<float*>(dv));
  else if (D == 64)
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<64>), gd, bd, 0, stream, static_cast<const float*>(dout),
                       static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v), lse,
                       delta, cu, items32, B, N, H, T, win, ld, c, scale, static_cast<float*>(dk),
                       static_cast<float*>(dv));
  else
    return hipErrorInvalidValue;
  timing_stop("bwd_dkdv", ev, stream);
  return hipGetLastError();
}

}  // namespace pe
