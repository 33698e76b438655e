// Backward of non-causal attention over packed sequences, recomputing the
// probabilities from the forward's log-sum-exp. Three launches, no atomics,
// so the result is bitwise reproducible:
//
//   delta:  D[h, i] = <dO[i, h, :], O[i, h, :]>                       (HBM-bound)
//   dK/dV:  per head and tile of 128 packed KEY rows (4 waves x 32 keys), over
//           the query rows of every sequence the tile touches, 64 at a time:
//             S  = Q K^T, dP = dO V^T                (mma_rows_regs, K and V in registers)
//             P  = exp(scale*S - lse), dS = P (dP - D)
//             dV^T += dO^T P, dK^T += Q^T dS          (mma_tr_regs, Q and dO from LDS)
//   dQ:     per head and tile of 128 packed QUERY rows, over their keys:
//             S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D)
//             dQ^T += K^T dS^T
//   and dK, dQ are scaled by the softmax scale at the store.
//
// The dQ pass recomputes S and dP once more than an atomic-accumulation scheme
// would (14 instead of 10 matrix products of the size of S per head), the price
// of determinism. On the fp32 one-wave path (attn_f32_wave.hip) the dQ pass runs
// first and computes D of its own rows on the way (it holds dO already and reads
// O once), so there are two launches and no delta pass.
#include <climits>

#include "attn_common.h"

namespace pe {

namespace {

// One group of CHP lanes (CH rounded up to a power of two) per (row, head): lane
// `sub` of the group reads 16-byte chunk `sub` of both head rows (lanes past CH
// read nothing and add 0), and the group sums by butterfly.
template <typename Et, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const void* __restrict__ dout, const void* __restrict__ out,
                                                        int32_t N, int32_t H, float* __restrict__ delta) {
  using G = Geo<Et, D>;
  constexpr int CHP = pow2_ceil(G::CH);
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t hr = idx / CHP;  // (row, head) pair, row-major over [N, H]
  const int sub = static_cast<int>(idx - hr * CHP);
  const int64_t total = static_cast<int64_t>(N) * H;
  float s = 0.f;
  if (hr < total && sub < G::CH) {
    const int64_t ch = hr * G::CH + sub;
    const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const char*>(dout) + ch * 16);
    const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const char*>(out) + ch * 16);
    if constexpr (kIs16<Et>) {
      const u16x8 x = __builtin_bit_cast(u16x8, a), y = __builtin_bit_cast(u16x8, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(h16_to_f32<Et>(x[e]), h16_to_f32<Et>(y[e]), s);
    } else {
      const float4 x = __builtin_bit_cast(float4, a), y = __builtin_bit_cast(float4, b);
      s = fmaf(x.x, y.x, fmaf(x.y, y.y, fmaf(x.z, y.z, x.w * y.w)));
    }
  }
#pragma unroll
  for (int o = 1; o < CHP; o <<= 1) s += __shfl_xor(s, o);
  if (hr < total && sub == 0) {
    const int64_t i = hr / H, hh = hr - i * H;
    delta[hh * N + i] = s;
  }
}

template <typename Et, int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(
    const void* __restrict__ dop, const void* __restrict__ qp, const void* __restrict__ kp,
    const void* __restrict__ vp, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N, int32_t H,
    int32_t T, int32_t win, int64_t ld, float c, float scale, void* __restrict__ dkp, void* __restrict__ dvp) {
  using G = Geo<Et, D>;
  using E = typename G::E;
  // bf16 tiles with whole 16-byte chunks per lane half use the XOR-swizzled layout
  // (conflict-free for both the row reads and the transposing reads)
  constexpr bool SWZ = kIs16<Et> && D % 32 == 0;
  constexpr int TS = SWZ ? kBlk * D : G::TSZ;
  __shared__ __align__(16) E qt[2][TS];
  __shared__ __align__(16) E dt[2][TS];
  __shared__ __align__(16) float ls[2][kBlk];
  __shared__ __align__(16) float dl[2][kBlk];
  __shared__ int32_t cul[kAttnTileRows + 2];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lin / T, t = lin - h * T;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, ql = lane & 31, g = lane >> 5;

  const TileSpan sp = tile_span(cu, items, t, B, N, cul);
  if (sp.rend <= sp.r0) return;  // block-uniform: no rows in this tile
  const int krow = sp.r0 + wv * 32 + ql;
  const bool kvalid = krow < sp.rend;
  int jk0 = 0, jk1 = 0;  // query rows of this key's sequence
  if (kvalid) {
    own_range(cul, sp.ncu, krow, jk0, jk1);
    band_limit(krow, win, jk0, jk1);
  }
  const int wq0 = wave_min_i(kvalid ? jk0 : INT_MAX);
  const int wq1 = wave_max_i(kvalid ? jk1 : INT_MIN);
  const int mq0 = wave_max_i(kvalid ? jk0 : INT_MIN);
  const int mq1 = wave_min_i(kvalid ? jk1 : INT_MAX);

  typename RegT<Et>::type kreg[G::QS], vreg[G::QS];
  const int64_t roff = static_cast<int64_t>(krow) * ld + h * D;  // rows of K, V, dK, dV are ld apart
  load_row_regs<Et, D>(kp, roff, g, kvalid, kreg);
  load_row_regs<Et, D>(vp, roff, g, kvalid, vreg);

  floatx16 dk[G::DB], dv[G::DB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db) {
    dk[db] = floatx16{};
    dv[db] = floatx16{};
  }

  // query rows of the tile's sequences, and within win of its keys for local attention
  const int qlo = win >= 0 ? max(sp.lo, sp.r0 - win) : sp.lo;
  const int qhi = win >= 0 ? min(sp.hi, sp.rend + win) : sp.hi;
  uint4 qr[G::PER], dr[G::PER];
  float lsr = 0.f, dlr = 0.f;
  const float* lse_h = lse + static_cast<int64_t>(h) * N;
  const float* del_h = delta + static_cast<int64_t>(h) * N;
  auto gload = [&](int qb) {
    tile_gload<Et, D>(qp, qb, qhi, ld, h, qr);
    tile_gload<Et, D>(dop, qb, qhi, static_cast<int64_t>(H) * D, h, dr);
    if (tid < kBlk) {  // raw values: any arithmetic here would wait for the whole prefetch
      const int row = min(qb + tid, qhi - 1);
      lsr = lse_h[row];
      dlr = del_h[row];
    }
  };

  int buf = 0;
  if (qlo < qhi) gload(qlo);
  for (int qb = qlo; qb < qhi; qb += kBlk) {
    if constexpr (SWZ) {
      tile_store_swz<D>(qt[buf], qr);
      tile_store_swz<D>(dt[buf], dr);
    } else {
      tile_store<Et, D>(qt[buf], qr);
      tile_store<Et, D>(dt[buf], dr);
    }
    if (tid < kBlk) {
      const bool in = qb + tid < qhi;
      ls[buf][tid] = in ? lsr * kLog2e : 0.f;
      dl[buf][tid] = in ? dlr : 0.f;
    }
    __syncthreads();
    if (qb + kBlk < qhi) gload(qb + kBlk);
    if (qb < wq1 && qb + kBlk > wq0) {
      const bool need_mask = !(qb >= mq0 && qb + kBlk <= mq1);
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        floatx16 s = floatx16{}, dp = floatx16{};
        if constexpr (SWZ) {
          mma_rows_swz<Et, D>(qt[buf], 32 * qq, kreg, s, ql, g);   // S[q][key]
          mma_rows_swz<Et, D>(dt[buf], 32 * qq, vreg, dp, ql, g);  // dP[q][key]
        } else {
          mma_rows_regs<Et, D>(qt[buf], 32 * qq, kreg, s, ql, g);
          mma_rows_regs<Et, D>(dt[buf], 32 * qq, vreg, dp, ql, g);
        }
        const int base = qb + 32 * qq + 4 * g;
        if (need_mask) mask_block(s, jk0 - base, jk1 - base);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const float4 l4 = *reinterpret_cast<const float4*>(&ls[buf][32 * qq + 8 * i4 + 4 * g]);
          const float4 d4 = *reinterpret_cast<const float4*>(&dl[buf][32 * qq + 8 * i4 + 4 * g]);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 4 * i4 + j;
            const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c, -lv[j]));
            s[i] = p;
            dp[i] = p * (dp[i] - dvv[j]);
          }
        }
        if constexpr (SWZ) {
          vec8<Et> pb[2], sb[2];
          acc_to_h16<Et>(s, pb);
          acc_to_h16<Et>(dp, sb);
          mma_tr_swz<Et, D>(dt[buf], 32 * qq, pb, dv, lane);  // dV^T += dO^T P
          mma_tr_swz<Et, D>(qt[buf], 32 * qq, sb, dk, lane);  // dK^T += Q^T dS
        } else {
          mma_tr_regs<Et, D>(dt[buf], 32 * qq, s, dv, lane);
          mma_tr_regs<Et, D>(qt[buf], 32 * qq, dp, dk, lane);
        }
      }
    }
    buf ^= 1;
  }
  if (kvalid) {
    store_acc_row<Et, D>(dkp, roff, dk, scale, g);
    store_acc_row<Et, D>(dvp, roff, dv, 1.f, g);
  }
}

template <typename Et, int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const void* __restrict__ dop, const void* __restrict__ qp, const void* __restrict__ kp,
    const void* __restrict__ vp, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N, int32_t H,
    int32_t T, int32_t win, int64_t ld, float c, float scale, void* __restrict__ dqp) {
  using G = Geo<Et, D>;
  using E = typename G::E;
  constexpr bool SWZ = kIs16<Et> && D % 32 == 0;
  constexpr int TS = SWZ ? kBlk * D : G::TSZ;
  __shared__ __align__(16) E kt[2][TS];
  __shared__ __align__(16) E vt[2][TS];
  __shared__ int32_t cul[kAttnTileRows + 2];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lin / T, t = lin - h * T;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, ql = lane & 31, g = lane >> 5;

  const TileSpan sp = tile_span(cu, items, t, B, N, cul);
  if (sp.rend <= sp.r0) return;  // block-uniform: no rows in this tile
  const int qrow = sp.r0 + wv * 32 + ql;
  const bool qvalid = qrow < sp.rend;
  int qk0 = 0, qk1 = 0;
  if (qvalid) {
    own_range(cul, sp.ncu, qrow, qk0, qk1);
    band_limit(qrow, win, qk0, qk1);
  }
  const int wk0 = wave_min_i(qvalid ? qk0 : INT_MAX);
  const int wk1 = wave_max_i(qvalid ? qk1 : INT_MIN);
  const int mk0 = wave_max_i(qvalid ? qk0 : INT_MIN);
  const int mk1 = wave_min_i(qvalid ? qk1 : INT_MAX);

  typename RegT<Et>::type qreg[G::QS], dreg[G::QS];
  const int64_t roff = static_cast<int64_t>(qrow) * ld + h * D;  // rows of Q and dQ are ld apart
  load_row_regs<Et, D>(qp, roff, g, qvalid, qreg);
  load_row_regs<Et, D>(dop, (static_cast<int64_t>(qrow) * H + h) * D, g, qvalid, dreg);
  const float lse2 = qvalid ? lse[static_cast<int64_t>(h) * N + qrow] * kLog2e : 0.f;
  const float dlq = qvalid ? delta[static_cast<int64_t>(h) * N + qrow] : 0.f;

  floatx16 dq[G::DB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db) dq[db] = floatx16{};

  uint4 kr[G::PER], vr[G::PER];
  const int klo = win >= 0 ? max(sp.lo, sp.r0 - win) : sp.lo;
  const int khi = win >= 0 ? min(sp.hi, sp.rend + win) : sp.hi;
  int buf = 0;
  if (klo < khi) {
    tile_gload<Et, D>(kp, klo, khi, ld, h, kr);
    tile_gload<Et, D>(vp, klo, khi, ld, h, vr);
  }
  for (int kb = klo; kb < khi; kb += kBlk) {
    if constexpr (SWZ) {
      tile_store_swz<D>(kt[buf], kr);
      tile_store_swz<D>(vt[buf], vr);
    } else {
      tile_store<Et, D>(kt[buf], kr);
      tile_store<Et, D>(vt[buf], vr);
    }
    __syncthreads();
    if (kb + kBlk < khi) {
      tile_gload<Et, D>(kp, kb + kBlk, khi, ld, h, kr);
      tile_gload<Et, D>(vp, kb + kBlk, khi, ld, h, vr);
    }
    if (kb < wk1 && kb + kBlk > wk0) {
      const bool need_mask = !(kb >= mk0 && kb + kBlk <= mk1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        floatx16 s = floatx16{}, dp = floatx16{};
        if constexpr (SWZ) {
          mma_rows_swz<Et, D>(kt[buf], 32 * kk, qreg, s, ql, g);   // S^T[key][q]
          mma_rows_swz<Et, D>(vt[buf], 32 * kk, dreg, dp, ql, g);  // dP^T[key][q]
        } else {
          mma_rows_regs<Et, D>(kt[buf], 32 * kk, qreg, s, ql, g);
          mma_rows_regs<Et, D>(vt[buf], 32 * kk, dreg, dp, ql, g);
        }
        if (need_mask) {
          const int base = kb + 32 * kk + 4 * g;
          mask_block(s, qk0 - base, qk1 - base);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c, -lse2));
          dp[i] = p * (dp[i] - dlq);
        }
        if constexpr (SWZ) {
          vec8<Et> sb[2];
          acc_to_h16<Et>(dp, sb);
          mma_tr_swz<Et, D>(kt[buf], 32 * kk, sb, dq, lane);  // dQ^T += K^T dS^T
        } else {
          mma_tr_regs<Et, D>(kt[buf], 32 * kk, dp, dq, lane);
        }
      }
    }
    buf ^= 1;
  }
  if (qvalid) store_acc_row<Et, D>(dqp, roff, dq, scale, g);
}

template <typename Et, int D>
hipError_t bwd_dispatch(const void* dout, const void* q, const void* k, const void* v, const void* out,
                        const float* lse, const int32_t* cu, const int32_t* items, const int32_t* items32, int32_t B,
                        int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* dq, void* dk, void* dv,
                        float* delta, float* ds, int32_t nb_max, hipStream_t stream) {
  using G = Geo<Et, D>;
  if (N == 0) return hipSuccess;
  const int64_t lanes = static_cast<int64_t>(N) * H * pow2_ceil(G::CH);
  auto delta_pass = [&]() {
    hipEvent_t ev_bwd_delta = timing_start(stream);
    hipLaunchKernelGGL((bwd_delta_kernel<Et, D>), dim3(static_cast<unsigned>((lanes + 255) / 256)), dim3(256), 0,
                       stream, dout, out, N, H, delta);
    timing_stop("bwd_delta", ev_bwd_delta, stream);
    return hipGetLastError();
  };
  if (!kIs16<Et> && items32 != nullptr && attn_f32_wave_supported(D, ld, H) && ds != nullptr && win < 0) {
    // dS handed from the dK/dV pass to the dQ pass: 10 products of the size of S instead of 14
    hipError_t e = delta_pass();
    if (e != hipSuccess) return e;
    e = launch_bwd_dkdv_f32_wave(D, dout, q, k, v, lse, delta, cu, items32, B, N, H, win, ld, scale, dk, dv, ds,
                                 nb_max, stream);
    if (e != hipSuccess) return e;
    return launch_bwd_dq_ds_f32_wave(D, k, ds, nb_max, cu, items32, B, N, H, ld, scale, dq, stream);
  }
  if (!kIs16<Et> && items32 != nullptr && attn_f32_wave_supported(D, ld, H)) {
    // the fp32 dQ pass computes D itself and stores it for the dK/dV pass
    hipError_t e = launch_bwd_dq_f32_wave(D, dout, q, k, v, out, lse, delta, cu, items32, B, N, H, win, ld, scale,
                                          dq, stream);
    if (e != hipSuccess) return e;
    return launch_bwd_dkdv_f32_wave(D, dout, q, k, v, lse, delta, cu, items32, B, N, H, win, ld, scale, dk, dv,
                                    nullptr, 0, stream);
  }
  hipError_t e = delta_pass();
  if (e != hipSuccess) return e;
  const int T = (N + kAttnTileRows - 1) / kAttnTileRows;
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(T) * H);
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipEvent_t ev_bwd_dkdv = timing_start(stream);
  hipLaunchKernelGGL((bwd_dkdv_kernel<Et, D>), dim3(blocks), dim3(kThreads), 0, stream, dout, q, k, v, lse, delta,
                   cu, items, B, N, H, T, win, ld, c, scale, dk, dv);
  timing_stop("bwd_dkdv", ev_bwd_dkdv, stream);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipEvent_t ev_bwd_dq = timing_start(stream);
  hipLaunchKernelGGL((bwd_dq_kernel<Et, D>), dim3(blocks), dim3(kThreads), 0, stream, dout, q, k, v, lse, delta,
                   cu, items, B, N, H, T, win, ld, c, scale, dq);
  timing_stop("bwd_dq", ev_bwd_dq, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(int dt, int D, const void* dout, const void* q, const void* k, const void* v,
                           const void* out, const float* lse, const int32_t* cu, const int32_t* items,
                           const int32_t* items32, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld,
                           float scale, void* dq, void* dk, void* dv, float* delta, float* ds, int32_t nb_max,
                           hipStream_t stream) {
#define PE_BWD_CASE(DD)                                                                                       \
  case DD:                                                                                                   \
    return dt == kDtF32  ? bwd_dispatch<float, DD>(dout, q, k, v, out, lse, cu, items, items32, B, N, H, win, ld, \
                                                  scale, dq, dk, dv, delta, ds, nb_max, stream)                             \
           : dt == kDtF16 ? bwd_dispatch<_Float16, DD>(dout, q, k, v, out, lse, cu, items, items32, B, N, H, win, \
                                                     ld, scale, dq, dk, dv, delta, ds, nb_max, stream)                      \
                         : bwd_dispatch<__bf16, DD>(dout, q, k, v, out, lse, cu, items, items32, B, N, H, win, ld, \
                                                   scale, dq, dk, dv, delta, ds, nb_max, stream);
  switch (D) {
    PE_HEAD_DIMS(PE_BWD_CASE)
    default: return hipErrorInvalidValue;
  }
#undef PE_BWD_CASE
}

}  // namespace pe
