// Backward of the first-token readout: one query per sequence (its first row),
// so every key row j of sequence b receives gradient from that single query:
//
//   P_j  = exp(scale <q_b, k_j> - lse_b)        D_b = <dO_b, O_b>
//   dS_j = P_j (<dO_b, v_j> - D_b)
//   dk_j = scale dS_j q_b     dv_j = P_j dO_b     dq_b = scale sum_j dS_j k_j
//
// One pass over K and V, HBM-bound like the forward: one block per (sequence,
// group of heads), threads laid out as [key slot][head][16-byte chunk of the
// head row] so each K/V row of the sequence (all heads of the group) is read
// once and each dK/dV row written once, fully coalesced. Each slot walks the
// keys slot, slot + KS, ... in batches of four rows whose loads are issued
// before any is used; dq partials of the slots merge through LDS at the end.
// A head row of GS chunks takes GSP lanes (GS rounded up to a power of two, for
// the butterfly sums); lanes past GS load nothing, add zero and store nothing.
// No atomics: every output element has exactly one writer.
#include <algorithm>
#include <type_traits>

#include "attn_common.h"

namespace pe {

namespace {

constexpr int kFbThreads = 512;
constexpr int kFbBatch = 4;

template <typename Et, int D>
__global__ __launch_bounds__(kFbThreads) void attn_bwd_first_kernel(
    const void* __restrict__ dof, const void* __restrict__ qf, const void* __restrict__ kp,
    const void* __restrict__ vp, const void* __restrict__ of, const float* __restrict__ lse,
    const int32_t* __restrict__ cu, int32_t B, int32_t N, int32_t H, int32_t HPB, int64_t ld, float c, float scale,
    void* __restrict__ dqp, void* __restrict__ dkp, void* __restrict__ dvp) {
  constexpr int ES = kIs16<Et> ? 2 : 4;
  constexpr int EPC = 16 / ES;  // elements per 16-byte chunk
  constexpr int GS = D / EPC;         // chunks per head row
  constexpr int GSP = pow2_ceil(GS);  // lanes per head row
  constexpr int U = kFbBatch;
  using Chunk = typename std::conditional<kIs16<Et>, u16x8, float4>::type;
  __shared__ float sq[kFbThreads * EPC];

  const int b = blockIdx.x;
  const int hg = blockIdx.y;
  const int tid = threadIdx.x;
  const int CPR = HPB * GSP;
  const int KS = kFbThreads / CPR;
  const int slot = tid / CPR, cidx = tid - slot * CPR;
  const int hl = cidx / GSP, sub = cidx - hl * GSP;
  const int h = hg * HPB + hl;
  const bool active = slot < KS && h < H;
  const bool live = GS == GSP || sub < GS;  // the lane holds a chunk of the row

  auto widen = [](const Chunk& x, float (&y)[EPC]) __attribute__((always_inline)) {
    if constexpr (kIs16<Et>) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) y[e] = h16_to_f32<Et>(x[e]);
    } else {
      y[0] = x.x; y[1] = x.y; y[2] = x.z; y[3] = x.w;
    }
  };
  auto narrow = [](const float (&y)[EPC]) __attribute__((always_inline)) {
    Chunk x;
    if constexpr (kIs16<Et>) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) x[e] = f32_to_h16<Et>(y[e]);
    } else {
      x = make_float4(y[0], y[1], y[2], y[3]);
    }
    return x;
  };

  float dq[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) dq[e] = 0.f;
  if (active) {
    const int c0 = cu[b], c1 = cu[b + 1];
    const int64_t hoff = static_cast<int64_t>(h) * D + sub * EPC;
    const int64_t boff = (static_cast<int64_t>(b) * H * D + hoff) * ES;
    float qv[EPC], dov[EPC], ov[EPC];
    if (live) {
      widen(*reinterpret_cast<const Chunk*>(static_cast<const char*>(qf) + boff), qv);
      widen(*reinterpret_cast<const Chunk*>(static_cast<const char*>(dof) + boff), dov);
      widen(*reinterpret_cast<const Chunk*>(static_cast<const char*>(of) + boff), ov);
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) qv[e] = dov[e] = ov[e] = 0.f;
    }
    float dd = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) dd = fmaf(dov[e], ov[e], dd);
#pragma unroll
    for (int o = 1; o < GSP; o <<= 1) dd += __shfl_xor(dd, o);
    const float lse2 = lse[static_cast<int64_t>(h) * B + b] * kLog2e;
    const char* kb = static_cast<const char*>(kp) + hoff * ES;
    const char* vb = static_cast<const char*>(vp) + hoff * ES;
    char* dkb = static_cast<char*>(dkp) + hoff * ES;
    char* dvb = static_cast<char*>(dvp) + hoff * ES;
    const int64_t rs = ld * ES;  // bytes between rows of K, V, dK, dV
    for (int j0 = c0 + slot; j0 < c1; j0 += U * KS) {
      Chunk xk[U], xv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {  // rows past the sequence re-read its last row and are not stored
        const int j = min(j0 + u * KS, c1 - 1);
        if (live) {
          xk[u] = *reinterpret_cast<const Chunk*>(kb + j * rs);
          xv[u] = *reinterpret_cast<const Chunk*>(vb + j * rs);
        } else {
          __builtin_memset(&xk[u], 0, sizeof(Chunk));
          __builtin_memset(&xv[u], 0, sizeof(Chunk));
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * KS;
        float kv[EPC], vv[EPC];
        widen(xk[u], kv);
        widen(xv[u], vv);
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          s = fmaf(qv[e], kv[e], s);
          dp = fmaf(dov[e], vv[e], dp);
        }
#pragma unroll
        for (int o = 1; o < GSP; o <<= 1) {
          s += __shfl_xor(s, o);
          dp += __shfl_xor(dp, o);
        }
        if (j < c1 && live) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s, c, -lse2));
          const float ds = p * (dp - dd);
          float dk[EPC], dv[EPC];
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            dk[e] = scale * ds * qv[e];
            dv[e] = p * dov[e];
            dq[e] = fmaf(ds, kv[e], dq[e]);
          }
          *reinterpret_cast<Chunk*>(dkb + j * rs) = narrow(dk);
          *reinterpret_cast<Chunk*>(dvb + j * rs) = narrow(dv);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) sq[tid * EPC + e] = dq[e];
  __syncthreads();
  if (slot == 0 && h < H && live) {
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    for (int s2 = 0; s2 < KS; ++s2) {
      const int t2 = s2 * CPR + cidx;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += sq[t2 * EPC + e];
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] *= scale;
    const int64_t off = (static_cast<int64_t>(b) * H + h) * D + sub * EPC;
    *reinterpret_cast<Chunk*>(static_cast<char*>(dqp) + off * ES) = narrow(acc);
  }
}

template <typename Et, int D>
hipError_t bwd_first_dispatch(const void* dof, const void* qf, const void* k, const void* v, const void* of,
                              const float* lse, const int32_t* cu, int32_t B, int32_t N, int32_t H,
                              int32_t max_seq_len, int64_t ld, float scale, void* dq, void* dk, void* dv,
                              hipStream_t stream) {
  constexpr int GS = pow2_ceil(D / (kIs16<Et> ? 8 : 4));  // lanes per head row
  // heads per block: as many as leave the key slots the first-token forward takes
  const int HPB0 = std::max(1, std::min<int>(H, kFbThreads / (GS * first_token_slots(max_seq_len))));
  const int HG = (H + HPB0 - 1) / HPB0;
  const int HPB = (H + HG - 1) / HG;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL((attn_bwd_first_kernel<Et, D>), dim3(B, HG), dim3(kFbThreads), 0, stream, dof, qf, k, v, of,
                     lse, cu, B, N, H, HPB, ld, c, scale, dq, dk, dv);
  timing_stop("attn_bwd_first", ev, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_first(int dt, int D, const void* dout_first, const void* q_first, const void* k,
                                 const void* v, const void* out_first, const float* lse_first, const int32_t* cu,
                                 int32_t B, int32_t N, int32_t H, int32_t max_seq_len, int64_t ld, float scale,
                                 void* dq_first, void* dk, void* dv, hipStream_t stream) {
#define PE_FB_CASE(DD)                                                                                        \
  case DD:                                                                                                   \
    return dt == kDtF32  ? bwd_first_dispatch<float, DD>(dout_first, q_first, k, v, out_first, lse_first, cu, B, N, \
                                                        H, max_seq_len, ld, scale, dq_first, dk, dv, stream)                   \
           : dt == kDtF16 ? bwd_first_dispatch<_Float16, DD>(dout_first, q_first, k, v, out_first, lse_first, cu, B, \
                                                           N, H, max_seq_len, ld, scale, dq_first, dk, dv, stream)             \
                         : bwd_first_dispatch<__bf16, DD>(dout_first, q_first, k, v, out_first, lse_first, cu, B, N, \
                                                         H, max_seq_len, ld, scale, dq_first, dk, dv, stream);
  switch (D) {
    PE_HEAD_DIMS(PE_FB_CASE)
    default: return hipErrorInvalidValue;
  }
#undef PE_FB_CASE
}

}  // namespace pe
