// Flash-style forward of non-causal attention over packed sequences, and the
// first-token query variant.
//
// Work item = one head and one tile of 128 consecutive packed query rows. A
// tile may span several short sequences or sit inside one long document; its
// keys are those of every sequence it touches, and each query row masks keys
// outside its own sequence. Short queries and long documents thus share one
// launch without padding any sequence to a tile.
//
// Each of the 4 waves owns 32 query rows. Per 64-key block staged in LDS:
//   S^T (32 keys x 32 queries) = K Q^T          MFMA, A = K rows from LDS, B = Q in registers
//   online softmax in base 2 (scale*log2(e) folded into one FMA)
//   O^T (d x 32 queries) += V^T P^T             MFMA, B = P straight from the S^T accumulators
// Computing S transposed leaves every lane with one query and 16 of its keys,
// the layout the PV product needs as its B operand, so P never goes through
// LDS. The order of the reduction index of an MFMA is free as long as A and B
// agree, which lets V^T be read in the order the S^T accumulators hold keys.
#include <climits>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pe {

namespace {

constexpr int BM = kAttnTileRows;  // query rows per block
constexpr int BN = 64;             // keys per LDS stage
constexpr int NT = 256;            // 4 waves

template <bool BF, int D>
struct Shape {
  static constexpr int ES = BF ? 2 : 4;
  static constexpr int ROWB = D * ES;           // bytes of one head row
  static constexpr int CH = ROWB / 16;          // 16-byte chunks per head row
  static constexpr int EPC = 16 / ES;           // elements per chunk
  static constexpr int KST = BF ? D + 8 : D + 4;    // K tile: [BN][KST]
  static constexpr int VST = BF ? BN + 8 : D + 8;   // bf16: V^T tile [D][VST]; fp32: V tile [BN][VST]
  static constexpr int KSZ = BN * KST;
  static constexpr int VSZ = BF ? D * VST : BN * VST;
  static constexpr int HALF = D / 2;            // head-dim elements per lane half
  static constexpr int QS = BF ? (HALF + 7) / 8 : HALF;  // MFMA steps of S
  static constexpr int DB = (D + 31) / 32;      // 32-row blocks of O^T
  static constexpr int TOTCH = BN * CH;
  static constexpr int PER = (TOTCH + NT - 1) / NT;
};

// Position of key r (0..63) inside the bf16 V^T tile: within every 16 keys
// the middle two quads swap, matching the key order of the S^T accumulators.
__device__ __forceinline__ int vt_pos(int r) {
  return (r & ~15) | (((r >> 2) & 1) << 3) | (((r >> 3) & 1) << 2) | (r & 3);
}

template <bool BF>
struct QReg;
template <>
struct QReg<true> { using T = bf16x8; };
template <>
struct QReg<false> { using T = float; };

__device__ __forceinline__ bf16x8 u16x8_as_bf16(u16x8 x) { return __builtin_bit_cast(bf16x8, x); }

template <bool BF, int D>
__device__ __forceinline__ void load_q(const void* qp, int64_t off, bool valid,
                                       typename QReg<BF>::T (&q)[Shape<BF, D>::QS]) {
  using Sh = Shape<BF, D>;
  if constexpr (BF) {
    const uint16_t* src = static_cast<const uint16_t*>(qp) + off;
#pragma unroll
    for (int s = 0; s < Sh::QS; ++s) {
      u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
      if (valid) {
        if constexpr (Sh::HALF >= 8) {
          x = *reinterpret_cast<const u16x8*>(src + 8 * s);
        } else {
#pragma unroll
          for (int j = 0; j < Sh::HALF; ++j) x[j] = src[j];
        }
      }
      q[s] = u16x8_as_bf16(x);
    }
  } else {
    const float* src = static_cast<const float*>(qp) + off;
#pragma unroll
    for (int s = 0; s < Sh::QS; ++s) q[s] = valid ? src[s] : 0.f;
  }
}

template <bool BF, int D>
__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(
    const void* __restrict__ qp, const void* __restrict__ kp, const void* __restrict__ vp,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N,
    int32_t H, int32_t T, float c, void* __restrict__ op, float* __restrict__ lse) {
  using Sh = Shape<BF, D>;
  using E = typename std::conditional<BF, uint16_t, float>::type;
  __shared__ __align__(16) E kl[2][Sh::KSZ];
  __shared__ __align__(16) E vl[2][Sh::VSZ];
  __shared__ int32_t cul[BM + 2];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lin / T, t = lin - h * T;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, ql = lane & 31, g = lane >> 5;

  // ---- the sequences this tile touches and the key range they span
  const int r0 = t * BM, rend = min(r0 + BM, N);
  const int blo = items[t], nxt = items[t + 1];
  const int bhi = nxt >= B ? B - 1 : (cu[nxt] == rend ? nxt - 1 : nxt);
  // at most BM + 1 sequences touch BM rows when every length is >= 1; the
  // clamp keeps LDS writes in bounds even for malformed offsets
  const int ncu = min(bhi - blo + 2, BM + 2);
  for (int i = tid; i < ncu; i += NT) cul[i] = cu[blo + i];
  __syncthreads();
  const int kb0 = cul[0], kb1 = cul[ncu - 1];

  // ---- this lane's query row and its own key range [qk0, qk1)
  const int qrow = r0 + wv * 32 + ql;
  const bool qvalid = qrow < rend;
  int qk0 = 0, qk1 = 0;
  if (qvalid) {
    int lo = 0, hi = ncu - 2;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cul[mid] <= qrow) lo = mid; else hi = mid - 1;
    }
    qk0 = cul[lo];
    qk1 = cul[lo + 1];
  }
  const int wk0 = wave_min_i(qvalid ? qk0 : INT_MAX);  // keys any row of the wave needs
  const int wk1 = wave_max_i(qvalid ? qk1 : INT_MIN);
  const int mk0 = wave_max_i(qvalid ? qk0 : INT_MIN);  // keys every row of the wave needs
  const int mk1 = wave_min_i(qvalid ? qk1 : INT_MAX);

  typename QReg<BF>::T qr[Sh::QS];
  load_q<BF, D>(qp, (static_cast<int64_t>(qrow) * H + h) * D + g * Sh::HALF, qvalid, qr);

  // ---- K/V staging: global -> registers (prefetch) -> LDS
  uint4 kr[Sh::PER], vr[Sh::PER];
  const char* kbase = static_cast<const char*>(kp);
  const char* vbase = static_cast<const char*>(vp);
  auto gload = [&](int kb) {
#pragma unroll
    for (int p = 0; p < Sh::PER; ++p) {
      const int ch = tid + p * NT;
      const int row = ch / Sh::CH, col = ch - row * Sh::CH;
      const int key = kb + row;
      if ((Sh::TOTCH % NT == 0 || ch < Sh::TOTCH) && key < kb1) {
        const int64_t off = (static_cast<int64_t>(key) * H + h) * Sh::ROWB + col * 16;
        kr[p] = *reinterpret_cast<const uint4*>(kbase + off);
        vr[p] = *reinterpret_cast<const uint4*>(vbase + off);
      } else {
        kr[p] = make_uint4(0, 0, 0, 0);
        vr[p] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int p = 0; p < Sh::PER; ++p) {
      const int ch = tid + p * NT;
      if (Sh::TOTCH % NT == 0 || ch < Sh::TOTCH) {
        const int row = ch / Sh::CH, col = ch - row * Sh::CH;
        *reinterpret_cast<uint4*>(&kl[buf][row * Sh::KST + col * Sh::EPC]) = kr[p];
        if constexpr (BF) {
          const u16x8 x = __builtin_bit_cast(u16x8, vr[p]);
          const int kpos = vt_pos(row);
#pragma unroll
          for (int i = 0; i < 8; ++i) vl[buf][(col * 8 + i) * Sh::VST + kpos] = x[i];
        } else {
          *reinterpret_cast<uint4*>(&vl[buf][row * Sh::VST + col * 4]) = vr[p];
        }
      }
    }
  };

  floatx16 o[Sh::DB];
#pragma unroll
  for (int db = 0; db < Sh::DB; ++db) o[db] = floatx16{};
  float m = kNegBig, l = 0.f;

  int buf = 0;
  if (kb0 < kb1) gload(kb0);
  for (int kb = kb0; kb < kb1; kb += BN) {
    swrite(buf);
    __syncthreads();
    if (kb + BN < kb1) gload(kb + BN);
    if (kb < wk1 && kb + BN > wk0) {
      const E* K = kl[buf];
      const E* V = vl[buf];
      floatx16 s[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        s[kk] = floatx16{};
        const E* krow = K + (kk * 32 + ql) * Sh::KST + g * Sh::HALF;
#pragma unroll
        for (int st = 0; st < Sh::QS; ++st) {
          if constexpr (BF) {
            u16x8 a;
            if constexpr (Sh::HALF >= 8) {
              a = *reinterpret_cast<const u16x8*>(krow + 8 * st);
            } else {
              a = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
              for (int j = 0; j < Sh::HALF; ++j) a[j] = krow[j];
            }
            s[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(u16x8_as_bf16(a), qr[st], s[kk], 0, 0, 0);
          } else {
            s[kk] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[st], qr[st], s[kk], 0, 0, 0);
          }
        }
      }
      // keys outside the lane's own sequence
      if (!(kb >= mk0 && kb + BN <= mk1)) {
        const int lo = qk0 - kb - 4 * g, hi = qk1 - kb - 4 * g;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kidx = 32 * kk + 8 * (i >> 2) + (i & 3);
            if (kidx < lo || kidx >= hi) s[kk][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kk][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m, mx * c);
      if (__any(mnew > m)) {
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < Sh::DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        m = mnew;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kk][i], c, -m));
          s[kk][i] = p;
          l += p;
        }
      // O^T += V^T P^T
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if constexpr (BF) {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            bf16x8 pb;
#pragma unroll
            for (int j = 0; j < 8; ++j) pb[j] = static_cast<__bf16>(s[kk][8 * st + j]);
#pragma unroll
            for (int db = 0; db < Sh::DB; ++db) {
              const int d = db * 32 + ql;
              u16x8 a = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
              if (D % 32 == 0 || d < D)
                a = *reinterpret_cast<const u16x8*>(V + d * Sh::VST + 32 * kk + 16 * st + 8 * g);
              o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(u16x8_as_bf16(a), pb, o[db], 0, 0, 0);
            }
          }
        } else {
#pragma unroll
          for (int st = 0; st < 16; ++st) {
            const int krow = 32 * kk + 8 * (st >> 2) + 4 * g + (st & 3);
#pragma unroll
            for (int db = 0; db < Sh::DB; ++db) {
              const int d = db * 32 + ql;
              const float a = (D % 32 == 0 || d < D) ? V[krow * Sh::VST + d] : 0.f;
              o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kk][st], o[db], 0, 0, 0);
            }
          }
        }
      }
    }
    buf ^= 1;
  }

  // ---- normalise and store
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qvalid) {
    const int64_t obase = (static_cast<int64_t>(qrow) * H + h) * D;
#pragma unroll
    for (int db = 0; db < Sh::DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = db * 32 + 8 * i4 + 4 * g;
        if (d0 < D) {
          if constexpr (BF) {
            uint16_t* O = static_cast<uint16_t*>(op) + obase + d0;
            const uint32_t lo = f32_to_bf16(o[db][4 * i4 + 0] * inv) | (uint32_t(f32_to_bf16(o[db][4 * i4 + 1] * inv)) << 16);
            const uint32_t hi = f32_to_bf16(o[db][4 * i4 + 2] * inv) | (uint32_t(f32_to_bf16(o[db][4 * i4 + 3] * inv)) << 16);
            *reinterpret_cast<uint2*>(O) = make_uint2(lo, hi);
          } else {
            float* O = static_cast<float*>(op) + obase + d0;
            *reinterpret_cast<float4*>(O) = make_float4(o[db][4 * i4 + 0] * inv, o[db][4 * i4 + 1] * inv,
                                                        o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv);
          }
        }
      }
    if (lse != nullptr && g == 0) lse[static_cast<int64_t>(h) * N + qrow] = (m + log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------- first-token query
// One block per (sequence, group of heads). Threads are laid out as
// [key slot][head][16-byte chunk of the head row]: every K and V row of the
// sequence (all heads of the group) is read once, fully coalesced, and each
// key slot keeps its own running max, sum and output; slots merge at the end.
template <bool BF, int D>
__global__ __launch_bounds__(256) void attn_fwd_first_kernel(
    const void* __restrict__ qf, const void* __restrict__ kp, const void* __restrict__ vp,
    const int32_t* __restrict__ cu, int32_t B, int32_t N, int32_t H, int32_t HPB, float c,
    void* __restrict__ outp, float* __restrict__ lse) {
  constexpr int ES = BF ? 2 : 4;
  constexpr int EPC = 16 / ES;       // elements per 16-byte chunk
  constexpr int GS = D / EPC;        // chunks (threads) per head row
  __shared__ float sm[256], sl[256];
  __shared__ float so[256 * EPC];

  const int b = blockIdx.x;
  const int hg = blockIdx.y;
  const int tid = threadIdx.x;
  const int CPR = HPB * GS;
  const int KS = 256 / CPR;
  const int slot = tid / CPR, cidx = tid - slot * CPR;
  const int hl = cidx / GS, sub = cidx - hl * GS;
  const int h = hg * HPB + hl;
  const bool active = slot < KS && h < H;

  const int c0 = cu[b], c1 = cu[b + 1];
  float qv[EPC], ov[EPC];
  float m = kNegBig, l = 0.f;
#pragma unroll
  for (int e = 0; e < EPC; ++e) ov[e] = 0.f;
  if (active) {
    const int64_t off = (static_cast<int64_t>(b) * H + h) * D + sub * EPC;
    if constexpr (BF) {
      const u16x8 x = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(qf) + off);
#pragma unroll
      for (int e = 0; e < EPC; ++e) qv[e] = bf16_to_f32(x[e]);
    } else {
      const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(qf) + off);
      qv[0] = x.x; qv[1] = x.y; qv[2] = x.z; qv[3] = x.w;
    }
    for (int j = c0 + slot; j < c1; j += KS) {
      const int64_t koff = (static_cast<int64_t>(j) * H + h) * D + sub * EPC;
      float kv[EPC], vv[EPC];
      if constexpr (BF) {
        const u16x8 xk = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(kp) + koff);
        const u16x8 xv = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(vp) + koff);
#pragma unroll
        for (int e = 0; e < EPC; ++e) { kv[e] = bf16_to_f32(xk[e]); vv[e] = bf16_to_f32(xv[e]); }
      } else {
        const float4 xk = *reinterpret_cast<const float4*>(static_cast<const float*>(kp) + koff);
        const float4 xv = *reinterpret_cast<const float4*>(static_cast<const float*>(vp) + koff);
        kv[0] = xk.x; kv[1] = xk.y; kv[2] = xk.z; kv[3] = xk.w;
        vv[0] = xv.x; vv[1] = xv.y; vv[2] = xv.z; vv[3] = xv.w;
      }
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) s = fmaf(qv[e], kv[e], s);
#pragma unroll
      for (int o = 1; o < GS; o <<= 1) s += __shfl_xor(s, o);
      const float x = s * c;
      const float mnew = fmaxf(m, x);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      const float p = __builtin_amdgcn_exp2f(x - mnew);
      l = fmaf(l, alpha, p);
#pragma unroll
      for (int e = 0; e < EPC; ++e) ov[e] = fmaf(ov[e], alpha, p * vv[e]);
      m = mnew;
    }
  }
  sm[tid] = m;
  sl[tid] = l;
#pragma unroll
  for (int e = 0; e < EPC; ++e) so[tid * EPC + e] = ov[e];
  __syncthreads();
  if (slot == 0 && h < H) {
    float M = kNegBig;
    for (int s2 = 0; s2 < KS; ++s2) M = fmaxf(M, sm[s2 * CPR + cidx]);
    float L = 0.f, acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    for (int s2 = 0; s2 < KS; ++s2) {
      const int t2 = s2 * CPR + cidx;
      const float w = __builtin_amdgcn_exp2f(sm[t2] - M);
      L = fmaf(sl[t2], w, L);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] = fmaf(so[t2 * EPC + e], w, acc[e]);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int64_t off = (static_cast<int64_t>(b) * H + h) * D + sub * EPC;
    if constexpr (BF) {
      u16x8 y;
#pragma unroll
      for (int e = 0; e < EPC; ++e) y[e] = f32_to_bf16(acc[e] * inv);
      *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(outp) + off) = y;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(outp) + off) =
          make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    }
    if (lse != nullptr && sub == 0) lse[static_cast<int64_t>(h) * B + b] = (M + log2f(L)) * kLn2;
  }
}

template <bool BF, int D>
hipError_t fwd_dispatch(const void* q, const void* k, const void* v, const int32_t* cu,
                        const int32_t* items, int32_t B, int32_t N, int32_t H, float scale, void* out,
                        float* lse, hipStream_t stream) {
  const int T = (N + BM - 1) / BM;
  const int64_t blocks = static_cast<int64_t>(T) * H;
  if (blocks == 0) return hipSuccess;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipLaunchKernelGGL((attn_fwd_kernel<BF, D>), dim3(static_cast<unsigned>(blocks)), dim3(NT), 0, stream,
                     q, k, v, cu, items, B, N, H, T, c, out, lse);
  return hipGetLastError();
}

template <bool BF, int D>
hipError_t first_dispatch(const void* q, const void* k, const void* v, const int32_t* cu, int32_t B,
                          int32_t N, int32_t H, float scale, void* out, float* lse, hipStream_t stream) {
  constexpr int GS = D / (BF ? 8 : 4);
  const int HPB = (H * GS <= 256) ? H : 256 / GS;
  const int HG = (H + HPB - 1) / HPB;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipLaunchKernelGGL((attn_fwd_first_kernel<BF, D>), dim3(B, HG), dim3(256), 0, stream, q, k, v, cu, B,
                     N, H, HPB, c, out, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(bool bf16, int D, const void* q, const void* k, const void* v,
                           const int32_t* cu, const int32_t* items, int32_t B, int32_t N, int32_t H,
                           float scale, void* out, float* lse, hipStream_t stream) {
#define PE_FWD_CASE(DD)                                                                      \
  case DD:                                                                                  \
    return bf16 ? fwd_dispatch<true, DD>(q, k, v, cu, items, B, N, H, scale, out, lse, stream) \
                : fwd_dispatch<false, DD>(q, k, v, cu, items, B, N, H, scale, out, lse, stream);
  switch (D) {
    PE_FWD_CASE(8)
    PE_FWD_CASE(16)
    PE_FWD_CASE(32)
    PE_FWD_CASE(64)
    PE_FWD_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef PE_FWD_CASE
}

hipError_t launch_attn_fwd_first(bool bf16, int D, const void* q_first, const void* k, const void* v,
                                 const int32_t* cu, int32_t B, int32_t N, int32_t H, float scale,
                                 void* out_first, float* lse_first, hipStream_t stream) {
#define PE_FIRST_CASE(DD)                                                                          \
  case DD:                                                                                        \
    return bf16 ? first_dispatch<true, DD>(q_first, k, v, cu, B, N, H, scale, out_first, lse_first, stream) \
                : first_dispatch<false, DD>(q_first, k, v, cu, B, N, H, scale, out_first, lse_first, stream);
  switch (D) {
    PE_FIRST_CASE(8)
    PE_FIRST_CASE(16)
    PE_FIRST_CASE(32)
    PE_FIRST_CASE(64)
    PE_FIRST_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef PE_FIRST_CASE
}

}  // namespace pe
