// 16-bit forward for batches of short sequences (every length at most 64) at head
// dims 32 and 64: one wave per (sequence, head), four independent waves per
// workgroup, no work list.
//
// A sequence of L <= 64 rows is one or two 32-row blocks of queries and of keys. The
// wave loads its K and Q rows straight into MFMA operand registers (the lane's own
// row, the layout the other forwards keep Q in) and its V rows by LDS DMA into a
// private XOR-swizzled tile, from which V^T is read with ds_read_b64_tr_b16. Then,
// per query block: S^T = K Q^T for every key block, the row's exact maximum over all
// its keys (keys past the sequence, or outside a window, masked), p = exp2(c s - m),
// the row sum, and O^T = V^T P^T with P straight from the accumulators; O and the LSE
// are written once. Every byte of Q, K, V and O crosses HBM once, with all of a
// wave's loads in flight together, where the packed 128-row tiles read again the keys
// of every sequence that straddles two tiles.
#include <climits>

#include "attn_common.h"

namespace pe {

namespace {

constexpr int kShortWaves = 4;  // independent waves per workgroup
constexpr int kShortMaxLen = 64;

// NB: 32-row blocks of the sequence (1 or 2), wave-uniform
template <typename Et, int D, int NB>
__device__ __forceinline__ void short_seq(const void* __restrict__ qp, const void* __restrict__ kp,
                                          const void* __restrict__ vp, int h, int lo, int hi, int32_t N, int32_t H,
                                          int32_t win, int64_t ld, float c, void* __restrict__ op,
                                          float* __restrict__ lse, char (*vt)[32 * D * 2]) {
  using G = Geo<Et, D>;
  constexpr int CH = D / 8;   // 16-byte chunks per row
  constexpr int QS = G::QS;   // MFMA steps over head_dim
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int NL = 32 * CH / 64;  // DMA instructions per 32-row tile
  const int lane = threadIdx.x & 63, ql = lane & 31, g = lane >> 5;
  const int64_t rowstride = ld * 2;  // bytes between packed rows

  // V rows -> the wave's LDS tiles (rows past the sequence repeat its last row: keys
  // that get no weight, read from valid memory)
  const char* vbase = static_cast<const char*>(vp) + static_cast<int64_t>(lo) * rowstride;
  const uint32_t vt0 = lds_addr(vt[0]);
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int slot = j * 64 + lane;
      const int r = slot / CH, pc = slot - r * CH;
      const int rr = min(32 * kb + r, hi - lo - 1);
      const uint32_t off = static_cast<uint32_t>(rr * rowstride + h * D * 2 + (pc ^ (swz(r) & (CH - 1))) * 16);
      dma16(vt0 + static_cast<uint32_t>(kb * 32 * D * 2 + j * 1024), vbase, off);
    }
  // K and Q rows as operands (rows past the sequence read as zero)
  vec8<Et> kr[NB][QS], qr[NB][QS];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int row = lo + 32 * b + ql;
    const int64_t off = static_cast<int64_t>(row) * ld + h * D;
    load_row_regs<Et, D>(kp, off, g, row < hi, kr[b]);
    load_row_regs<Et, D>(qp, off, g, row < hi, qr[b]);
  }
  wait_vmcnt<0>();  // the V tiles have landed (this wave alone reads them)

  // V^T operand of step s2: rows 16 s2 + 4 g + sub/4 (+8 for hh = 1) of the tile
  const int sub = lane & 15, grp = (lane >> 4) & 1;
  int voff[2][DB];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      voff[hh][db] = chunk_off<CH>(4 * g + (sub >> 2) + 8 * hh, 4 * db + 2 * grp + ((sub >> 1) & 1)) + 8 * (sub & 1);

#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    const int qrow = lo + 32 * qb + ql;
    floatx16 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      s[kb] = mfma16<Et>(kr[kb][0], qr[qb][0], floatx16{});
#pragma unroll
      for (int q = 1; q < QS; ++q) s[kb] = mfma16<Et>(kr[kb][q], qr[qb][q], s[kb]);
    }
    // keys past the sequence, and with a window keys farther than win from the query
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      const int k0 = lo + 32 * kb + 4 * g;  // key of register 0
      if (win >= 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 8 * (i >> 2) + (i & 3);
          if (key >= hi || key < qrow - win || key > qrow + win) s[kb][i] = -INFINITY;
        }
      } else if (kb == NB - 1) {
        mask_block(s[kb], -INT_MAX, hi - k0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = xhalf_max(mx);
    // (a row past the sequence may see no key through a window; it is not stored)
    const float m = mx == -INFINITY ? 0.f : mx * c;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        s[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c, -m));
        s[kb][i + 1] = __builtin_amdgcn_exp2f(fmaf(s[kb][i + 1], c, -m));
        a0 += s[kb][i];
        a1 += s[kb][i + 1];
      }
    const float lt = xhalf_sum(a0 + a1);

    floatx16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = floatx16{};
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      vec8<Et> pb[2];
      acc_to_h16<Et>(s[kb], pb);
      const uint32_t tile = vt0 + static_cast<uint32_t>(kb * 32 * D * 2);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u16x4 lo4 = ds_read_tr16_at(tile + s2 * (16 * CH * 16) + voff[0][db]);
          const u16x4 hi4 = ds_read_tr16_at(tile + s2 * (16 * CH * 16) + voff[1][db]);
          const vec8<Et> va = as_vec8<Et>(u16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]});
          o[db] = mfma16<Et>(va, pb[s2], o[db]);
        }
    }
    if (qrow < hi) {  // the same for both lane halves, which store together
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      store_acc_row<Et, D>(op, (static_cast<int64_t>(qrow) * H + h) * D, o, inv, g);
      if (lse != nullptr && g == 0) lse[static_cast<int64_t>(h) * N + qrow] = (m + log2f(lt)) * kLn2;
    }
  }
}

template <typename Et, int D>
__global__ __launch_bounds__(64 * kShortWaves, 3) void attn_fwd_short_kernel(
    const void* __restrict__ qp, const void* __restrict__ kp, const void* __restrict__ vp,
    const int32_t* __restrict__ cu, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float c,
    void* __restrict__ op, float* __restrict__ lse) {
  __shared__ __align__(16) char vt[kShortWaves][2][32 * D * 2];  // [wave][key block][tile]
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kShortWaves + w;  // (sequence, head), heads fastest
  const int b = static_cast<int>(item / H), h = static_cast<int>(item - static_cast<int64_t>(b) * H);
  if (b >= B) return;
  const int lo = cu[b];
  // a length above the stated bound of 64 is cut to its first 64 rows (rows past them
  // are left as they were), so no access leaves the sequence
  const int hi = min(cu[b + 1], lo + kShortMaxLen);
  if (hi <= lo) return;
  if (hi - lo <= 32) short_seq<Et, D, 1>(qp, kp, vp, h, lo, hi, N, H, win, ld, c, op, lse, vt[w]);
  else short_seq<Et, D, 2>(qp, kp, vp, h, lo, hi, N, H, win, ld, c, op, lse, vt[w]);
}

template <typename Et, int D>
hipError_t dispatch_short(const void* q, const void* k, const void* v, const int32_t* cu, int32_t B, int32_t N,
                          int32_t H, int32_t win, int64_t ld, float scale, void* out, float* lse,
                          hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(B) * H;
  if (items == 0) return hipSuccess;
  const int64_t blocks = (items + kShortWaves - 1) / kShortWaves;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL((attn_fwd_short_kernel<Et, D>), dim3(static_cast<unsigned>(blocks)), dim3(64 * kShortWaves), 0,
                     stream, q, k, v, cu, B, N, H, win, ld, c, out, lse);
  timing_stop("attn_fwd", ev, stream);
  return hipGetLastError();
}

}  // namespace

bool attn_fwd_short_supported(int dt, int D, int max_seq_len) {
  return dt != kDtF32 && (D == 32 || D == 64) && max_seq_len <= kShortMaxLen;
}

hipError_t launch_attn_fwd_short(bool f16, int D, const void* q, const void* k, const void* v, const int32_t* cu,
                                 int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* out,
                                 float* lse, hipStream_t stream) {
  switch (D) {
    case 32:
      return f16 ? dispatch_short<_Float16, 32>(q, k, v, cu, B, N, H, win, ld, scale, out, lse, stream)
                 : dispatch_short<__bf16, 32>(q, k, v, cu, B, N, H, win, ld, scale, out, lse, stream);
    case 64:
      return f16 ? dispatch_short<_Float16, 64>(q, k, v, cu, B, N, H, win, ld, scale, out, lse, stream)
                 : dispatch_short<__bf16, 64>(q, k, v, cu, B, N, H, win, ld, scale, out, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pe
