// bf16 forward for head dims 32, 64 and 128, the long-sequence workhorse.
//
// Same work items and MFMA formulation as the generic forward (a head and 128
// consecutive packed query rows per block, 32 rows per wave, S^T = K Q^T and
// O^T += V^T P^T with P straight from the accumulators), rebuilt for gfx950:
//   * K and V tiles of 64 keys travel global -> LDS by LDS DMA
//     (global_load_lds_dwordx4) into a ring of 4 stages, three blocks ahead of
//     the softmax, with no registers or VALU spent on staging: each lane's
//     source offset is fixed and only the scalar base moves;
//   * tiles are unpadded with XOR-swizzled 16-byte chunks (attn_common.h);
//   * software pipeline inside each wave: the S MFMAs of block j+1 are issued
//     before the softmax of block j, so the exponentials and conversions run
//     on the VALU while the matrix core computes;
//   * the loop is unrolled over the ring, so every LDS read has an immediate
//     offset from a handful of per-lane base addresses.
#include <climits>

#include "attn_common.h"

namespace pe {

namespace {

constexpr int kStages = 4;

template <int ST>
struct StageTag {
  static constexpr int value = ST;
};

template <typename Et, int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const void* __restrict__ qp, const void* __restrict__ kp, const void* __restrict__ vp,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N, int32_t H,
    int32_t T, int32_t win, int64_t ld, float c, void* __restrict__ op, float* __restrict__ lse) {
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int TB = kBlk * D * 2;    // bytes per tile
  constexpr int QS = D / 16;          // MFMA steps over head_dim
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int NL = dma_per_tile<D>();  // DMA instructions per thread per tile
  __shared__ __align__(16) char ring[kStages][2][TB];  // [stage][K, V][tile]
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
  // keys of the tile: those of its sequences, and within win of its rows for local attention
  const int klo = __builtin_amdgcn_readfirstlane(win >= 0 ? max(sp.lo, sp.r0 - win) : sp.lo);
  const int khi = __builtin_amdgcn_readfirstlane(win >= 0 ? min(sp.hi, sp.rend + win) : sp.hi);

  vec8<Et> qr[QS];
  load_row_regs<Et, D>(qp, static_cast<int64_t>(qrow) * ld + h * D, g, qvalid, qr);
  // Retire the Q loads with a wait the compiler sees: otherwise it places a
  // vmcnt wait for them inside the loop, which would also drain the DMA ring.
  vmem_fence_for_compiler();

  // ---- DMA: per-lane source offsets relative to the block's first row
  const int64_t rowstride = ld * 2;  // bytes between packed K/V rows
  uint32_t doff[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int slot = j * kThreads + wv * 64 + lane;
    const int r = slot / CH, pc = slot - r * CH;
    doff[j] = static_cast<uint32_t>(r * rowstride + h * D * 2 + (pc ^ (swz(r) & (CH - 1))) * 16);
  }
  const char* kbase = static_cast<const char*>(kp);
  const char* vbase = static_cast<const char*>(vp);
  const int nblk = (khi - klo + kBlk - 1) / kBlk;
  auto issue = [&](int blk, int st) __attribute__((always_inline)) {
    const int row0 = klo + blk * kBlk;
    const bool full = row0 + kBlk <= khi;
    const char* kb = kbase + static_cast<int64_t>(row0) * rowstride;
    const char* vb = vbase + static_cast<int64_t>(row0) * rowstride;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      uint32_t off = doff[j];
      if (!full) {  // rows past the range repeat the last row (masked keys, valid memory)
        const int slot = j * kThreads + wv * 64 + lane;
        const int rr = slot / CH, pc = slot - rr * CH;
        const int r = min(rr, khi - 1 - row0);
        off = static_cast<uint32_t>(r * rowstride + h * D * 2 + (pc ^ (swz(rr) & (CH - 1))) * 16);
      }
      const uint32_t slotb = static_cast<uint32_t>((j * kThreads + wv * 64) * 16);
      dma16(lds_addr(ring[st][0]) + slotb, kb, off);
      dma16(lds_addr(ring[st][1]) + slotb, vb, off);
    }
  };

  // ---- per-lane LDS read offsets (bytes within a tile)
  int koff[2][QS];  // K operand: row 32*kk + ql, logical chunk g*(CH/2)+st
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int st = 0; st < QS; ++st) koff[kk][st] = chunk_off<CH>(32 * kk + ql, g * (CH / 2) + st);
  const int sub = lane & 15, grp = (lane >> 4) & 1;
  int voff[2][2][2][DB];  // V^T operand: [kk][s][hi][db], row 32kk+16s+4g+sub/4 (+8 for hi)
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int rowa = 32 * kk + 16 * s + 4 * g + (sub >> 2) + 8 * hi;
          const int cc = 4 * db + 2 * grp + ((sub >> 1) & 1);
          voff[kk][s][hi][db] = chunk_off<CH>(rowa, cc) + 8 * (sub & 1);
        }

  auto qk = [&](const char* ktile, floatx16 (&s)[2]) __attribute__((always_inline)) {
    vec8<Et> ka[2][QS];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int st = 0; st < QS; ++st)
        ka[kk][st] = as_vec8<Et>(*reinterpret_cast<const u16x8*>(ktile + koff[kk][st]));
    s[0] = floatx16{};
    s[1] = floatx16{};
#pragma unroll
    for (int st = 0; st < QS; ++st)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        s[kk] = mfma16<Et>(ka[kk][st], qr[st], s[kk]);
  };

  floatx16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = floatx16{};
  float m = kNegBig, l = 0.f;

  auto softmax_pv = [&](floatx16 (&s)[2], int kb, const char* vtile) __attribute__((always_inline)) {
    if (!(kb >= mk0 && kb + kBlk <= mk1)) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int base = kb + 32 * kk + 4 * g;
        mask_block(s[kk], qk0 - base, qk1 - base);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i2 = 0; i2 < 16; ++i2) mx = fmaxf(mx, s[kk][i2]);
    mx = xhalf_max(mx);
    const float mnew = fmaxf(m, mx * c);
    if (__any(mnew > m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) o[db][i2] *= alpha;
      m = mnew;
    }
    vec8<Et> pb[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i2 = 0; i2 < 16; ++i2) s[kk][i2] = __builtin_amdgcn_exp2f(fmaf(s[kk][i2], c, -m));
      probs_to_h16<Et>(s[kk], pb[kk], l);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u16x4 lo4 = ds_read_tr16(reinterpret_cast<const uint16_t*>(vtile + voff[kk][s2][0][db]));
          const u16x4 hi4 = ds_read_tr16(reinterpret_cast<const uint16_t*>(vtile + voff[kk][s2][1][db]));
          const u16x8 a = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          o[db] = mfma16<Et>(as_vec8<Et>(a), pb[kk][s2], o[db]);
        }
  };

  auto wave_needs = [&](int blk) __attribute__((always_inline)) {
    const int kb = klo + blk * kBlk;
    return kb < wk1 && kb + kBlk > wk0;
  };

  // ---- prologue: blocks 0..2 in flight, S of block 0
  floatx16 sa[2], sb[2];  // S of the current and the next block, alternating roles
  if (nblk > 0) issue(0, 0);
  if (nblk > 1) issue(1, 1);
  if (nblk > 2) issue(2, 2);
  if (nblk > 0) {
    if (nblk > 2) wait_vmcnt<4 * NL>();
    else if (nblk > 1) wait_vmcnt<2 * NL>();
    else wait_vmcnt<0>();
    raw_barrier();
    if (wave_needs(0)) qk(ring[0][0], sa);
  }

  // iteration j reads K of block j+1 and V of block j; block b lives in stage b % 4
  auto step = [&](auto tag, int j, floatx16 (&scur)[2], floatx16 (&snext)[2]) __attribute__((always_inline)) {
    constexpr int STJ = decltype(tag)::value;   // stage of block j
    constexpr int STN = (STJ + 1) % kStages;    // stage of block j+1
    constexpr int STF = (STJ + 3) % kStages;    // stage receiving block j+3
    if (j + 1 < nblk) {
      if (j + 2 < nblk) wait_vmcnt<2 * NL>(); else wait_vmcnt<0>();  // block j+1 landed
    }
    raw_barrier();  // block j+1 visible to all; the stage of block j-1 is no longer read
    if (j + 3 < nblk) issue(j + 3, STF);
    if (j + 1 < nblk && wave_needs(j + 1)) qk(ring[STN][0], snext);
    if (wave_needs(j)) softmax_pv(scur, klo + j * kBlk, ring[STJ][1]);
  };
  for (int j = 0; j < nblk; j += kStages) {
    step(StageTag<0>{}, j, sa, sb);
    if (j + 1 < nblk) step(StageTag<1>{}, j + 1, sb, sa);
    if (j + 2 < nblk) step(StageTag<2>{}, j + 2, sa, sb);
    if (j + 3 < nblk) step(StageTag<3>{}, j + 3, sb, sa);
  }

  const float lt = xhalf_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qvalid) {
    store_acc_row<Et, D>(op, (static_cast<int64_t>(qrow) * H + h) * D, o, inv, g);
    if (lse != nullptr && g == 0) lse[static_cast<int64_t>(h) * N + qrow] = (m + log2f(lt)) * kLn2;
  }
}

template <typename Et, int D>
hipError_t dispatch(const void* q, const void* k, const void* v, const int32_t* cu, const int32_t* items,
                    int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* out, float* lse,
                    hipStream_t stream) {
  const int T = (N + kAttnTileRows - 1) / kAttnTileRows;
  const int64_t blocks = static_cast<int64_t>(T) * H;
  if (blocks == 0) return hipSuccess;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<Et, D>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, q,
                     k, v, cu, items, B, N, H, T, win, ld, c, out, lse);
  timing_stop("attn_fwd", ev, stream);
  return hipGetLastError();
}

}  // namespace

// The LDS-DMA pipeline pays off once sequences span several 64-key blocks; for
// batches whose length bound is at most two blocks the generic kernel's
// shorter prologue wins.
bool attn_fwd_bf16_supported(int D, int max_seq_len) {
  return (D == 32 || D == 64 || D == 128) && max_seq_len > 2 * kBlk;
}

template <typename Et>
hipError_t launch_typed(int D, const void* q, const void* k, const void* v, const int32_t* cu, const int32_t* items,
                        int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* out, float* lse,
                        hipStream_t stream) {
  switch (D) {
    case 32: return dispatch<Et, 32>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream);
    case 64: return dispatch<Et, 64>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream);
    case 128: return dispatch<Et, 128>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_fwd_bf16(bool f16, int D, const void* q, const void* k, const void* v, const int32_t* cu,
                                const int32_t* items, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld,
                                float scale, void* out, float* lse, hipStream_t stream) {
  return f16 ? launch_typed<_Float16>(D, q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream)
             : launch_typed<__bf16>(D, q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream);
}

}  // namespace pe
