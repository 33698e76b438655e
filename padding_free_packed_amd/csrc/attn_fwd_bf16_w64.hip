// bf16 forward for head dims 32 and 64 with 64 query rows per wave.
//
// A block takes a head and up to 128 query rows of ONE sequence: slot t of the
// sequence-aligned work list (launch_seq_worklist with tile height 128) belongs
// to the sequence b = items[t] and covers its rows from
// cu[b] + 128 * (t - cu[b] / 128 - b); slots past a sequence's end exit at
// once. Every row of a block then has the same key range, no key block of a
// neighbouring sequence is staged, and only a sequence's last key block needs a
// mask. Blocks are mapped XCD-aware. A block has two waves and each wave owns
// two 32-row query blocks. Every K or V operand a wave reads from LDS
// therefore feeds two MFMAs instead of one: on gfx950 the LDS instruction rate
// (about one wave-wide ds_read per 7 cycles per CU, whatever its width) is
// otherwise the limit of the d=64 attention loop, ahead of the matrix core.
//
//   * K and V tiles of 32 keys travel global -> LDS by LDS DMA into a ring of
//     three stages, two blocks ahead; tiles are unpadded with XOR-swizzled
//     16-byte chunks;
//   * S^T = K Q^T per query block (K rows as A operand, Q^T from registers),
//     then O^T += V^T P^T with P taken straight from the accumulators and V^T
//     read by ds_read_b64_tr_b16;
//   * within a wave the two query blocks interleave: the softmax of block 0
//     runs on the VALU while the S MFMAs of block 1 drain, and the softmax of
//     block 1 while the PV MFMAs of block 0 drain;
//   * the running max only moves when a new score exceeds it by more than 2^8
//     (log2 domain), so the O rescale is rare; probabilities stay below 256,
//     which bf16 and the fp32 sums hold exactly enough, and the result is
//     unchanged because O, l and the log-sum-exp use the same reference.
#include <climits>

#include "attn_common.h"

namespace pe {

namespace {

constexpr int kW64Waves = 2;
constexpr int kW64Threads = 64 * kW64Waves;
constexpr int kW64Keys = 32;    // keys per ring stage
constexpr int kW64Stages = 3;  // 2..6
static_assert(kW64Stages >= 2 && kW64Stages <= 6, "ring stages");
constexpr float kRescaleHeadroom = 8.f;

template <int ST>
struct W64Stage {
  static constexpr int value = ST;
};

template <typename Et, int D>
__global__ __launch_bounds__(kW64Threads) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd_bf16_w64_kernel(
    const void* __restrict__ qp, const void* __restrict__ kp, const void* __restrict__ vp,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N, int32_t H,
    int32_t T, int32_t win, int64_t ld, float c, void* __restrict__ op, float* __restrict__ lse) {
  constexpr int CH = D / 8;                    // 16-byte chunks per row
  constexpr int TB = kW64Keys * D * 2;         // bytes per tile
  constexpr int QS = D / 16;                   // MFMA steps over head_dim
  constexpr int DB = D / 32;                   // 32-row blocks of O^T
  constexpr int NL = kW64Keys * CH / kW64Threads;  // DMA instructions per thread per tile
  static_assert(NL >= 1 && (kW64Keys * CH) % kW64Threads == 0, "whole DMA instructions per tile");
  __shared__ __align__(16) char ring[kW64Stages][2][TB];  // [stage][K, V][tile]

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lin / T, t = lin - h * T;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, ql = lane & 31, g = lane >> 5;

  // sequence-aligned tile: slot t of sequence b covers rows r0 .. r0 + 127 of it
  const int b = items[t];
  if (b >= B) return;  // block-uniform: a slot past the last sequence
  const int lo = cu[b], hi = cu[b + 1];
  const int r0 = lo + (t - (lo / kAttnTileRows + b)) * kAttnTileRows;
  if (r0 >= hi) return;  // block-uniform: an empty slot at the end of the sequence
  const int rend = min(r0 + kAttnTileRows, hi);
  int qrow[2], qk0[2], qk1[2], bk0[2], bk1[2], mk0[2], mk1[2];
  bool qvalid[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qrow[qb] = r0 + wv * 64 + 32 * qb + ql;
    qvalid[qb] = qrow[qb] < rend;
    qk0[qb] = qk1[qb] = 0;
    if (qvalid[qb]) {
      qk0[qb] = lo;
      qk1[qb] = hi;
      band_limit(qrow[qb], win, qk0[qb], qk1[qb]);
    }
    // wave-uniform bounds (scalar registers, so the per-block tests are scalar branches)
    bk0[qb] = __builtin_amdgcn_readfirstlane(wave_min_i(qvalid[qb] ? qk0[qb] : INT_MAX));  // keys it needs
    bk1[qb] = __builtin_amdgcn_readfirstlane(wave_max_i(qvalid[qb] ? qk1[qb] : INT_MIN));
    mk0[qb] = __builtin_amdgcn_readfirstlane(wave_max_i(qvalid[qb] ? qk0[qb] : INT_MIN));  // every lane needs
    mk1[qb] = __builtin_amdgcn_readfirstlane(wave_min_i(qvalid[qb] ? qk1[qb] : INT_MAX));
  }
  // keys of the tile: those of its sequences, and within win of its rows for local attention
  const int klo = __builtin_amdgcn_readfirstlane(win >= 0 ? max(lo, r0 - win) : lo);
  const int khi = __builtin_amdgcn_readfirstlane(win >= 0 ? min(hi, rend + win) : hi);

  vec8<Et> qr[2][QS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
    load_row_regs<Et, D>(qp, static_cast<int64_t>(qrow[qb]) * ld + h * D, g, qvalid[qb], qr[qb]);
  // retire the Q loads with a wait the compiler sees, so none lands inside the DMA loop
  vmem_fence_for_compiler();

  // ---- DMA: per-lane source offsets relative to the tile's first row
  const int64_t rowstride = ld * 2;  // bytes between packed K/V rows
  uint32_t doff[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int slot = j * kW64Threads + wv * 64 + lane;
    const int r = slot / CH, pc = slot - r * CH;
    doff[j] = static_cast<uint32_t>(r * rowstride + h * D * 2 + (pc ^ (swz(r) & (CH - 1))) * 16);
  }
  const char* kbase = static_cast<const char*>(kp);
  const char* vbase = static_cast<const char*>(vp);
  const int nblk = (khi - klo + kW64Keys - 1) / kW64Keys;
  auto issue = [&](int blk, int st) __attribute__((always_inline)) {
    const int row0 = klo + blk * kW64Keys;
    const bool full = row0 + kW64Keys <= khi;
    const char* kb = kbase + static_cast<int64_t>(row0) * rowstride;
    const char* vb = vbase + static_cast<int64_t>(row0) * rowstride;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      uint32_t off = doff[j];
      if (!full) {  // rows past the range repeat the last row (masked keys, valid memory)
        const int slot = j * kW64Threads + wv * 64 + lane;
        const int rr = slot / CH, pc = slot - rr * CH;
        const int r = min(rr, khi - 1 - row0);
        off = static_cast<uint32_t>(r * rowstride + h * D * 2 + (pc ^ (swz(rr) & (CH - 1))) * 16);
      }
      const uint32_t slotb = static_cast<uint32_t>((j * kW64Threads + wv * 64) * 16);
      dma16(lds_addr(ring[st][0]) + slotb, kb, off);
      dma16(lds_addr(ring[st][1]) + slotb, vb, off);
    }
  };

  // ---- per-lane LDS read offsets (bytes within a tile)
  int koff[QS];  // K operand: row ql, logical chunk g*(CH/2)+st
#pragma unroll
  for (int st = 0; st < QS; ++st) koff[st] = chunk_off<CH>(ql, g * (CH / 2) + st);
  const int sub = lane & 15, grp = (lane >> 4) & 1;
  int voff[2][2][DB];  // V^T operand: [s][hi][db], row 16s+4g+sub/4 (+8 for hi)
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int rowa = 16 * s + 4 * g + (sub >> 2) + 8 * hi;
        const int cc = 4 * db + 2 * grp + ((sub >> 1) & 1);
        voff[s][hi][db] = chunk_off<CH>(rowa, cc) + 8 * (sub & 1);
      }

  floatx16 o[2][DB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = floatx16{};
  float m[2] = {kNegBig, kNegBig}, l[2] = {0.f, 0.f};

  // ---- the pieces of one step
  // S^T of both query blocks for the key block in `ktile`
  auto qk_both = [&](const char* ktile, floatx16 (&s)[2]) __attribute__((always_inline)) {
    vec8<Et> ka[QS];
#pragma unroll
    for (int st = 0; st < QS; ++st) ka[st] = as_vec8<Et>(*reinterpret_cast<const u16x8*>(ktile + koff[st]));
    s[0] = mfma16<Et>(ka[0], qr[0][0], floatx16{});
    s[1] = mfma16<Et>(ka[0], qr[1][0], floatx16{});
#pragma unroll
    for (int st = 1; st < QS; ++st) {
      s[0] = mfma16<Et>(ka[st], qr[0][st], s[0]);
      s[1] = mfma16<Et>(ka[st], qr[1][st], s[1]);
    }
  };
  auto read_vt = [&](const char* vtile, vec8<Et> (&vt)[2][DB]) __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u16x4 lo4 = ds_read_tr16(reinterpret_cast<const uint16_t*>(vtile + voff[s2][0][db]));
        const u16x4 hi4 = ds_read_tr16(reinterpret_cast<const uint16_t*>(vtile + voff[s2][1][db]));
        vt[s2][db] = as_vec8<Et>(u16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]});
      }
  };
  // mask, block max and (rarely) the move of the running max with the O rescale
  auto row_max = [&](int qb, floatx16& s, int kb) __attribute__((always_inline)) {
    if (!(kb >= mk0[qb] && kb + kW64Keys <= mk1[qb])) {
      const int base = kb + 4 * g;
      mask_block(s, qk0[qb] - base, qk1[qb] - base);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = xhalf_max(mx);
    const float mnew = fmaxf(m[qb], mx * c);
    if (__any(mnew > m[qb] + kRescaleHeadroom)) {
      const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
      l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha;
      m[qb] = mnew;
    }
  };
  auto probs = [&](int qb, floatx16& s, vec8<Et> (&pb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m[qb]));
    probs_to_h16<Et>(s, pb, l[qb]);
  };
  auto pv = [&](int qb, const vec8<Et> (&pb)[2], const vec8<Et> (&vt)[2][DB]) __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[qb][db] = mfma16<Et>(vt[s2][db], pb[s2], o[qb][db]);
  };

  // Step j: S of both query blocks for key block j, then softmax and PV per query
  // block. A query block that does not need block j sees it fully masked (P = 0,
  // no max change), so one straight-line path serves every needed block.
  constexpr int AHEAD = kW64Stages - 1;  // blocks in flight ahead of the one computed
  // Wait until block j has landed: `later` blocks issued after it may stay in
  // flight (each 2*NL DMA instructions per thread; loads complete in order).
  auto wait_block = [&](int later) __attribute__((always_inline)) {
    if constexpr (AHEAD - 1 >= 4) {
      if (later >= 4) { wait_vmcnt<8 * NL>(); return; }
    }
    if constexpr (AHEAD - 1 >= 3) {
      if (later >= 3) { wait_vmcnt<6 * NL>(); return; }
    }
    if constexpr (AHEAD - 1 >= 2) {
      if (later >= 2) { wait_vmcnt<4 * NL>(); return; }
    }
    if (later >= 1) { wait_vmcnt<2 * NL>(); return; }
    wait_vmcnt<0>();
  };
  auto step = [&](auto tag, int j) __attribute__((always_inline)) {
    constexpr int ST = decltype(tag)::value;
    constexpr int STF = (ST + AHEAD) % kW64Stages;  // stage receiving block j+AHEAD
    wait_block(min(AHEAD - 1, nblk - 1 - j));
    raw_barrier();  // block j visible to all; the stage of block j-1 is no longer read
    if (j + AHEAD < nblk) issue(j + AHEAD, STF);
    const int kb = klo + j * kW64Keys;
    const bool need0 = kb < bk1[0] && kb + kW64Keys > bk0[0];
    const bool need1 = kb < bk1[1] && kb + kW64Keys > bk0[1];
    if (!(need0 || need1)) return;
    floatx16 s[2];
    qk_both(ring[ST][0], s);
    vec8<Et> vt[2][DB], pb0[2], pb1[2];
    read_vt(ring[ST][1], vt);
    row_max(0, s[0], kb);
    probs(0, s[0], pb0);
    pv(0, pb0, vt);
    row_max(1, s[1], kb);
    probs(1, s[1], pb1);
    pv(1, pb1, vt);
  };

  for (int i = 0; i < AHEAD; ++i)
    if (i < nblk) issue(i, i);
  for (int j = 0; j < nblk; j += kW64Stages) {
    step(W64Stage<0>{}, j);
    if (j + 1 < nblk) step(W64Stage<1>{}, j + 1);
    if constexpr (kW64Stages > 2) {
      if (j + 2 < nblk) step(W64Stage<2>{}, j + 2);
    }
    if constexpr (kW64Stages > 3) {
      if (j + 3 < nblk) step(W64Stage<3>{}, j + 3);
    }
    if constexpr (kW64Stages > 4) {
      if (j + 4 < nblk) step(W64Stage<4>{}, j + 4);
    }
    if constexpr (kW64Stages > 5) {
      if (j + 5 < nblk) step(W64Stage<5>{}, j + 5);
    }
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = xhalf_sum(l[qb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qvalid[qb]) {
      store_acc_row<Et, D>(op, (static_cast<int64_t>(qrow[qb]) * H + h) * D, o[qb], inv, g);
      if (lse != nullptr && g == 0) lse[static_cast<int64_t>(h) * N + qrow[qb]] = (m[qb] + log2f(lt)) * kLn2;
    }
  }
}

template <typename Et, int D>
hipError_t dispatch_w64(const void* q, const void* k, const void* v, const int32_t* cu, const int32_t* items,
                        int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* out,
                        float* lse, hipStream_t stream) {
  const int T = N / kAttnTileRows + B;  // sequence-aligned slots
  const int64_t blocks = static_cast<int64_t>(T) * H;
  if (blocks == 0) return hipSuccess;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipEvent_t ev = timing_start(stream);
  hipLaunchKernelGGL((attn_fwd_bf16_w64_kernel<Et, D>), dim3(static_cast<unsigned>(blocks)), dim3(kW64Threads), 0,
                     stream, q, k, v, cu, items, B, N, H, T, win, ld, c, out, lse);
  timing_stop("attn_fwd", ev, stream);
  return hipGetLastError();
}

}  // namespace

bool attn_fwd_bf16_w64_supported(int D) { return D == 32 || D == 64; }

hipError_t launch_attn_fwd_bf16_w64(bool f16, int D, const void* q, const void* k, const void* v, const int32_t* cu,
                                    const int32_t* items, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld,
                                    float scale, void* out, float* lse, hipStream_t stream) {
#define PE_W64_CASE(DD)                                                                                       \
  case DD:                                                                                                    \
    return f16 ? dispatch_w64<_Float16, DD>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream) \
               : dispatch_w64<__bf16, DD>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream);
  switch (D) {
    PE_W64_CASE(32)
    PE_W64_CASE(64)
    default: return hipErrorInvalidValue;
  }
#undef PE_W64_CASE
}

}  // namespace pe
