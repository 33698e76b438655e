// 16-bit forward of global or local (windowed) attention for head dims 32 and 64
// over sequence-aligned 128-row tiles: four waves of 32 query rows per workgroup at
// d = 64, two waves of 64 rows at d = 32.
//
// A workgroup takes slot t of the sequence-aligned work list of 128-row tiles
// (launch_seq_worklist with tile height 128): rows cu[b] + 128 * (t - cu[b] /
// 128 - b) .. of sequence b = items[t]. Every row of it has the key range
// [cu[b], cu[b+1]), so the loop needs no per-row range tests and only the
// sequence's last key block needs a mask. Wave w owns 32 or 64 rows (one or two
// 32-row query blocks); a wave whose rows all lie past the sequence's end still
// stages its share of every key block but computes nothing.
//
//   * K and V tiles of 32 keys travel global -> LDS by LDS DMA into a ring of two
//     stages (one block in flight) the waves fill together, tiles unpadded with
//     XOR-swizzled 16-byte chunks; one barrier per key block;
//   * S^T = K Q^T per query block (K rows from LDS as the A operand, Q^T in
//     registers), O^T += V^T P^T with P straight from the accumulators and V^T
//     read by ds_read_b64_tr_b16;
//   * the first key block sets each row's reference m to its exact maximum;
//     after it, p = exp2(c s - m) and their sums are taken against the current m
//     and only a block whose sum exceeds 2^15 (or is infinite) takes its exact
//     maximum, rescales O and l and recomputes p. p stays at most 2^15, which the
//     fp32 sums and the 16-bit products hold without loss of relative precision
//     (fp16's largest finite value is 65504: at 2^16 a p could round to infinity), and
//     O, l and the log-sum-exp share the one m, so the result is that of the
//     exact running maximum; the per-score maximum of the usual online softmax
//     is not computed. A middle key block is then one basic block (no branch
//     between its reads, MFMAs and softmax), which the other wave on the SIMD
//     overlaps.
// Local attention (LOCAL, window win: key j is seen by row i when |i - j| <= win)
// stages only the keys within win of the tile's rows; a wave computes only the
// key blocks that hold a key within win of one of its rows, and masks the keys
// farther than win from a row in the blocks that are not wholly within win of
// all of them. A wave whose first computed block is not the tile's first still
// has the initial reference: its first block's sums are infinite and take the
// exact-maximum path above, as does a row whose first keys come in a later block.
#include <climits>
#include <type_traits>

#include "attn_common.h"

namespace pe {

namespace {

// 32-row query blocks per wave, waves per 128-row tile, threads per workgroup and the
// waves per SIMD the register budget is sized for. At d = 64 one query block per wave
// (124 registers, four waves per SIMD) measured 10-12% faster side by side than two
// (213 registers, two waves per SIMD): the loop is latency-bound, and the extra waves
// outweigh reading each K and V^T operand from LDS for one MFMA instead of two. At
// d = 32 a 32-key tile is too small to split between four waves' DMA.
template <int D>
constexpr int b64_nq() { return D == 64 ? 1 : 2; }
template <int D>
constexpr int b64_threads() { return 64 * (4 / b64_nq<D>()); }
template <int D>
constexpr int b64_waves_per_simd() { return D == 64 ? 4 : 2; }
constexpr int kB64Keys = 32;      // keys per ring stage
// ring stages: one block in flight ahead of the one computed (2, 3 and 4 stages measured
// side by side on the long-document and mixed-batch forwards: 3 was 8% slower, 4 even
// with 2); the key loop below is written for two
constexpr int kB64Stages = 2;
constexpr float kB64Overflow = 32768.f;  // largest block sum of p kept without a new reference

// NQ: query blocks of this wave holding rows (0, 1 or 2; 0 only stages keys)
// [lo, hi): the keys of the tile (its sequence's; with LOCAL, those within win of its rows)
template <typename Et, int D, int NQ, bool LOCAL>
__device__ __forceinline__ void b64_run(const void* __restrict__ qp, const void* __restrict__ kp,
                                        const void* __restrict__ vp, int h, int rw, int rend, int lo, int hi,
                                        int win, int32_t N, int32_t H, int64_t ld, float c, void* __restrict__ op,
                                        float* __restrict__ lse, char (*ring)[2][kB64Keys * D * 2]) {
  constexpr int CH = D / 8;                     // 16-byte chunks per row
  constexpr int QS = D / 16;                    // MFMA steps over head_dim
  constexpr int DB = D / 32;                    // 32-row blocks of O^T
  constexpr int kB64Threads = b64_threads<D>();
  constexpr int NL = kB64Keys * CH / kB64Threads;  // DMA instructions per lane per tile
  static_assert(NL >= 1 && (kB64Keys * CH) % kB64Threads == 0, "whole DMA instructions per tile");
  constexpr int QB = NQ > 0 ? NQ : 1;           // array extents
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, g = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: DMA addresses stay scalar

  int qrow[QB];
  bool qvalid[QB];
  vec8<Et> qr[QB][QS];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    qrow[qb] = rw + 32 * qb + ql;
    qvalid[qb] = qrow[qb] < rend;
    load_row_regs<Et, D>(qp, static_cast<int64_t>(qrow[qb]) * ld + h * D, g, qvalid[qb], qr[qb]);
  }
  // LOCAL: key blocks starting in [bnd0, bnd1] hold a key within win of some row of this
  // wave, and those starting in [in0, in1] only keys within win of all of them
  const int bnd0 = rw - win - (kB64Keys - 1), bnd1 = rw + 32 * NQ - 1 + win;
  const int in0 = rw + 32 * NQ - 1 - win, in1 = rw + win - (kB64Keys - 1);
  // retire the Q loads with a wait the compiler sees, so none lands inside the DMA loop
  vmem_fence_for_compiler();

  // ---- DMA: per-lane source offsets relative to the tile's first row
  const int64_t rowstride = ld * 2;  // bytes between packed K/V rows
  uint32_t doff[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int slot = j * kB64Threads + wv * 64 + lane;
    const int r = slot / CH, pc = slot - r * CH;
    doff[j] = static_cast<uint32_t>(r * rowstride + h * D * 2 + (pc ^ (swz(r) & (CH - 1))) * 16);
  }
  const char* kbase = static_cast<const char*>(kp);
  const char* vbase = static_cast<const char*>(vp);
  const int nblk = (hi - lo + kB64Keys - 1) / kB64Keys;
  constexpr int TB = kB64Keys * D * 2;   // bytes per tile
  constexpr int STB = 2 * TB;            // bytes per ring stage (K and V tiles)
  const uint32_t ring0 = lds_addr(ring[0][0]);
  // The next block in order into ring stage st_tag (its index % 2, a constant or an int at
  // run time); its source rows advance by a constant per block (no per-block multiply).
  const int64_t blkbytes = static_cast<int64_t>(kB64Keys) * rowstride;
  const char* knext = kbase + static_cast<int64_t>(lo) * rowstride;
  const char* vnext = vbase + static_cast<int64_t>(lo) * rowstride;
  int rnext = lo;
  auto issue = [&](auto st_tag) __attribute__((always_inline)) {
    const int row0 = rnext;
    const uint32_t st = static_cast<uint32_t>(stage_of(st_tag) * STB);
    const char* kb = knext;
    const char* vb = vnext;
    rnext += kB64Keys;
    knext += blkbytes;
    vnext += blkbytes;
    if (row0 + kB64Keys <= hi) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const uint32_t slotb = static_cast<uint32_t>((j * kB64Threads + wv * 64) * 16);
        dma16(ring0 + st + slotb, kb, doff[j]);
        dma16(ring0 + st + TB + slotb, vb, doff[j]);
      }
    } else {  // the last block: rows past the sequence repeat its last row (masked keys, valid memory)
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int slot = j * kB64Threads + wv * 64 + lane;
        const int rr = slot / CH, pc = slot - rr * CH;
        const int r = min(rr, hi - 1 - row0);
        const uint32_t off = static_cast<uint32_t>(r * rowstride + h * D * 2 + (pc ^ (swz(rr) & (CH - 1))) * 16);
        const uint32_t slotb = static_cast<uint32_t>((j * kB64Threads + wv * 64) * 16);
        dma16(ring0 + st + slotb, kb, off);
        dma16(ring0 + st + TB + slotb, vb, off);
      }
    }
  };

  // ---- per-lane LDS read offsets (bytes within a tile)
  int koff[QS];  // K operand: row ql, logical chunk g*(CH/2)+st
#pragma unroll
  for (int q = 0; q < QS; ++q) koff[q] = chunk_off<CH>(ql, g * (CH / 2) + q);
  const int sub = lane & 15, grp = (lane >> 4) & 1;
  // V^T operand of step s: rows 16s + 4g + sub/4 (+8 for hi). Rows 16 + r carry the
  // swizzle of row r (it depends on bits 1-3 of the row), so step 1's offsets are step 0's
  // plus 16 rows, a constant: only step 0's are kept, voff[hi][db].
  int voff[2][DB];
  constexpr int VSTEP1 = 16 * CH * 16;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int rowa = 4 * g + (sub >> 2) + 8 * hh;
      const int cc = 4 * db + 2 * grp + ((sub >> 1) & 1);
      voff[hh][db] = chunk_off<CH>(rowa, cc) + 8 * (sub & 1);
    }

  floatx16 o[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = floatx16{};
    m[qb] = kNegBig;
    l[qb] = 0.f;
  }

  // p = exp2(c s - m) of one query block in place, returning the block's sum
  // (two chains of sums, each started at its first p: p >= 0, so 0 + p would be the same
  // value, but the compiler cannot drop that add)
  auto probs = [&](int qb, floatx16& s) __attribute__((always_inline)) {
    s[0] = __builtin_amdgcn_exp2f(fmaf(s[0], c, -m[qb]));
    s[1] = __builtin_amdgcn_exp2f(fmaf(s[1], c, -m[qb]));
    float a0 = s[0], a1 = s[1];
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
      s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m[qb]));
      s[i + 1] = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c, -m[qb]));
      a0 += s[i];
      a1 += s[i + 1];
    }
    return a0 + a1;
  };
  // the exact maximum of one query block's scores becomes its reference (O and l rescaled)
  auto rebase = [&](int qb, const floatx16& s) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = xhalf_max(mx);
    const float mnew = fmaxf(m[qb], mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
    l[qb] *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha;
    m[qb] = mnew;
  };

  vec8<Et> pb[QB][2], vt[2][DB];  // block j's probabilities and V^T operands
  auto pv = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] = mfma16<Et>(vt[s2][db], pb[qb][s2], o[qb][db]);
  };

  // Step j. FIRST: block 0 (each query block's exact maximum becomes its reference).
  // LAST: the sequence's last key block (keys past its end masked).
  // st_tag: block j's ring stage, j % 2 (a constant in the loop, so its LDS addresses are a
  // lane offset plus an immediate)
  auto step = [&](int j, auto st_tag, auto first_tag, auto last_tag) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_tag)::value;
    constexpr bool LAST = decltype(last_tag)::value;
    wait_vmcnt<0>();  // block j landed (the only block in flight)
    // this wave's reads of block j-1's stage have completed before the barrier, after which
    // the DMA below overwrites that stage
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    raw_barrier();  // block j visible to both waves; both have read block j-1's stage
    if (j + 1 < nblk) issue(other_stage(st_tag));
    if constexpr (NQ == 0) return;
    const int kb = lo + j * kB64Keys;
    if constexpr (LOCAL) {
      if (kb < bnd0 || kb > bnd1) return;  // wave-uniform: no key of the block is within win of a row
    }
    const uint32_t kt = ring0 + static_cast<uint32_t>(stage_of(st_tag) * STB);
    const uint32_t vtl = kt + static_cast<uint32_t>(TB);
    vec8<Et> ka[QS];
#pragma unroll
    for (int q = 0; q < QS; ++q) ka[q] = as_vec8<Et>(ds_read_b128_at(kt + koff[q]));
    floatx16 s[QB];
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) s[qb] = mfma16<Et>(ka[0], qr[qb][0], floatx16{});
#pragma unroll
    for (int q = 1; q < QS; ++q)
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb) s[qb] = mfma16<Et>(ka[q], qr[qb][q], s[qb]);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u16x4 lo4 = ds_read_tr16_at(vtl + s2 * VSTEP1 + voff[0][db]);
        const u16x4 hi4 = ds_read_tr16_at(vtl + s2 * VSTEP1 + voff[1][db]);
        vt[s2][db] = as_vec8<Et>(u16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]});
      }
    if constexpr (LAST) {  // keys past the sequence's end get no weight
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb) mask_block(s[qb], -INT_MAX, hi - (kb + 4 * g));
    }
    if constexpr (LOCAL) {  // keys farther than win from the row get no weight
      if (kb < in0 || kb > in1) {
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb) mask_block(s[qb], qrow[qb] - win - (kb + 4 * g), qrow[qb] + win + 1 - (kb + 4 * g));
      }
    }
    float ps[QB];
    bool ovf = false;
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
      if constexpr (FIRST) rebase(qb, s[qb]);
      floatx16 p = s[qb];
      ps[qb] = probs(qb, p);
      if constexpr (!FIRST) ovf |= !(ps[qb] <= kB64Overflow);  // also true for inf
      acc_to_h16<Et>(p, pb[qb]);
    }
    if constexpr (!FIRST) {
      if (__any(ovf)) {  // rare (scores far above the reference): rebase and redo
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb) {
          if (!__any(!(ps[qb] <= kB64Overflow))) continue;
          rebase(qb, s[qb]);
          floatx16 p = s[qb];
          ps[qb] = probs(qb, p);
          acc_to_h16<Et>(p, pb[qb]);
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) l[qb] += ps[qb];
    pv();
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  issue(S0{});
  if (nblk == 1) {
    step(0, S0{}, T_{}, T_{});
  } else {  // blocks 1 .. nblk-1 two per iteration (stages 1, 0), the last one masked
    step(0, S0{}, T_{}, F_{});
    int j = 1;
    for (; j + 2 < nblk; j += 2) {
      step(j, S1{}, F_{}, F_{});
      step(j + 1, S0{}, F_{}, F_{});
    }
    if (j + 1 < nblk) step(j++, S1{}, F_{}, F_{});
    step(j, j & 1, F_{}, T_{});  // (the stage at run time: as constants, the two copies of
                                 // this step spilled registers to scratch)
  }

#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    const float lt = xhalf_sum(l[qb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qvalid[qb]) {
      store_acc_row<Et, D>(op, (static_cast<int64_t>(qrow[qb]) * H + h) * D, o[qb], inv, g);
      if (lse != nullptr && g == 0) lse[static_cast<int64_t>(h) * N + qrow[qb]] = (m[qb] + log2f(lt)) * kLn2;
    }
  }
}

template <typename Et, int D, bool LOCAL>
__global__ __launch_bounds__(b64_threads<D>(), b64_waves_per_simd<D>()) void attn_fwd_w64b_kernel(
    const void* __restrict__ qp, const void* __restrict__ kp, const void* __restrict__ vp,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N, int32_t H,
    int32_t T, int32_t win, int64_t ld, float c, void* __restrict__ op, float* __restrict__ lse) {
  __shared__ __align__(16) char ring[kB64Stages][2][kB64Keys * D * 2];  // [stage][K, V][tile]
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lin / T, t = lin - h * T;
  // sequence-aligned tile: slot t of sequence b covers rows r0 .. r0 + 127 of it
  const int b = items[t];
  if (b >= B) return;  // block-uniform: a slot past the last sequence
  const int lo = cu[b], hi = cu[b + 1];
  const int r0 = lo + (t - (lo / kAttnTileRows + b)) * kAttnTileRows;
  if (r0 >= hi) return;  // block-uniform: an empty slot at the end of the sequence
  const int rend = min(r0 + kAttnTileRows, hi);
  // the tile's keys: its sequence's, with LOCAL only those within win of one of its rows
  const int klo = LOCAL ? max(lo, r0 - win) : lo;
  const int khi = LOCAL ? min(hi, rend + win) : hi;
  constexpr int NQ = b64_nq<D>();
  const int rw = r0 + 32 * NQ * static_cast<int>(threadIdx.x >> 6);  // this wave's first row
  const int nq = rw >= rend ? 0 : min(NQ, (rend - rw + 31) / 32);   // wave-uniform
  if constexpr (NQ == 2) {
    if (nq == 2) {
      b64_run<Et, D, 2, LOCAL>(qp, kp, vp, h, rw, rend, klo, khi, win, N, H, ld, c, op, lse, ring);
      return;
    }
  }
  if (nq == 1) b64_run<Et, D, 1, LOCAL>(qp, kp, vp, h, rw, rend, klo, khi, win, N, H, ld, c, op, lse, ring);
  else b64_run<Et, D, 0, LOCAL>(qp, kp, vp, h, rw, rend, klo, khi, win, N, H, ld, c, op, lse, ring);
}

template <typename Et, int D>
hipError_t dispatch_w64b(const void* q, const void* k, const void* v, const int32_t* cu, const int32_t* items,
                         int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* out, float* lse,
                         hipStream_t stream) {
  const int T = N / kAttnTileRows + B;  // sequence-aligned slots
  const int64_t blocks = static_cast<int64_t>(T) * H;
  if (blocks == 0) return hipSuccess;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipEvent_t ev = timing_start(stream);
  if (win >= 0)
    hipLaunchKernelGGL((attn_fwd_w64b_kernel<Et, D, true>), dim3(static_cast<unsigned>(blocks)),
                       dim3(b64_threads<D>()), 0, stream, q, k, v, cu, items, B, N, H, T, win, ld, c, out, lse);
  else
    hipLaunchKernelGGL((attn_fwd_w64b_kernel<Et, D, false>), dim3(static_cast<unsigned>(blocks)),
                       dim3(b64_threads<D>()), 0, stream, q, k, v, cu, items, B, N, H, T, win, ld, c, out, lse);
  timing_stop("attn_fwd", ev, stream);
  return hipGetLastError();
}

}  // namespace

bool attn_fwd_w64b_supported(int D) { return D == 32 || D == 64; }

hipError_t launch_attn_fwd_w64b(bool f16, int D, const void* q, const void* k, const void* v, const int32_t* cu,
                                const int32_t* items, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld,
                                float scale, void* out, float* lse, hipStream_t stream) {
  switch (D) {
    case 32:
      return f16 ? dispatch_w64b<_Float16, 32>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream)
                 : dispatch_w64b<__bf16, 32>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream);
    case 64:
      return f16 ? dispatch_w64b<_Float16, 64>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream)
                 : dispatch_w64b<__bf16, 64>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pe
