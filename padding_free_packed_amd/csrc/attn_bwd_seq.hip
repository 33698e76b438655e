// 16-bit backward of global or local (windowed) attention for head dims 32 and 64. For a
// length bound of at most 64 one single-pass kernel (see "short sequences" below); else
// three launches over sequence-aligned 128-row tiles. No atomics, so the result is bitwise
// reproducible:
//
//   prep:   per (head, row): nl = -lse * log2(e) and nd = -<dO, O> (minus the row's D)
//   dK/dV:  wave w of the workgroup on slot t of the sequence-aligned list of 128-row
//           tiles (rows r0 .. r0 + 127 of sequence b = items[t]) owns the keys
//           r0 + 32w .. + 31, K and V rows in registers, and streams its sequence's
//           query rows 32 at a time. Per 32 query rows:
//             S = Q K^T,  dP - D = dO V^T + nd    (nd is the accumulator's initial value)
//             P = exp2(c S + nl),  dS = P (dP - D)
//             dV^T += dO^T P,  dK^T += Q^T dS     (dO^T, Q^T by ds_read_b64_tr_b16)
//   dQ:     the same tiles over query rows: wave w owns 32 queries (Q and dO rows in
//           registers, nl and nd in one register each) and streams the sequence's key
//           rows 32 at a time:
//             S^T = K Q^T,  dP^T - D = V dO^T + nd,  dS^T = P^T (dP^T - D),  dQ^T += K^T dS^T
//   and dK, dQ are scaled by the softmax scale at the store.
//
// The streamed rows travel global -> LDS by LDS DMA into a ring of two stages that
// the four waves fill together (one block in flight while the other is computed),
// tiles unpadded with XOR-swizzled 16-byte chunks; one barrier per block. Every row
// of a tile has the same key and query range, its sequence, so no block needs a
// range test except the sequence's last, whose rows past the sequence's end repeat
// its last row (valid memory) and get probability 0. A wave whose 32 rows all lie
// past the end stages its share of every block and computes nothing.
//
// Against the 128-row packed tiles of attn_bwd.hip (a tile spans the sequences its
// rows fall in; query blocks start at the tile's first sequence), no product runs on
// rows of another sequence, and subtracting D and scaling by log2(e) leave the loop.
//
// Local attention (LOCAL, window win: row i and key j interact when |i - j| <= win):
// a tile streams only the rows within win of its own rows, a wave computes only the
// streamed blocks that reach its 32 rows, and in blocks not wholly within win of all
// of them the pairs farther apart get probability 0.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "attn_common.h"

namespace pe {

namespace {

// Rows per ring stage of the dK/dV and dQ passes, and the waves per SIMD their register
// budgets are sized for. Measured side by side on the mixed-batch backward at d = 64:
// 64-row stages (two 32-row sub-blocks per barrier) were 1-6% slower in both passes; the
// dK/dV pass at three waves per SIMD (168 registers) beat two (213) by 7%; the dQ pass at
// four waves (128 registers, spilling inside the loop) was 35% slower than at three; raising
// the wave priority around each run of MFMAs (s_setprio) was 3% slower; software-pipelining
// the dQ pass (the S^T, dP^T MFMAs of key block j+1 issued beside the softmax of block j,
// a three-stage ring, 222 registers so two waves per SIMD) was 15% slower.
constexpr int kKvRows = 32;
constexpr int kQRows = 32;
constexpr int kKvWaves = 3;
constexpr int kQWaves = 3;

// A workgroup takes R consecutive rows with all their heads (R = kPrepCells / H, at most
// kPrepRows): its lanes read the rows' dO and O as one contiguous run, one group of CH lanes
// per (row, head) with the 16-byte chunks fastest, and each group sums by butterfly (the
// summation order of the delta pass of attn_bwd.hip, so D is the same value). The sums go
// through LDS so that nl and nd of each head leave as one run of R values of [H, N].
constexpr int kPrepRows = 32;
constexpr int kPrepCells = 2048;  // (row, head) sums per workgroup at most
template <typename Et, int D>
__global__ __launch_bounds__(256) void bwd_seq_prep_kernel(const void* __restrict__ dout, const void* __restrict__ out,
                                                           const float* __restrict__ lse, int32_t N, int32_t H,
                                                           int32_t R, float* __restrict__ nl, float* __restrict__ nd) {
  constexpr int CH = D / 8;  // 16-byte chunks per head row (4 or 8)
  __shared__ float res[kPrepCells];  // [head][row] sums of the workgroup's rows
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * R;
  const int rows = static_cast<int>(min(static_cast<int64_t>(R), static_cast<int64_t>(N) - r0));
  const int cells = rows * H;
  const int chunks = cells * CH;
  const char* a = static_cast<const char*>(dout) + r0 * H * D * 2;
  const char* b = static_cast<const char*>(out) + r0 * H * D * 2;
  constexpr int U = 4;  // chunks per lane whose loads are in flight together
  for (int u0 = 0; u0 < chunks; u0 += U * 256) {  // block-uniform trip count: every lane takes part in the sums
    uint4 xa[U], xb[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int u = u0 + k * 256 + static_cast<int>(threadIdx.x);
      if (u < chunks) {
        xa[k] = *reinterpret_cast<const uint4*>(a + static_cast<int64_t>(u) * 16);
        xb[k] = *reinterpret_cast<const uint4*>(b + static_cast<int64_t>(u) * 16);
      } else {
        xa[k] = uint4{0, 0, 0, 0};
        xb[k] = uint4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int u = u0 + k * 256 + static_cast<int>(threadIdx.x);
      const u16x8 x = __builtin_bit_cast(u16x8, xa[k]), y = __builtin_bit_cast(u16x8, xb[k]);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(h16_to_f32<Et>(x[e]), h16_to_f32<Et>(y[e]), s);
#pragma unroll
      for (int o = 1; o < CH; o <<= 1) s += __shfl_xor(s, o);
      if (u < chunks && (u & (CH - 1)) == 0) {
        const int cell = u / CH, row = cell / H, hh = cell - row * H;
        res[hh * R + row] = s;
      }
    }
  }
  __syncthreads();
  for (int v = threadIdx.x; v < cells; v += 256) {  // rows fastest: each head's run is contiguous
    const int hh = v / rows, row = v - hh * rows;
    const int64_t o = static_cast<int64_t>(hh) * N + r0 + row;
    nd[o] = -res[hh * R + row];
    nl[o] = -(lse[o] * kLog2e);
  }
}

// The tile of slot t: [r0, rend) within sequence [lo, hi); false for an empty slot.
__device__ __forceinline__ bool seq_tile(const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int t,
                                         int B, int& lo, int& hi, int& r0, int& rend) {
  const int b = items[t];
  if (b >= B) return false;  // a slot past the last sequence
  lo = cu[b];
  hi = cu[b + 1];
  r0 = lo + (t - (lo / kAttnTileRows + b)) * kAttnTileRows;
  rend = min(r0 + kAttnTileRows, hi);
  return r0 < hi;  // else an empty slot at the end of the sequence
}

// Per-lane LDS offsets of the operands read from a 32-row swizzled stage tile:
// rows (row ql, logical chunk g*(CH/2) + q: an A operand over head_dim) and the
// transposed reads (two ds_read_b64_tr_b16 per A operand over the 32 rows, in the
// row order of the accumulator layout, as mma_tr_swz). The rows 16 s + r of step s = 1
// have the swizzle of row r (it depends on bits 1-3 of the row), so their offsets are
// those of step 0 plus 16 rows: only step 0's are kept.
template <int D>
struct StageOffsets {
  static constexpr int CH = D / 8, QS = D / 16, DB = D / 32;
  static constexpr int STEP1 = 16 * CH * 16;  // bytes of 16 rows
  int row[QS];
  int tr[2][DB];  // step 0, rows 4g + sub/4 (+8 for [1])
  __device__ __forceinline__ StageOffsets(int lane) {
    const int ql = lane & 31, g = lane >> 5, sub = lane & 15, grp = (lane >> 4) & 1;
#pragma unroll
    for (int q = 0; q < QS; ++q) row[q] = chunk_off<CH>(ql, g * (CH / 2) + q);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        tr[hh][db] = chunk_off<CH>(4 * g + (sub >> 2) + 8 * hh, 4 * db + 2 * grp + ((sub >> 1) & 1)) + 8 * (sub & 1);
  }
};

// The transposed A operand of step s, head-dim block db, from the tile at LDS byte tile.
template <typename Et, int D>
__device__ __forceinline__ vec8<Et> tr_operand(uint32_t tile, const StageOffsets<D>& so, int s, int db) {
  const uint32_t t = tile + static_cast<uint32_t>(s * StageOffsets<D>::STEP1);
  const u16x4 lo4 = ds_read_tr16_at(t + so.tr[0][db]);
  const u16x4 hi4 = ds_read_tr16_at(t + so.tr[1][db]);
  return as_vec8<Et>(u16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]});
}

// Staging of one RS-row block of two 16-bit tensors (tile 0 and tile 1 of a stage,
// rows `s0` and `s1` bytes apart) by the workgroup's 256 lanes: DMA instruction j of
// wave wv copies 16-byte chunks u = 256 j + 64 wv + lane of the two tiles (tile u / TC).
template <int D, int RS>
struct PairDma {
  static constexpr int CH = D / 8;
  static constexpr int TB = RS * D * 2;  // bytes of one tile
  static constexpr int TC = RS * CH;     // chunks of one tile
  static constexpr int NI = 2 * TC / kThreads;
  static_assert(NI >= 1 && (2 * TC) % kThreads == 0 && TC % 64 == 0, "whole DMA instructions per wave");
  uint32_t off[NI];  // source offsets of a full block relative to its first row
  int64_t s0, s1;
  int hoff, wv, lane;
  __device__ __forceinline__ PairDma(int64_t stride0, int64_t stride1, int h, int wv_, int lane_)
      : s0(stride0), s1(stride1), hoff(h * D * 2), wv(wv_), lane(lane_) {
#pragma unroll
    for (int j = 0; j < NI; ++j) off[j] = src_off(j, RS);
  }
  // source offset of this lane's chunk of instruction j; rows >= nrows repeat row nrows - 1
  __device__ __forceinline__ uint32_t src_off(int j, int nrows) const {
    const int u0 = j * kThreads + wv * 64;
    const int tl = u0 / TC;
    const int slot = u0 - tl * TC + lane;
    const int r = slot / CH, pc = slot - r * CH;
    const int rs = min(r, nrows - 1);
    return static_cast<uint32_t>(rs * (tl ? s1 : s0) + hoff + (pc ^ (swz(r) & (CH - 1))) * 16);
  }
  // the block whose first rows are at p0 and p1 (nrows of its RS rows inside the sequence)
  // into the stage at LDS byte st
  __device__ __forceinline__ void issue(uint32_t st, const char* p0, const char* p1, int nrows) const {
    if (nrows >= RS) {
#pragma unroll
      for (int j = 0; j < NI; ++j) dma16(dst(st, j), (j * kThreads + wv * 64) / TC ? p1 : p0, off[j]);
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) dma16(dst(st, j), (j * kThreads + wv * 64) / TC ? p1 : p0, src_off(j, nrows));
    }
  }
  // LDS destination of wave wv's instruction j (wave-uniform; lane l adds 16 l)
  __device__ __forceinline__ uint32_t dst(uint32_t st, int j) const {
    const int u0 = j * kThreads + wv * 64;
    const int tl = u0 / TC;
    return st + static_cast<uint32_t>(tl * TB + (u0 - tl * TC) * 16);
  }
};

template <typename Issue, typename Step>
__device__ __forceinline__ void run_blocks(int nblk, Issue& issue, Step& step) {
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  issue(S0{});
  int j = 0;
  for (; j + 2 < nblk; j += 2) {
    step(j, S0{}, std::false_type{});
    step(j + 1, S1{}, std::false_type{});
  }
  if (j + 1 < nblk) step(j++, S0{}, std::false_type{});
  step(j, j & 1, std::true_type{});  // one copy of the masked step, its stage at run time
}

template <typename Et, int D, bool LOCAL>
__global__ __launch_bounds__(kThreads, kKvWaves) void bwd_kv_seq_kernel(
    const void* __restrict__ dop, const void* __restrict__ qp, const void* __restrict__ kp,
    const void* __restrict__ vp, const float* __restrict__ nl, uint32_t nd_off, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ items, int32_t B, int32_t N, int32_t H, int32_t T, int32_t win, int64_t ld, float c,
    float scale, void* __restrict__ dkp, void* __restrict__ dvp) {
  constexpr int RS = kKvRows, QS = D / 16, DB = D / 32;
  using Dma = PairDma<D, RS>;
  constexpr int TB = Dma::TB;
  constexpr int SUBB = 32 * D * 2;               // bytes of 32 rows of a tile
  constexpr int SB = 2 * TB + 2 * RS * 4;        // stage: Q tile, dO tile, nl[RS], nd[RS]
  static_assert(2 * RS <= kThreads, "nl and nd of a stage in one DMA instruction per wave");
  __shared__ __align__(16) char ring[2][SB];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lin / T, t = lin - h * T;
  int slo, shi, r0, rend;
  if (!seq_tile(cu, items, t, B, slo, shi, r0, rend)) return;  // block-uniform
  // [lo, hi): the query rows streamed, the sequence's (LOCAL: those within win of a key of the tile)
  const int lo = LOCAL ? max(slo, r0 - win) : slo;
  const int hi = LOCAL ? min(shi, rend + win) : shi;
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, g = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // LOCAL: query blocks starting in [bnd0, bnd1] hold a row within win of a key of this wave,
  // those starting in [in0, in1] only rows within win of all of them
  const int kw = r0 + 32 * wv;
  const int bnd0 = kw - win - 31, bnd1 = kw + 31 + win, in0 = kw + 31 - win, in1 = kw + win - 31;
  const int krow = r0 + 32 * wv + ql;
  const bool kvalid = krow < rend;
  const bool active = r0 + 32 * wv < rend;  // wave-uniform

  vec8<Et> kreg[QS], vreg[QS];
  const int64_t roff = static_cast<int64_t>(krow) * ld + h * D;  // rows of K, V, dK, dV are ld apart
  load_row_regs<Et, D>(kp, roff, g, kvalid, kreg);
  load_row_regs<Et, D>(vp, roff, g, kvalid, vreg);
  // retire the row loads with a wait the compiler sees, so none lands inside the DMA loop
  vmem_fence_for_compiler();

  const Dma dma(ld * 2, static_cast<int64_t>(H) * D * 2, h, wv, lane);
  const char* qbase = static_cast<const char*>(qp);
  const char* dbase = static_cast<const char*>(dop);
  const float* nlh = nl + static_cast<int64_t>(h) * N;
  const uint32_t ring0 = lds_addr(ring[0]);
  const int nblk = (hi - lo + RS - 1) / RS;
  // The next block in order into ring stage st_tag (its index % 2); the source rows
  // advance by a constant per block.
  const char* qnext = qbase + static_cast<int64_t>(lo) * dma.s0;
  const char* dnext = dbase + static_cast<int64_t>(lo) * dma.s1;
  int rnext = lo;
  auto issue = [&](auto st_tag) __attribute__((always_inline)) {
    const int ST = stage_of(st_tag);
    const int row0 = rnext;
    const int nrows = hi - row0;
    const uint32_t st = ring0 + static_cast<uint32_t>(ST * SB);
    dma.issue(st, qnext, dnext, nrows);
    rnext += RS;
    qnext += RS * dma.s0;
    dnext += RS * dma.s1;
    if (wv < 2 * RS / 64) {  // dwords u = 64 wv + lane: nl (u < RS) then nd of the RS rows
      const int u = 64 * wv + lane;
      const int arr = u >= RS, r = u - arr * RS;
      const uint32_t o = static_cast<uint32_t>(min(r, nrows - 1)) * 4 + (arr ? nd_off : 0u);
      dma4(st + 2 * TB + 256 * wv, nlh + row0, o);
    }
  };

  const StageOffsets<D> so(lane);
  floatx16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = floatx16{};
    dv[db] = floatx16{};
  }

  // query rows 32 sb .. 32 sb + 31 of the stage at LDS byte st (first row qr0)
  auto sub = [&](uint32_t st, int sb, int qr0, auto last_tag) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last_tag)::value;
    const uint32_t qt = st + static_cast<uint32_t>(sb * SUBB);
    const uint32_t dt = qt + TB;
    const uint32_t lt = st + 2 * TB + 4 * (32 * sb + 4 * g);  // nl of rows 4g .. 4g+3 (+32 bytes per 8 rows)
    floatx16 s = floatx16{}, dp;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {  // dP starts at -D of its rows
      const floatx4 n4 = __builtin_bit_cast(floatx4, ds_read_b128_at(lt + 4 * RS + 32 * i4));
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[4 * i4 + e] = n4[e];
    }
#pragma unroll
    for (int q = 0; q < QS; ++q) s = mfma16<Et>(as_vec8<Et>(ds_read_b128_at(qt + so.row[q])), kreg[q], s);
#pragma unroll
    for (int q = 0; q < QS; ++q) dp = mfma16<Et>(as_vec8<Et>(ds_read_b128_at(dt + so.row[q])), vreg[q], dp);
    if constexpr (LAST) mask_block(s, -INT_MAX, hi - (qr0 + 4 * g));  // query rows past the end
    if constexpr (LOCAL) {  // rows farther than win from this lane's key
      if (qr0 < in0 || qr0 > in1) mask_block(s, krow - win - (qr0 + 4 * g), krow + win + 1 - (qr0 + 4 * g));
    }
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const floatx4 l4 = __builtin_bit_cast(floatx4, ds_read_b128_at(lt + 32 * i4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * i4 + e;
        const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c, l4[e]));
        s[i] = p;
        dp[i] *= p;
      }
    }
    vec8<Et> pb[2], sb16[2];
    acc_to_h16<Et>(s, pb);
    acc_to_h16<Et>(dp, sb16);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db) dv[db] = mfma16<Et>(tr_operand<Et, D>(dt, so, s2, db), pb[s2], dv[db]);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db) dk[db] = mfma16<Et>(tr_operand<Et, D>(qt, so, s2, db), sb16[s2], dk[db]);
  };

  // block j from ring stage ST = j % 2
  auto step = [&](int j, auto st_tag, auto last_tag) __attribute__((always_inline)) {
    const int ST = stage_of(st_tag);
    constexpr bool LAST = decltype(last_tag)::value;
    wait_vmcnt<0>();
    // this wave's reads of block j-1's stage have completed before the barrier, after
    // which the DMA below overwrites that stage
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    raw_barrier();  // block j visible to every wave; all have read block j-1's stage
    if (j + 1 < nblk) issue(other_stage(st_tag));
    if (!active) return;
    const uint32_t st = ring0 + static_cast<uint32_t>(ST * SB);
#pragma unroll
    for (int sb = 0; sb < RS / 32; ++sb) {
      const int qr0 = lo + j * RS + 32 * sb;
      if constexpr (LOCAL) {
        if (qr0 < bnd0 || qr0 > bnd1) continue;  // wave-uniform: no row within win of this wave's keys
      }
      if constexpr (LAST) {
        if (qr0 >= hi) break;  // wave-uniform: past the sequence's end
        sub(st, sb, qr0, std::true_type{});
      } else {
        sub(st, sb, qr0, std::false_type{});
      }
    }
  };

  run_blocks(nblk, issue, step);

  if (kvalid) {
    store_acc_row<Et, D>(dkp, roff, dk, scale, g);
    store_acc_row<Et, D>(dvp, roff, dv, 1.f, g);
  }
}

template <typename Et, int D, bool LOCAL>
__global__ __launch_bounds__(kThreads, kQWaves) void bwd_q_seq_kernel(
    const void* __restrict__ dop, const void* __restrict__ qp, const void* __restrict__ kp,
    const void* __restrict__ vp, const float* __restrict__ nl, const float* __restrict__ nd,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N, int32_t H, int32_t T,
    int32_t win, int64_t ld, float c, float scale, void* __restrict__ dqp) {
  constexpr int RS = kQRows, QS = D / 16, DB = D / 32;
  using Dma = PairDma<D, RS>;
  constexpr int TB = Dma::TB;
  constexpr int SUBB = 32 * D * 2;  // bytes of 32 rows of a tile
  constexpr int SB = 2 * TB;        // stage: K tile, V tile
  __shared__ __align__(16) char ring[2][SB];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lin / T, t = lin - h * T;
  int slo, shi, r0, rend;
  if (!seq_tile(cu, items, t, B, slo, shi, r0, rend)) return;  // block-uniform
  // [lo, hi): the keys streamed, the sequence's (LOCAL: those within win of a row of the tile)
  const int lo = LOCAL ? max(slo, r0 - win) : slo;
  const int hi = LOCAL ? min(shi, rend + win) : shi;
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, g = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // LOCAL: key blocks starting in [bnd0, bnd1] hold a key within win of a row of this wave,
  // those starting in [in0, in1] only keys within win of all of them
  const int qw = r0 + 32 * wv;
  const int bnd0 = qw - win - 31, bnd1 = qw + 31 + win, in0 = qw + 31 - win, in1 = qw + win - 31;
  const int qrow = r0 + 32 * wv + ql;
  const bool qvalid = qrow < rend;
  const bool active = r0 + 32 * wv < rend;  // wave-uniform

  vec8<Et> qreg[QS], dreg[QS];
  const int64_t roff = static_cast<int64_t>(qrow) * ld + h * D;  // rows of Q and dQ are ld apart
  load_row_regs<Et, D>(qp, roff, g, qvalid, qreg);
  load_row_regs<Et, D>(dop, (static_cast<int64_t>(qrow) * H + h) * D, g, qvalid, dreg);
  const float nlq = qvalid ? nl[static_cast<int64_t>(h) * N + qrow] : 0.f;
  const float ndq = qvalid ? nd[static_cast<int64_t>(h) * N + qrow] : 0.f;
  vmem_fence_for_compiler();

  const Dma dma(ld * 2, ld * 2, h, wv, lane);
  const char* kbase = static_cast<const char*>(kp);
  const char* vbase = static_cast<const char*>(vp);
  const uint32_t ring0 = lds_addr(ring[0]);
  const int nblk = (hi - lo + RS - 1) / RS;
  // The next block in order into ring stage st_tag (its index % 2); the source rows
  // advance by a constant per block.
  const char* knext = kbase + static_cast<int64_t>(lo) * dma.s0;
  const char* vnext = vbase + static_cast<int64_t>(lo) * dma.s1;
  int rnext = lo;
  auto issue = [&](auto st_tag) __attribute__((always_inline)) {
    const int ST = stage_of(st_tag);
    dma.issue(ring0 + static_cast<uint32_t>(ST * SB), knext, vnext, hi - rnext);
    rnext += RS;
    knext += RS * dma.s0;
    vnext += RS * dma.s1;
  };

  const StageOffsets<D> so(lane);
  floatx16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = floatx16{};

  // keys 32 sb .. 32 sb + 31 of the stage at LDS byte st (first key kr0)
  auto sub = [&](uint32_t st, int sb, int kr0, auto last_tag) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last_tag)::value;
    const uint32_t kt = st + static_cast<uint32_t>(sb * SUBB);
    const uint32_t vt = kt + TB;
    floatx16 s = floatx16{}, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] = ndq;  // dP^T starts at -D of this lane's query
#pragma unroll
    for (int q = 0; q < QS; ++q) s = mfma16<Et>(as_vec8<Et>(ds_read_b128_at(kt + so.row[q])), qreg[q], s);
#pragma unroll
    for (int q = 0; q < QS; ++q) dp = mfma16<Et>(as_vec8<Et>(ds_read_b128_at(vt + so.row[q])), dreg[q], dp);
    if constexpr (LAST) mask_block(s, -INT_MAX, hi - (kr0 + 4 * g));  // keys past the end
    if constexpr (LOCAL) {  // keys farther than win from this lane's row
      if (kr0 < in0 || kr0 > in1) mask_block(s, qrow - win - (kr0 + 4 * g), qrow + win + 1 - (kr0 + 4 * g));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] *= __builtin_amdgcn_exp2f(fmaf(s[i], c, nlq));
    vec8<Et> sb16[2];
    acc_to_h16<Et>(dp, sb16);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db) dq[db] = mfma16<Et>(tr_operand<Et, D>(kt, so, s2, db), sb16[s2], dq[db]);
  };

  auto step = [&](int j, auto st_tag, auto last_tag) __attribute__((always_inline)) {
    const int ST = stage_of(st_tag);
    constexpr bool LAST = decltype(last_tag)::value;
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    raw_barrier();
    if (j + 1 < nblk) issue(other_stage(st_tag));
    if (!active) return;
    const uint32_t st = ring0 + static_cast<uint32_t>(ST * SB);
#pragma unroll
    for (int sb = 0; sb < RS / 32; ++sb) {
      const int kr0 = lo + j * RS + 32 * sb;
      if constexpr (LOCAL) {
        if (kr0 < bnd0 || kr0 > bnd1) continue;  // wave-uniform: no key within win of this wave's rows
      }
      if constexpr (LAST) {
        if (kr0 >= hi) break;  // wave-uniform: past the sequence's end
        sub(st, sb, kr0, std::true_type{});
      } else {
        sub(st, sb, kr0, std::false_type{});
      }
    }
  };

  run_blocks(nblk, issue, step);

  if (qvalid) store_acc_row<Et, D>(dqp, roff, dq, scale, g);
}

// ---------------------------------------------------------------- short sequences
// Every length at most 64 (one or two 32-row blocks): one workgroup of two waves per
// (sequence, head) computes dQ, dK and dV in a single pass, with no prep pass and no
// work list. The sequence's Q, K, V and dO rows travel by LDS DMA into XOR-swizzled
// tiles the two waves share (read back as row operands and, by ds_read_b64_tr_b16, as
// transposed ones), and D = <dO, O> and -lse log2(e) of its rows are formed in place. Wave 0 takes, per key block, S = Q K^T and dP - D =
// dO V^T + nd over every query block and accumulates dV^T += dO^T P, dK^T += Q^T dS;
// wave 1 takes, per query block, S^T and dP^T - D over every key block and accumulates
// dQ^T += K^T dS^T. S and dP are formed in both orientations (seven products where five
// would do), so every P and dS enters its product straight from the accumulators: a
// short sequence moves many bytes per flop, and the extra products cost less than a
// transpose through LDS.
constexpr int kShortBwdMaxLen = 64;

// NB: 32-row blocks of this sequence (1 or 2, block-uniform); NBT: blocks per tile array
template <typename Et, int D, int NB, int NBT>
__device__ __forceinline__ void short_bwd(const void* __restrict__ dop, const void* __restrict__ qp,
                                          const void* __restrict__ kp, const void* __restrict__ vp,
                                          const void* __restrict__ op, const float* __restrict__ lse, int w, int h,
                                          int lo, int hi, int32_t N, int32_t H, int32_t win, int64_t ld, float c,
                                          float scale, void* __restrict__ dqp, void* __restrict__ dkp,
                                          void* __restrict__ dvp, char (*tiles)[NBT][32 * D * 2], float* nlnd) {
  // tiles: [Q, K, dO, V][block]
  constexpr int CH = D / 8, QS = D / 16, DB = D / 32;
  constexpr int TB = 32 * D * 2;     // bytes of one 32-row tile
  constexpr int NL = 32 * CH / 64;   // DMA instructions per tile and wave
  const int lane = threadIdx.x & 63, ql = lane & 31, g = lane >> 5;
  const int64_t hd = static_cast<int64_t>(H) * D;  // elements between dO (and O) rows
  const uint32_t tq = lds_addr(tiles[0][0]), tk = lds_addr(tiles[1][0]), td = lds_addr(tiles[2][0]);
  const uint32_t tv = lds_addr(tiles[3][0]);

  // Q, K (wave 0), dO and V (wave 1) rows -> the tiles (rows past the sequence repeat its last
  // row: valid memory, and every product they enter is masked or never stored)
  const char* qb0 = static_cast<const char*>(qp) + static_cast<int64_t>(lo) * ld * 2;
  const char* kb0 = static_cast<const char*>(kp) + static_cast<int64_t>(lo) * ld * 2;
  const char* db0 = static_cast<const char*>(dop) + static_cast<int64_t>(lo) * hd * 2;
  const char* vb0 = static_cast<const char*>(vp) + static_cast<int64_t>(lo) * ld * 2;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int slot = j * 64 + lane;
      const int r = slot / CH, pc = slot - r * CH;
      const int rr = min(32 * b + r, hi - lo - 1);
      const uint32_t cofs = static_cast<uint32_t>(h * D * 2 + (pc ^ (swz(r) & (CH - 1))) * 16);
      const uint32_t dst = static_cast<uint32_t>(b * TB + j * 1024);
      if (w == 0) {
        dma16(tq + dst, qb0, static_cast<uint32_t>(rr * ld * 2) + cofs);
        dma16(tk + dst, kb0, static_cast<uint32_t>(rr * ld * 2) + cofs);
      } else {
        dma16(td + dst, db0, static_cast<uint32_t>(rr * hd * 2) + cofs);
        dma16(tv + dst, vb0, static_cast<uint32_t>(rr * ld * 2) + cofs);
      }
    }
  // the lane's rows of O and the LSE (rows past the sequence: zero)
  vec8<Et> orw[NB][QS];
  float lq[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int row = lo + 32 * b + ql;
    load_row_regs<Et, D>(op, static_cast<int64_t>(row) * hd + h * D, g, row < hi, orw[b]);
    lq[b] = row < hi ? lse[static_cast<int64_t>(h) * N + row] : 0.f;
  }
  wait_vmcnt<0>();  // this wave's tile rows have landed
  raw_barrier();    // and the other wave's

  const StageOffsets<D> so(lane);
  // nl = -lse log2(e) and nd = -<dO, O> of every row: the lane's own in registers, and (wave 0)
  // all of them in LDS (nl[0..63], nd[64..127]) for the products whose rows span 16 lanes' rows
  float nlq[NB], ndq[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float dsum = 0.f;
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      const vec8<Et> dv8 = as_vec8<Et>(ds_read_b128_at(td + static_cast<uint32_t>(b * TB + so.row[q])));
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = fmaf(static_cast<float>(dv8[e]), static_cast<float>(orw[b][q][e]), dsum);
    }
    ndq[b] = -xhalf_sum(dsum);
    nlq[b] = -(lq[b] * kLog2e);
    if (w == 0 && g == 0) {
      nlnd[32 * b + ql] = nlq[b];
      nlnd[64 + 32 * b + ql] = ndq[b];
    }
  }

  if (w == 0) {  // ---- dK and dV, one key block at a time (lane = key)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // nl, nd written before they are read
    const uint32_t nl0 = lds_addr(nlnd);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      asm volatile("" ::: "memory");  // no LDS read of this block is hoisted above the previous one's work
      const int krow = lo + 32 * kb + ql;
      vec8<Et> kreg[QS], vreg[QS];
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        kreg[q] = as_vec8<Et>(ds_read_b128_at(tk + static_cast<uint32_t>(kb * TB + so.row[q])));
        vreg[q] = as_vec8<Et>(ds_read_b128_at(tv + static_cast<uint32_t>(kb * TB + so.row[q])));
      }
      floatx16 dk[DB], dv[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dk[db] = floatx16{};
        dv[db] = floatx16{};
      }
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) {
        asm volatile("" ::: "memory");
        const uint32_t qt = tq + static_cast<uint32_t>(qb * TB), dt = td + static_cast<uint32_t>(qb * TB);
        const int qr0 = lo + 32 * qb;
        const uint32_t lt = nl0 + static_cast<uint32_t>(4 * (32 * qb + 4 * g));  // nl of rows 4g.. (+32 bytes per 8 rows)
        floatx16 s = floatx16{}, dp;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {  // dP starts at -D of its rows
          const floatx4 n4 = __builtin_bit_cast(floatx4, ds_read_b128_at(lt + 256 + 32 * i4));
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[4 * i4 + e] = n4[e];
        }
#pragma unroll
        for (int q = 0; q < QS; ++q) s = mfma16<Et>(as_vec8<Et>(ds_read_b128_at(qt + so.row[q])), kreg[q], s);
#pragma unroll
        for (int q = 0; q < QS; ++q) dp = mfma16<Et>(as_vec8<Et>(ds_read_b128_at(dt + so.row[q])), vreg[q], dp);
        mask_block(s, -INT_MAX, hi - (qr0 + 4 * g));  // query rows past the end
        if (win >= 0) mask_block(s, krow - win - (qr0 + 4 * g), krow + win + 1 - (qr0 + 4 * g));
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const floatx4 l4 = __builtin_bit_cast(floatx4, ds_read_b128_at(lt + 32 * i4));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * i4 + e;
            const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c, l4[e]));
            s[i] = p;
            dp[i] *= p;
          }
        }
        vec8<Et> pb[2], sb16[2];
        acc_to_h16<Et>(s, pb);
        acc_to_h16<Et>(dp, sb16);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            dv[db] = mfma16<Et>(tr_operand<Et, D>(dt, so, s2, db), pb[s2], dv[db]);
            dk[db] = mfma16<Et>(tr_operand<Et, D>(qt, so, s2, db), sb16[s2], dk[db]);
          }
      }
      if (krow < hi) {  // the same for both lane halves, which store together
        const int64_t roff = static_cast<int64_t>(krow) * ld + h * D;
        store_acc_row<Et, D>(dkp, roff, dk, scale, g);
        store_acc_row<Et, D>(dvp, roff, dv, 1.f, g);
      }
    }
  } else {  // ---- dQ, one query block at a time (lane = query)
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      asm volatile("" ::: "memory");
      const int qrow = lo + 32 * qb + ql;
      vec8<Et> qreg[QS], dreg[QS];
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        qreg[q] = as_vec8<Et>(ds_read_b128_at(tq + static_cast<uint32_t>(qb * TB + so.row[q])));
        dreg[q] = as_vec8<Et>(ds_read_b128_at(td + static_cast<uint32_t>(qb * TB + so.row[q])));
      }
      floatx16 dq[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) dq[db] = floatx16{};
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        asm volatile("" ::: "memory");
        const uint32_t kt = tk + static_cast<uint32_t>(kb * TB);
        const int kr0 = lo + 32 * kb;
        floatx16 s = floatx16{}, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) dp[i] = ndq[qb];  // dP^T starts at -D of this lane's query
#pragma unroll
        for (int q = 0; q < QS; ++q) s = mfma16<Et>(as_vec8<Et>(ds_read_b128_at(kt + so.row[q])), qreg[q], s);
#pragma unroll
        for (int q = 0; q < QS; ++q)
          dp = mfma16<Et>(as_vec8<Et>(ds_read_b128_at(tv + static_cast<uint32_t>(kb * TB + so.row[q]))), dreg[q], dp);
        mask_block(s, -INT_MAX, hi - (kr0 + 4 * g));  // keys past the end
        if (win >= 0) mask_block(s, qrow - win - (kr0 + 4 * g), qrow + win + 1 - (kr0 + 4 * g));
#pragma unroll
        for (int i = 0; i < 16; ++i) dp[i] *= __builtin_amdgcn_exp2f(fmaf(s[i], c, nlq[qb]));
        vec8<Et> sb16[2];
        acc_to_h16<Et>(dp, sb16);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int db = 0; db < DB; ++db) dq[db] = mfma16<Et>(tr_operand<Et, D>(kt, so, s2, db), sb16[s2], dq[db]);
      }
      if (qrow < hi) store_acc_row<Et, D>(dqp, static_cast<int64_t>(qrow) * ld + h * D, dq, scale, g);
    }
  }
}

template <typename Et, int D, int NBT>
__global__ __launch_bounds__(128) void bwd_short_kernel(
    const void* __restrict__ dop, const void* __restrict__ qp, const void* __restrict__ kp,
    const void* __restrict__ vp, const void* __restrict__ op, const float* __restrict__ lse,
    const int32_t* __restrict__ cu, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld, float c, float scale,
    void* __restrict__ dqp, void* __restrict__ dkp, void* __restrict__ dvp) {
  __shared__ __align__(16) char tiles[4][NBT][32 * D * 2];  // [Q, K, dO, V][block][tile]
  __shared__ __align__(16) float nlnd[128];
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t item = blockIdx.x;  // (sequence, head), heads fastest
  const int b = static_cast<int>(item / H), h = static_cast<int>(item - static_cast<int64_t>(b) * H);
  if (b >= B) return;  // block-uniform
  const int lo = cu[b];
  // a length above the bound is cut to its first 32 NBT rows (rows past them are left as
  // they were), so no access leaves the sequence or the tiles
  const int hi = min(cu[b + 1], lo + 32 * NBT);
  if (hi <= lo) return;  // block-uniform
  if (NBT == 1 || hi - lo <= 32)
    short_bwd<Et, D, 1, NBT>(dop, qp, kp, vp, op, lse, w, h, lo, hi, N, H, win, ld, c, scale, dqp, dkp, dvp, tiles,
                             nlnd);
  else
    short_bwd<Et, D, (NBT > 1 ? 2 : 1), NBT>(dop, qp, kp, vp, op, lse, w, h, lo, hi, N, H, win, ld, c, scale, dqp,
                                             dkp, dvp, tiles, nlnd);
}

template <typename Et, int D>
hipError_t bwd_short_dispatch(const void* dout, const void* q, const void* k, const void* v, const void* out,
                              const float* lse, const int32_t* cu, int32_t B, int32_t N, int32_t H,
                              int32_t max_seq_len, int32_t win, int64_t ld, float scale, void* dq, void* dk, void* dv,
                              hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(B) * H;
  if (items == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(items);
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipEvent_t ev = timing_start(stream);
  if (max_seq_len <= 32)
    hipLaunchKernelGGL((bwd_short_kernel<Et, D, 1>), dim3(blocks), dim3(128), 0, stream, dout, q, k,
                       v, out, lse, cu, B, N, H, win, ld, c, scale, dq, dk, dv);
  else
    hipLaunchKernelGGL((bwd_short_kernel<Et, D, 2>), dim3(blocks), dim3(128), 0, stream, dout, q, k,
                       v, out, lse, cu, B, N, H, win, ld, c, scale, dq, dk, dv);
  timing_stop("bwd_short", ev, stream);
  return hipGetLastError();
}

template <typename Et, int D>
hipError_t bwd_seq_dispatch(const void* dout, const void* q, const void* k, const void* v, const void* out,
                            const float* lse, const int32_t* cu, const int32_t* items, int32_t B, int32_t N,
                            int32_t H, int32_t win, int64_t ld, float scale, void* dq, void* dk, void* dv, float* nl,
                            float* nd, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int R = std::max(1, std::min(kPrepRows, kPrepCells / H));  // rows per prep workgroup
  hipEvent_t ev_prep = timing_start(stream);
  hipLaunchKernelGGL((bwd_seq_prep_kernel<Et, D>), dim3(static_cast<unsigned>((N + R - 1) / R)), dim3(256), 0, stream,
                     dout, out, lse, N, H, R, nl, nd);
  timing_stop("bwd_delta", ev_prep, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int T = N / kAttnTileRows + B;  // sequence-aligned slots
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(T) * H);
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  const uint32_t nd_off = static_cast<uint32_t>((nd - nl) * static_cast<int64_t>(sizeof(float)));
  hipEvent_t ev_kv = timing_start(stream);
  if (win >= 0)
    hipLaunchKernelGGL((bwd_kv_seq_kernel<Et, D, true>), dim3(blocks), dim3(kThreads), 0, stream, dout, q, k, v, nl,
                       nd_off, cu, items, B, N, H, T, win, ld, c, scale, dk, dv);
  else
    hipLaunchKernelGGL((bwd_kv_seq_kernel<Et, D, false>), dim3(blocks), dim3(kThreads), 0, stream, dout, q, k, v, nl,
                       nd_off, cu, items, B, N, H, T, win, ld, c, scale, dk, dv);
  timing_stop("bwd_dkdv", ev_kv, stream);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipEvent_t ev_q = timing_start(stream);
  if (win >= 0)
    hipLaunchKernelGGL((bwd_q_seq_kernel<Et, D, true>), dim3(blocks), dim3(kThreads), 0, stream, dout, q, k, v, nl, nd,
                       cu, items, B, N, H, T, win, ld, c, scale, dq);
  else
    hipLaunchKernelGGL((bwd_q_seq_kernel<Et, D, false>), dim3(blocks), dim3(kThreads), 0, stream, dout, q, k, v, nl,
                       nd, cu, items, B, N, H, T, win, ld, c, scale, dq);
  timing_stop("bwd_dq", ev_q, stream);
  return hipGetLastError();
}

}  // namespace

bool attn_bwd_seq_supported(int dt, int D, int32_t win, int64_t N, int32_t H, int64_t ld) {
  if (dt != kDtBF16 && dt != kDtF16) return false;
  if (D != 32 && D != 64) return false;
  if (H > kPrepCells) return false;  // the prep pass holds a row's sums of every head in LDS
  // 32-bit DMA offsets: 32 rows of the widest stride, and nl/nd ([H, N] floats each,
  // nd after nl) within 4 GiB of nl
  if (ld * 2 * max(kKvRows, kQRows) >= (int64_t{1} << 31)) return false;
  return N * H * 2 * static_cast<int64_t>(sizeof(float)) + 256 < (int64_t{1} << 32);
}

bool attn_bwd_short_supported(int dt, int D, int32_t max_seq_len, int64_t ld, int32_t H) {
  if (dt != kDtBF16 && dt != kDtF16) return false;
  if ((D != 32 && D != 64) || max_seq_len > kShortBwdMaxLen) return false;
  // 32-bit DMA offsets: 64 rows of the widest stride
  return std::max(ld, static_cast<int64_t>(H) * D) * 2 * kShortBwdMaxLen < (int64_t{1} << 31);
}

hipError_t launch_attn_bwd_short(int dt, int D, const void* dout, const void* q, const void* k, const void* v,
                                 const void* out, const float* lse, const int32_t* cu, int32_t B, int32_t N,
                                 int32_t H, int32_t max_seq_len, int32_t win, int64_t ld, float scale, void* dq,
                                 void* dk, void* dv, hipStream_t stream) {
  const bool f16 = dt == kDtF16;
  switch (D) {
    case 32:
      return f16 ? bwd_short_dispatch<_Float16, 32>(dout, q, k, v, out, lse, cu, B, N, H, max_seq_len, win, ld, scale,
                                                   dq, dk, dv, stream)
                 : bwd_short_dispatch<__bf16, 32>(dout, q, k, v, out, lse, cu, B, N, H, max_seq_len, win, ld, scale,
                                                 dq, dk, dv, stream);
    case 64:
      return f16 ? bwd_short_dispatch<_Float16, 64>(dout, q, k, v, out, lse, cu, B, N, H, max_seq_len, win, ld, scale,
                                                   dq, dk, dv, stream)
                 : bwd_short_dispatch<__bf16, 64>(dout, q, k, v, out, lse, cu, B, N, H, max_seq_len, win, ld, scale,
                                                 dq, dk, dv, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bwd_seq(int dt, int D, const void* dout, const void* q, const void* k, const void* v,
                               const void* out, const float* lse, const int32_t* cu, const int32_t* items, int32_t B,
                               int32_t N, int32_t H, int32_t win, int64_t ld, float scale, void* dq, void* dk, void* dv,
                               float* nl, float* nd, hipStream_t stream) {
  const bool f16 = dt == kDtF16;
  switch (D) {
    case 32:
      return f16 ? bwd_seq_dispatch<_Float16, 32>(dout, q, k, v, out, lse, cu, items, B, N, H, win, ld, scale, dq, dk, dv,
                                                 nl, nd, stream)
                 : bwd_seq_dispatch<__bf16, 32>(dout, q, k, v, out, lse, cu, items, B, N, H, win, ld, scale, dq, dk, dv,
                                               nl, nd, stream);
    case 64:
      return f16 ? bwd_seq_dispatch<_Float16, 64>(dout, q, k, v, out, lse, cu, items, B, N, H, win, ld, scale, dq, dk, dv,
                                                 nl, nd, stream)
                 : bwd_seq_dispatch<__bf16, 64>(dout, q, k, v, out, lse, cu, items, B, N, H, win, ld, scale, dq, dk, dv,
                                               nl, nd, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pe
