// Building blocks shared by the attention kernels: tile geometry, staging of
// 64-row tiles through LDS, and the two MFMA products every kernel is made of.
//
// All products work on 32x32 output blocks of v_mfma_f32_32x32x16_bf16 / _f16
// (16-bit elements) or v_mfma_f32_32x32x2_f32 (fp32). In the 32x32 accumulator layout lane l,
// register i holds row 8*(i/4) + 4*(l/32) + (i%4), column l%32. Kernels place
// the index they keep per lane (a query in the forward and dQ kernels, a key in
// the dK/dV kernel) on the columns, so each lane owns one row of attention
// scores and the score block can be fed back as the B operand of the next
// product without leaving registers.
//
//   mma_rows_regs:  acc[32 x 32] += X[32 rows of an LDS tile] . Y^T,
//                   Y = the lane's own row held in registers; reduction over head_dim.
//   mma_tr_regs:    acc[d x 32]  += X[32 rows of an LDS tile]^T . P,
//                   P = a 32x32 accumulator block; reduction over the 32 rows.
//
// The reduction index of an MFMA may be permuted freely as long as A and B use
// the same order. mma_tr_regs uses the order in which the accumulator layout
// holds rows (lane half g owns rows 4g..4g+3 and 8+4g..8+4g+3 of every 16), and
// reads X^T in that order with ds_read_b64_tr_b16: within each group of 16
// lanes, lane i receives element i%4 of the 8-byte chunks addressed by lanes
// i/4 + 4j, j = 0..3, i.e. four consecutive rows of one column when lane s
// addresses row s/4 and columns 4*(s%4)..4*(s%4)+3.
#pragma once
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pe {

constexpr int kBlk = 64;       // rows per LDS stage
constexpr int kThreads = 256;  // 4 waves per block

typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

template <typename Et, int D>
struct Geo {
  using E = typename std::conditional<kIs16<Et>, uint16_t, float>::type;
  static constexpr int ES = kIs16<Et> ? 2 : 4;
  static constexpr int ROWB = D * ES;              // bytes of one head row
  static constexpr int CH = ROWB / 16;             // 16-byte chunks per head row
  static constexpr int EPC = 16 / ES;              // elements per chunk
  static constexpr int ST = kIs16<Et> ? D + 8 : D + 4;    // LDS row stride in elements
  static constexpr int TSZ = kBlk * ST;            // elements of one staged tile
  static constexpr int HALF = D / 2;               // head-dim elements per lane half
  // How the two lane halves split head_dim in an MFMA over it. Normally half g
  // holds elements g*HALF + 8s .. (16-bit) or g*HALF + s (fp32) at step s. For
  // 16-bit head dims whose half is not a whole number of 8-element chunks
  // (24, 40, ..., 120) the split is by chunks instead: half g holds chunk 2s + g
  // (elements 16s + 8g .. 16s + 8g + 7) at step s, so every operand is one aligned
  // 16-byte chunk, and the chunk of half 1 past the row at the last step is zero.
  // A and B operands always use the same split, so the product is unchanged.
  static constexpr bool CHUNKED = kIs16<Et> && HALF > 8 && HALF % 8 != 0;
  static constexpr int QS = kIs16<Et> ? (CHUNKED ? (D + 15) / 16 : (HALF + 7) / 8) : HALF;  // MFMA steps
  static constexpr int GOFF = CHUNKED ? 8 : HALF;  // lane half g starts at element g * GOFF
  static constexpr int SSTEP = CHUNKED ? 16 : 8;   // elements between the 16-bit steps
  static constexpr int DB = (D + 31) / 32;         // 32-row blocks over head_dim
  static constexpr int TOTCH = kBlk * CH;
  static constexpr int PER = (TOTCH + kThreads - 1) / kThreads;
};

// per-lane operand type of the products: an 8-element vector, or one float
template <typename Et>
struct RegT { using type = vec8<Et>; };
template <>
struct RegT<float> { using type = float; };

__device__ __forceinline__ u16x4 ds_read_tr16(const uint16_t* p) {
  const shortx4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)(p));
  return __builtin_bit_cast(u16x4, r);
}

// The same reads at an LDS byte address (a 32-bit LDS pointer value)
__device__ __forceinline__ u16x8 ds_read_b128_at(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u16x8*>(static_cast<size_t>(addr));
}
__device__ __forceinline__ u16x4 ds_read_tr16_at(uint32_t addr) {
  const shortx4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) shortx4*>(static_cast<size_t>(addr)));
  return __builtin_bit_cast(u16x4, r);
}

// max / sum of a value with the same lane of the other half wave
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The lane's share of its own head row as MFMA operands (the split of head_dim
// between the lane halves described at Geo); row_off is the element offset of
// the row's first element, g the lane half.
template <typename Et, int D>
__device__ __forceinline__ void load_row_regs(const void* base, int64_t row_off, int g, bool valid,
                                              typename RegT<Et>::type (&r)[Geo<Et, D>::QS]) {
  using G = Geo<Et, D>;
  const int64_t off = row_off + g * G::GOFF;
  if constexpr (kIs16<Et>) {
    const uint16_t* src = static_cast<const uint16_t*>(base) + off;
#pragma unroll
    for (int s = 0; s < G::QS; ++s) {
      u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
      if constexpr (G::CHUNKED) {
        if (valid && (s + 1 < G::QS || g == 0)) x = *reinterpret_cast<const u16x8*>(src + G::SSTEP * s);
      } else if (valid) {
        if constexpr (G::HALF >= 8) {
          x = *reinterpret_cast<const u16x8*>(src + 8 * s);
        } else {
#pragma unroll
          for (int j = 0; j < G::HALF; ++j) x[j] = src[j];
        }
      }
      r[s] = as_vec8<Et>(x);
    }
  } else {
    const float* src = static_cast<const float*>(base) + off;
#pragma unroll
    for (int s = 0; s < G::QS; ++s) r[s] = valid ? src[s] : 0.f;
  }
}

// Global -> registers for one 64-row tile of head h of a tensor whose rows are
// `ld` elements apart; rows >= row_lim are zero.
template <typename Et, int D>
__device__ __forceinline__ void tile_gload(const void* base, int row0, int row_lim, int64_t ld, int h,
                                           uint4 (&r)[Geo<Et, D>::PER]) {
  using G = Geo<Et, D>;
  const char* b = static_cast<const char*>(base);
#pragma unroll
  for (int p = 0; p < G::PER; ++p) {
    const int ch = threadIdx.x + p * kThreads;
    const int row = ch / G::CH, col = ch - row * G::CH;
    const int gr = row0 + row;
    if ((G::TOTCH % kThreads == 0 || ch < G::TOTCH) && gr < row_lim) {
      r[p] = *reinterpret_cast<const uint4*>(b + (static_cast<int64_t>(gr) * ld + static_cast<int64_t>(h) * D) * G::ES +
                                             col * 16);
    } else {
      r[p] = make_uint4(0, 0, 0, 0);
    }
  }
}

// Registers -> LDS tile [kBlk][ST], row-major.
template <typename Et, int D>
__device__ __forceinline__ void tile_store(typename Geo<Et, D>::E* tile, const uint4 (&r)[Geo<Et, D>::PER]) {
  using G = Geo<Et, D>;
#pragma unroll
  for (int p = 0; p < G::PER; ++p) {
    const int ch = threadIdx.x + p * kThreads;
    if (G::TOTCH % kThreads == 0 || ch < G::TOTCH) {
      const int row = ch / G::CH, col = ch - row * G::CH;
      *reinterpret_cast<uint4*>(tile + row * G::ST + col * G::EPC) = r[p];
    }
  }
}

// acc += X . Y^T over head_dim; X = rows row0..row0+31 of an LDS tile (row l%32
// for lane l), Y = the lane's row in registers.
template <typename Et, int D>
__device__ __forceinline__ void mma_rows_regs(const typename Geo<Et, D>::E* tile, int row0,
                                              const typename RegT<Et>::type (&y)[Geo<Et, D>::QS],
                                              floatx16& acc, int ql, int g) {
  using G = Geo<Et, D>;
  const typename G::E* xr = tile + (row0 + ql) * G::ST + g * G::GOFF;
#pragma unroll
  for (int st = 0; st < G::QS; ++st) {
    if constexpr (kIs16<Et>) {
      u16x8 a;
      if constexpr (G::CHUNKED) {
        a = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (st + 1 < G::QS || g == 0) a = *reinterpret_cast<const u16x8*>(xr + G::SSTEP * st);
      } else if constexpr (G::HALF >= 8) {
        a = *reinterpret_cast<const u16x8*>(xr + 8 * st);
      } else {
        a = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < G::HALF; ++j) a[j] = xr[j];
      }
      acc = mfma16<Et>(as_vec8<Et>(a), y[st], acc);
    } else {
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xr[st], y[st], acc, 0, 0, 0);
    }
  }
}

// acc[db] += X^T . P; X = rows row0..row0+31 of an LDS tile (reduction index),
// P = 32x32 accumulator block whose rows are those 32 tile rows.
template <typename Et, int D>
__device__ __forceinline__ void mma_tr_regs(const typename Geo<Et, D>::E* tile, int row0, const floatx16& p,
                                            floatx16 (&acc)[Geo<Et, D>::DB], int lane) {
  using G = Geo<Et, D>;
  const int ql = lane & 31, g = lane >> 5;
  if constexpr (kIs16<Et>) {
    const int sub = lane & 15, grp = (lane >> 4) & 1;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      vec8<Et> pb;
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = static_cast<Et>(p[8 * s + j]);
      const int rowa = row0 + 16 * s + 4 * g + (sub >> 2);
#pragma unroll
      for (int db = 0; db < G::DB; ++db) {
        int col = db * 32 + 16 * grp + 4 * (sub & 3);
        if constexpr (D % 32 != 0) col = min(col, D - 4);   // stay inside the row; zeroed below
        const u16x4 lo = ds_read_tr16(tile + rowa * G::ST + col);
        const u16x4 hi = ds_read_tr16(tile + (rowa + 8) * G::ST + col);
        u16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (D % 32 != 0) {
          if (db * 32 + ql >= D) a = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        acc[db] = mfma16<Et>(as_vec8<Et>(a), pb, acc[db]);
      }
    }
  } else {
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int row = row0 + 8 * (st >> 2) + 4 * g + (st & 3);
#pragma unroll
      for (int db = 0; db < G::DB; ++db) {
        const int d = db * 32 + ql;
        const float a = (D % 32 == 0 || d < D) ? tile[row * G::ST + d] : 0.f;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[st], acc[db], 0, 0, 0);
      }
    }
  }
}

// Store a [d x 32] accumulator (lane = row of the output, registers = head dim)
// to out[row][h][:], multiplied by `mul`.
template <typename Et, int D>
__device__ __forceinline__ void store_acc_row(void* outp, int64_t off, const floatx16 (&acc)[Geo<Et, D>::DB],
                                              float mul, int g) {
  using G = Geo<Et, D>;
  if constexpr (kIs16<Et> && D % 32 == 0) {
    // Pair the two half-waves (same row, alternate groups of 4 columns) through one
    // permlane32 swap per value, so each lane stores 8 consecutive columns (16 bytes)
    // instead of two runs of 4.
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        float mine[4], sent[4], got[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = acc[db][8 * k + e] * mul, b = acc[db][8 * k + 4 + e] * mul;  // columns 16k+4g+e, 16k+8+4g+e
          mine[e] = g == 0 ? a : b;
          sent[e] = g == 0 ? b : a;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(sent[e]), __float_as_uint(sent[e]), false, false);
          got[e] = __uint_as_float(g == 0 ? r[1] : r[0]);
        }
        // lane g = 0: columns 16k .. 16k+7 = own 0..3, partner's 4..7; g = 1: 16k+8 .. 16k+15
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = g == 0 ? mine[e] : got[e];
          v[4 + e] = g == 0 ? got[e] : mine[e];
        }
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = f32_to_h16<Et>(v[2 * e]) | (uint32_t(f32_to_h16<Et>(v[2 * e + 1])) << 16);
        uint16_t* O = static_cast<uint16_t*>(outp) + off + db * 32 + 16 * k + 8 * g;
        *reinterpret_cast<uint4*>(O) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    return;
  }
#pragma unroll
  for (int db = 0; db < G::DB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = db * 32 + 8 * i4 + 4 * g;
      if (d0 < D) {
        if constexpr (kIs16<Et>) {
          uint16_t* O = static_cast<uint16_t*>(outp) + off + d0;
          const uint32_t lo = f32_to_h16<Et>(acc[db][4 * i4 + 0] * mul) | (uint32_t(f32_to_h16<Et>(acc[db][4 * i4 + 1] * mul)) << 16);
          const uint32_t hi = f32_to_h16<Et>(acc[db][4 * i4 + 2] * mul) | (uint32_t(f32_to_h16<Et>(acc[db][4 * i4 + 3] * mul)) << 16);
          *reinterpret_cast<uint2*>(O) = make_uint2(lo, hi);
        } else {
          float* O = static_cast<float*>(outp) + off + d0;
          *reinterpret_cast<float4*>(O) = make_float4(acc[db][4 * i4 + 0] * mul, acc[db][4 * i4 + 1] * mul,
                                                      acc[db][4 * i4 + 2] * mul, acc[db][4 * i4 + 3] * mul);
        }
      }
    }
}

// The sequences one tile of kAttnTileRows packed rows touches: their offsets
// are staged in `cul` (at most kAttnTileRows + 2 entries) and the range of
// rows they span [lo, hi) is returned.
struct TileSpan {
  int r0, rend, ncu, lo, hi;
};

template <int NT = kThreads>
__device__ __forceinline__ TileSpan tile_span(const int32_t* __restrict__ cu, const int32_t* __restrict__ items,
                                              int t, int B, int N, int32_t* cul) {
  TileSpan s;
  s.r0 = t * kAttnTileRows;
  s.rend = min(s.r0 + kAttnTileRows, N);
  const int blo = items[t], nxt = items[t + 1];
  const int bhi = nxt >= B ? B - 1 : (cu[nxt] == s.rend ? nxt - 1 : nxt);
  // at most kAttnTileRows + 1 sequences touch a tile when every length is >= 1;
  // the clamp keeps LDS writes in bounds even for malformed offsets
  s.ncu = min(bhi - blo + 2, kAttnTileRows + 2);
  for (int i = threadIdx.x; i < s.ncu; i += NT) cul[i] = cu[blo + i];
  __syncthreads();
  s.lo = cul[0];
  s.hi = cul[s.ncu - 1];
  // rows past cu[B] (a row count given as a capacity) belong to no sequence;
  // a tile after the last sequence (items[t] == B) ends up empty
  s.rend = min(s.rend, s.hi);
  return s;
}

// [first, last) rows of the sequence holding `row` (binary search in cul).
__device__ __forceinline__ void own_range(const int32_t* cul, int ncu, int row, int& lo_out, int& hi_out) {
  int lo = 0, hi = ncu - 2;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cul[mid] <= row) lo = mid; else hi = mid - 1;
  }
  lo_out = cul[lo];
  hi_out = cul[lo + 1];
}

// Local (sliding-window) attention: narrow a row's own key range [lo, hi) to
// the keys within distance win of the row (win < 0: global attention).
__device__ __forceinline__ void band_limit(int row, int win, int& lo, int& hi) {
  if (win >= 0) {
    lo = max(lo, row - win);
    hi = min(hi, row + win + 1);
  }
}

// Set entries of a 32x32 score block outside [lo, hi) (row index relative to
// the block's first row, per register) to -inf.
__device__ __forceinline__ void mask_block(floatx16& s, int lo, int hi) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * (i >> 2) + (i & 3);
    if (r < lo || r >= hi) s[i] = -INFINITY;
  }
}

// ---------------------------------------------------------------- 16-bit tiles staged by LDS DMA
// bf16 or fp16 tiles of kBlk rows x D elements are copied global -> LDS by
// global_load_lds_dwordx4 (no registers, no VALU) into a ring of stages. Rows
// are not padded; instead the 16-byte chunk c of row r sits at position
// c ^ swz(r) of the row. With 64 LDS banks of 4 bytes this puts the 16 rows of
// one ds_read_b128 phase (same logical chunk) on 16 distinct bank groups, and
// the 4 rows x 4 chunks of one ds_read_b64_tr_b16 phase likewise.
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// byte offset of logical 16-byte chunk c of row r in a tile with CH chunks per row
template <int CH>
__device__ __forceinline__ int chunk_off(int r, int c) {
  return (r * CH + (c ^ (swz(r) & (CH - 1)))) * 16;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<size_t>((__attribute__((address_space(3))) const char*)(p)));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(0) issued through the builtin, so the compiler's own wait
// tracking knows every earlier VMEM load has completed (gfx9 encoding: expcnt
// and lgkmcnt left at their no-wait maxima).
__device__ __forceinline__ void vmem_fence_for_compiler() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Barrier without the memory fence of __syncthreads(): the waits that matter
// (LDS-DMA completion) are issued explicitly before it.
__device__ __forceinline__ void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }

// DMA instructions each thread issues per 16-bit tile of head dim D
template <int D>
constexpr int dma_per_tile() { return kBlk * (D / 8) / kThreads; }

// One LDS-DMA instruction: 16 bytes per lane from sbase + voff (sbase wave-
// uniform, voff per lane) to LDS bytes [lds, lds + 1024) of the wave, lane l
// writing lds + 16*l.
__device__ __forceinline__ void dma16(uint32_t lds, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
               "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// The same with 4 bytes per lane: lane l writes lds + 4*l.
__device__ __forceinline__ void dma4(uint32_t lds, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
               "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// A ring stage given as a constant (std::integral_constant) or at run time (int), and
// the other stage of a two-stage ring. A constant stage turns every LDS address of the
// stage into a lane offset plus an immediate.
template <typename S>
__device__ __forceinline__ int stage_of(S st) {
  if constexpr (std::is_integral<S>::value) return st;
  else return S::value;
}
template <typename S>
__device__ __forceinline__ auto other_stage(S st) {
  if constexpr (std::is_integral<S>::value) return 1 - st;
  else return std::integral_constant<int, 1 - S::value>{};
}

// A operand (8 16-bit elements along head_dim) of mma over a swizzled tile:
// row r, logical chunk c.
template <typename Et, int CH>
__device__ __forceinline__ vec8<Et> swz_read_b128(const uint16_t* tile, int r, int c) {
  return as_vec8<Et>(*reinterpret_cast<const u16x8*>(reinterpret_cast<const char*>(tile) + chunk_off<CH>(r, c)));
}

// Registers (as loaded by tile_gload) -> unpadded 16-bit tile of kBlk rows with
// XOR-swizzled 16-byte chunks.
template <int D>
__device__ __forceinline__ void tile_store_swz(uint16_t* tile, const uint4 (&r)[Geo<__bf16, D>::PER]) {
  using G = Geo<__bf16, D>;
  constexpr int CH = D / 8;
#pragma unroll
  for (int p = 0; p < G::PER; ++p) {
    const int ch = threadIdx.x + p * kThreads;
    if (G::TOTCH % kThreads == 0 || ch < G::TOTCH) {
      const int row = ch / CH, col = ch - row * CH;
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(tile) + chunk_off<CH>(row, col)) = r[p];
    }
  }
}

// The mma_rows_regs product over a swizzled 16-bit tile.
template <typename Et, int D>
__device__ __forceinline__ void mma_rows_swz(const uint16_t* tile, int row0, const vec8<Et> (&y)[D / 16],
                                             floatx16& acc, int ql, int g) {
  constexpr int CH = D / 8;
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    acc = mfma16<Et>(swz_read_b128<Et, CH>(tile, row0 + ql, g * (CH / 2) + st), y[st], acc);
}

// The 16 values of a 32x32 accumulator block as two 16-bit MFMA B operands.
template <typename Et>
__device__ __forceinline__ void acc_to_h16(const floatx16& p, vec8<Et> (&pb)[2]) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[s][j] = static_cast<Et>(p[8 * s + j]);
}

// acc[db] += X^T . P over a swizzled 16-bit tile (the mma_tr_regs product).
template <typename Et, int D>
__device__ __forceinline__ void mma_tr_swz(const uint16_t* tile, int row0, const vec8<Et> (&pb)[2],
                                           floatx16 (&acc)[D / 32], int lane) {
  constexpr int CH = D / 8;
  const int g = lane >> 5, sub = lane & 15, grp = (lane >> 4) & 1;
  const char* t = reinterpret_cast<const char*>(tile);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int rowa = row0 + 16 * s + 4 * g + (sub >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int c = 4 * db + 2 * grp + ((sub >> 1) & 1);
      const int within = 8 * (sub & 1);
      const u16x4 lo = ds_read_tr16(reinterpret_cast<const uint16_t*>(t + chunk_off<CH>(rowa, c) + within));
      const u16x4 hi = ds_read_tr16(reinterpret_cast<const uint16_t*>(t + chunk_off<CH>(rowa + 8, c) + within));
      const u16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[db] = mfma16<Et>(as_vec8<Et>(a), pb[s], acc[db]);
    }
  }
}

// Round the 16 probabilities of a 32x32 accumulator block to the 16-bit type
// (two MFMA B operands) and add their fp32 sum to l. The log-sum-exp needs the
// sum of the unrounded values: bf16 rounding would move it by up to 2^-9
// relative (fp16 by 2^-12).
template <typename Et>
__device__ __forceinline__ void probs_to_h16(const floatx16& p, vec8<Et> (&pb)[2], float& l) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[s][j] = static_cast<Et>(p[8 * s + j]);
  float acc0 = p[0], acc1 = p[1];  // two chains
#pragma unroll
  for (int i = 2; i < 16; i += 2) {
    acc0 += p[i];
    acc1 += p[i + 1];
  }
  l += acc0 + acc1;
}

}  // namespace pe
