// Flash-style forward of non-causal attention over packed sequences, and the
// first-token query variant.
//
// Work item = one tile of 128 consecutive packed query rows and a group of
// heads (as many as keep the launch wide). A tile may span several short
// sequences or sit inside one long document; its keys are those of every
// sequence it touches, and each query row masks keys outside its own sequence.
// Short queries and long documents thus share one launch without padding any
// sequence to a tile. The offsets of the tile's sequences are read once per
// block, and its K/V loads stream on from one head to the next.
//
// Each of the 4 waves owns 32 query rows. Per 64-key block staged in LDS:
//   S^T (32 keys x 32 queries) = K Q^T     (mma_rows_regs: K from LDS, Q in registers)
//   online softmax in base 2 (scale*log2(e) folded into one FMA)
//   O^T (d x 32 queries) += V^T P^T        (mma_tr_regs: V from LDS, P straight from S^T)
// Computing S transposed leaves every lane with one query and 16 of its keys,
// the layout the PV product needs as its B operand, so P never goes through LDS.
// For 16-bit types (d <= 64) each head's Q rows arrive by LDS DMA into a tile of
// the block's 128 rows, issued during the previous head's last key block, so a
// head switch does not wait for its Q (and the rows load whole, 8 lanes per
// 128-byte row, instead of one row per lane).
#include <algorithm>
#include <climits>
#include <type_traits>

#include "attn_common.h"

namespace pe {

namespace {

// the generic forward groups heads per block while the launch keeps this many blocks
// (2048-16384 measured; on ~30-token sequences 8192 gives 6 of 12 heads per block)
constexpr int64_t kFwdMinBlocks = 8192;

template <typename Et, int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const void* __restrict__ qp, const void* __restrict__ kp, const void* __restrict__ vp,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items, int32_t B, int32_t N,
    int32_t H, int32_t T, int32_t HG, int32_t win, int64_t ld, float c, void* __restrict__ op,
    float* __restrict__ lse) {
  using G = Geo<Et, D>;
  using E = typename G::E;
  // bf16 tiles with whole 16-byte chunks per lane half use the XOR-swizzled layout
  // (conflict-free for both the row reads and the transposing reads)
  constexpr bool SWZ = kIs16<Et> && D % 32 == 0;
  constexpr int TS = SWZ ? kBlk * D : G::TSZ;
  // 16-bit tiles: each head's Q rows come by LDS DMA into a tile of the block's 128 rows,
  // issued during the previous head's last key block; otherwise the next head's Q rows are
  // fetched one step early where the registers allow it
  constexpr bool QDMA = SWZ && D <= 64;  // (the d = 128 tile would cost a block per CU)
  constexpr bool PREFQ = !QDMA && D <= 32;
  constexpr int QCH = D / 8;                                  // 16-byte chunks per Q row
  constexpr int QNL = QDMA ? kAttnTileRows * QCH / kThreads : 1;  // DMA instructions per thread
  __shared__ __align__(16) E kt[2][TS];
  __shared__ __align__(16) E vt[2][TS];
  __shared__ __align__(16) uint16_t qtile[QDMA ? kAttnTileRows * D : 8];
  __shared__ int32_t cul[kAttnTileRows + 2];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int hgi = lin / T, t = lin - hgi * T;
  const int h0 = hgi * HG, nh = min(HG, H - h0);
  if (nh <= 0) return;  // block-uniform; the host's even grouping never leaves an empty group
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, ql = lane & 31, g = lane >> 5;

  // the sequences this tile touches; their keys are [sp.lo, sp.hi)
  const TileSpan sp = tile_span(cu, items, t, B, N, cul);
  if (sp.rend <= sp.r0) return;  // block-uniform: no rows in this tile

  // this lane's query row and its own key range [qk0, qk1) (the same for every head)
  const int qrow = sp.r0 + wv * 32 + ql;
  const bool qvalid = qrow < sp.rend;
  int qk0 = 0, qk1 = 0;
  if (qvalid) {
    own_range(cul, sp.ncu, qrow, qk0, qk1);
    band_limit(qrow, win, qk0, qk1);
  }
  const int wk0 = wave_min_i(qvalid ? qk0 : INT_MAX);  // keys any row of the wave needs
  const int wk1 = wave_max_i(qvalid ? qk1 : INT_MIN);
  const int mk0 = wave_max_i(qvalid ? qk0 : INT_MIN);  // keys every row of the wave needs
  const int mk1 = wave_min_i(qvalid ? qk1 : INT_MAX);
  const int64_t qoff = static_cast<int64_t>(qrow) * ld;

  typename RegT<Et>::type qr[G::QS];
  // Q DMA: thread slot j*256 + tid fills LDS chunk position j*256 + tid of the tile, i.e.
  // row pos / QCH, physical chunk pos % QCH, which holds logical chunk (pos % QCH) ^ swz(row);
  // rows past the tile's last one repeat it (their queries are not stored)
  uint32_t qdoff[QNL];
  if constexpr (QDMA) {
#pragma unroll
    for (int jn = 0; jn < QNL; ++jn) {
      const int pos = jn * kThreads + tid, r = pos / QCH, pc = pos - r * QCH;
      const int rr = min(r, sp.rend - 1 - sp.r0);
      qdoff[jn] = static_cast<uint32_t>(rr) * static_cast<uint32_t>(ld) * 2u + ((pc ^ (swz(r) & (QCH - 1))) * 16u);
    }
  }
  auto q_dma = [&](int h) __attribute__((always_inline)) {
    if constexpr (QDMA) {
      const char* base = static_cast<const char*>(qp) + (static_cast<int64_t>(sp.r0) * ld + static_cast<int64_t>(h) * D) * 2;
#pragma unroll
      for (int jn = 0; jn < QNL; ++jn)
        dma16(lds_addr(qtile) + static_cast<uint32_t>((jn * kThreads + wv * 64) * 16), base, qdoff[jn]);
    }
  };
  auto q_from_lds = [&]() __attribute__((always_inline)) {
    if constexpr (QDMA) {
#pragma unroll
      for (int st = 0; st < G::QS; ++st) qr[st] = swz_read_b128<Et, QCH>(qtile, wv * 32 + ql, g * (QCH / 2) + st);
    }
  };
  if constexpr (!QDMA) load_row_regs<Et, D>(qp, qoff + h0 * D, g, qvalid, qr);

  uint4 kr[G::PER], vr[G::PER];
  floatx16 o[G::DB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db) o[db] = floatx16{};
  float m = kNegBig, l = 0.f;

  auto finish = [&](int h) __attribute__((always_inline)) {
    const float lt = xhalf_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qvalid) {
      store_acc_row<Et, D>(op, (static_cast<int64_t>(qrow) * H + h) * D, o, inv, g);
      if (lse != nullptr && g == 0) lse[static_cast<int64_t>(h) * N + qrow] = (m + log2f(lt)) * kLn2;
    }
#pragma unroll
    for (int db = 0; db < G::DB; ++db) o[db] = floatx16{};
    m = kNegBig;
    l = 0.f;
  };

  // one 64-key block of LDS tile `buf` against the lane's query row
  auto block = [&](int kb, int buf) __attribute__((always_inline)) {
    if (!(kb < wk1 && kb + kBlk > wk0)) return;
    floatx16 s[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      s[kk] = floatx16{};
      if constexpr (SWZ) mma_rows_swz<Et, D>(kt[buf], 32 * kk, qr, s[kk], ql, g);
      else mma_rows_regs<Et, D>(kt[buf], 32 * kk, qr, s[kk], ql, g);
    }
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
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kk][i]);
    mx = xhalf_max(mx);
    const float mnew = fmaxf(m, mx * c);
    if (__any(mnew > m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
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
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if constexpr (SWZ) {
        vec8<Et> pb[2];
        acc_to_h16<Et>(s[kk], pb);
        mma_tr_swz<Et, D>(vt[buf], 32 * kk, pb, o, lane);
      } else {
        mma_tr_regs<Et, D>(vt[buf], 32 * kk, s[kk], o, lane);
      }
    }
  };

  // keys of the tile: those of its sequences, and within win of its rows for local attention
  const int klo = win >= 0 ? max(sp.lo, sp.r0 - win) : sp.lo;
  const int khi = win >= 0 ? min(sp.hi, sp.rend + win) : sp.hi;
  const int nkb = klo < khi ? (khi - klo + kBlk - 1) / kBlk : 0;
  if (nkb == 0) {  // no keys at all (not reached by valid offsets): zero outputs
    for (int hh = 0; hh < nh; ++hh) finish(h0 + hh);
    return;
  }
  // Steps run over (head, key block) pairs, heads outer. The key blocks are the
  // same for every head, so the register-staged prefetch of the next step's
  // K and V rows runs on across the head boundary.
  q_dma(h0);  // waited for with the first K/V loads below
  tile_gload<Et, D>(kp, klo, khi, ld, h0, kr);
  tile_gload<Et, D>(vp, klo, khi, ld, h0, vr);
  int buf = 0, hh = 0, j = 0;
  const int nsteps = nh * nkb;
  for (int step = 0; step < nsteps; ++step) {
    const int kb = klo + j * kBlk;
    if constexpr (SWZ) {
      tile_store_swz<D>(kt[buf], kr);
      tile_store_swz<D>(vt[buf], vr);
    } else {
      tile_store<Et, D>(kt[buf], kr);
      tile_store<Et, D>(vt[buf], vr);
    }
    __syncthreads();
    const bool last = j + 1 == nkb;  // last key block of head h0 + hh
    if constexpr (QDMA) {
      // the DMA of this head's Q completed with the K/V loads waited for above (it was
      // issued before them); all waves read it here, then the tile is free again
      if (j == 0) {
        q_from_lds();
        if (last) __syncthreads();  // one key block per head: reads before the next DMA
      }
      if (last && hh + 1 < nh) q_dma(h0 + hh + 1);
    }
    if (step + 1 < nsteps) {
      const int hn = h0 + (last ? hh + 1 : hh);
      const int kn = last ? klo : kb + kBlk;
      tile_gload<Et, D>(kp, kn, khi, ld, hn, kr);
      tile_gload<Et, D>(vp, kn, khi, ld, hn, vr);
    }
    typename RegT<Et>::type qn[G::QS];
    const bool next_head = last && hh + 1 < nh;
    if (PREFQ && next_head) load_row_regs<Et, D>(qp, qoff + (h0 + hh + 1) * D, g, qvalid, qn);
    block(kb, buf);
    if (last) {
      finish(h0 + hh);
      if (next_head) {
        if constexpr (PREFQ) {
#pragma unroll
          for (int st = 0; st < G::QS; ++st) qr[st] = qn[st];
        } else if constexpr (!QDMA) {
          load_row_regs<Et, D>(qp, qoff + (h0 + hh + 1) * D, g, qvalid, qr);
        }
      }
      ++hh;
      j = 0;
    } else {
      ++j;
    }
    buf ^= 1;
  }
}

// ---------------------------------------------------------------- first-token query
// One block of kFirstThreads per (sequence, group of heads). Threads are laid out
// as [key slot][head][16-byte chunk of the head row]: the K and V rows of all
// heads of a key are contiguous, so every row of the sequence is read once,
// fully coalesced. Each key slot walks the keys slot, slot + KS, ... in batches
// of kFirstBatch rows whose loads are all issued before any is used (several
// HBM round trips in flight per thread), keeps its own running max, sum and
// output, and the slots merge through LDS at the end. A head row of GS chunks
// takes GSP lanes (GS rounded up to a power of two, for the butterfly sums);
// lanes past GS load nothing, add zero and store nothing.
constexpr int kFirstThreads = 512;

// Key slots per block of the first-token kernels: few for short sequences (a
// block then covers many heads of a row, read as one contiguous run), more as
// the length bound grows (a long sequence is one block's work, and its loads
// in flight scale with the slots): max_seq_len / 16, within [4, 32]. Defined
// at the end of this file (first_token_slots, declared in kernels.h).
constexpr int kFirstBatch = 4;

template <typename Et, int D>
__global__ __launch_bounds__(kFirstThreads) void attn_fwd_first_kernel(
    const void* __restrict__ qf, const void* __restrict__ kp, const void* __restrict__ vp,
    const int32_t* __restrict__ cu, int32_t B, int32_t N, int32_t H, int32_t HPB, int32_t gather, int64_t ld,
    float c, void* __restrict__ outp, float* __restrict__ lse) {
  constexpr int ES = kIs16<Et> ? 2 : 4;
  constexpr int EPC = 16 / ES;       // elements per 16-byte chunk
  constexpr int GS = D / EPC;        // chunks per head row
  constexpr int GSP = pow2_ceil(GS);  // lanes per head row
  constexpr int U = kFirstBatch;
  using Chunk = typename std::conditional<kIs16<Et>, u16x8, float4>::type;
  __shared__ float sm[kFirstThreads], sl[kFirstThreads];
  __shared__ float so[kFirstThreads * EPC];

  const int b = blockIdx.x;
  const int hg = blockIdx.y;
  const int tid = threadIdx.x;
  const int CPR = HPB * GSP;
  const int KS = kFirstThreads / CPR;
  const int slot = tid / CPR, cidx = tid - slot * CPR;
  const int hl = cidx / GSP, sub = cidx - hl * GSP;
  const int h = hg * HPB + hl;
  const bool active = slot < KS && h < H;
  const bool live = GS == GSP || sub < GS;  // the lane holds a chunk of the row

  const int c0 = cu[b], c1 = cu[b + 1];
  float qv[EPC], ov[EPC];
  float m = kNegBig, l = 0.f;
#pragma unroll
  for (int e = 0; e < EPC; ++e) ov[e] = 0.f;
  auto widen = [](const Chunk& x, float (&y)[EPC]) __attribute__((always_inline)) {
    if constexpr (kIs16<Et>) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) y[e] = h16_to_f32<Et>(x[e]);
    } else {
      y[0] = x.x; y[1] = x.y; y[2] = x.z; y[3] = x.w;
    }
  };
  if (active) {
    const int64_t hoff = static_cast<int64_t>(h) * D + sub * EPC;
    // the query is row b of q_first [B, H, D], or (gather) row cu[b] of the packed Q (rows ld apart)
    const int64_t qoff = gather ? static_cast<int64_t>(c0) * ld : static_cast<int64_t>(b) * H * D;
    if (live) {
      widen(*reinterpret_cast<const Chunk*>(static_cast<const char*>(qf) + (qoff + hoff) * ES), qv);
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) qv[e] = 0.f;
    }
    const char* kb = static_cast<const char*>(kp) + hoff * ES;
    const char* vb = static_cast<const char*>(vp) + hoff * ES;
    const int64_t rs = ld * ES;  // bytes between packed K/V rows
    for (int j0 = c0 + slot; j0 < c1; j0 += U * KS) {
      Chunk xk[U], xv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {  // rows past the sequence re-read its last row; their weight is 0
        const int j = min(j0 + u * KS, c1 - 1);
        if (live) {
          xk[u] = *reinterpret_cast<const Chunk*>(kb + j * rs);
          xv[u] = *reinterpret_cast<const Chunk*>(vb + j * rs);
        } else {
          __builtin_memset(&xk[u], 0, sizeof(Chunk));
          __builtin_memset(&xv[u], 0, sizeof(Chunk));
        }
      }
      float x[U];
      float bmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float kv[EPC];
        widen(xk[u], kv);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) s = fmaf(qv[e], kv[e], s);
#pragma unroll
        for (int o = 1; o < GSP; o <<= 1) s += __shfl_xor(s, o);
        x[u] = j0 + u * KS < c1 ? s * c : -INFINITY;
        bmax = fmaxf(bmax, x[u]);
      }
      const float mnew = fmaxf(m, bmax);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < EPC; ++e) ov[e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = __builtin_amdgcn_exp2f(x[u] - mnew);
        float vv[EPC];
        widen(xv[u], vv);
        l += p;
#pragma unroll
        for (int e = 0; e < EPC; ++e) ov[e] = fmaf(p, vv[e], ov[e]);
      }
      m = mnew;
    }
  }
  sm[tid] = m;
  sl[tid] = l;
#pragma unroll
  for (int e = 0; e < EPC; ++e) so[tid * EPC + e] = ov[e];
  __syncthreads();
  if (slot == 0 && h < H && live) {
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
    if constexpr (kIs16<Et>) {
      u16x8 y;
#pragma unroll
      for (int e = 0; e < EPC; ++e) y[e] = f32_to_h16<Et>(acc[e] * inv);
      *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(outp) + off) = y;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(outp) + off) =
          make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    }
    if (lse != nullptr && sub == 0) lse[static_cast<int64_t>(h) * B + b] = (M + log2f(L)) * kLn2;
  }
}

template <typename Et, int D>
hipError_t fwd_dispatch(const void* q, const void* k, const void* v, const int32_t* cu,
                        const int32_t* items, int32_t B, int32_t N, int32_t H, int32_t win, int64_t ld,
                        float scale, void* out, float* lse, hipStream_t stream) {
  const int T = (N + kAttnTileRows - 1) / kAttnTileRows;
  if (T == 0) return hipSuccess;
  // heads per block: as many as keep at least kFwdMinBlocks blocks in the launch
  int HG = static_cast<int>(std::min<int64_t>(H, std::max<int64_t>(1, static_cast<int64_t>(T) * H / kFwdMinBlocks)));
  const int HGN = (H + HG - 1) / HG;
  HG = (H + HGN - 1) / HGN;  // even groups
  const int64_t blocks = static_cast<int64_t>(T) * HGN;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipEvent_t ev_attn_fwd = timing_start(stream);
  hipLaunchKernelGGL((attn_fwd_kernel<Et, D>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                   q, k, v, cu, items, B, N, H, T, HG, win, ld, c, out, lse);
  timing_stop("attn_fwd", ev_attn_fwd, stream);
  return hipGetLastError();
}

template <typename Et, int D>
hipError_t first_dispatch(const void* q, const void* k, const void* v, const int32_t* cu, int32_t B,
                          int32_t N, int32_t H, int32_t max_seq_len, int32_t gather, int64_t ld, float scale,
                          void* out, float* lse, hipStream_t stream) {
  constexpr int GS = pow2_ceil(D / (kIs16<Et> ? 8 : 4));  // lanes per head row
  // heads per block: as many as leave the key slots wanted, then even groups
  const int HPB0 = std::max(1, std::min<int>(H, kFirstThreads / (GS * first_token_slots(max_seq_len))));
  const int HG = (H + HPB0 - 1) / HPB0;
  const int HPB = (H + HG - 1) / HG;
  const float c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipEvent_t ev_attn_fwd_first = timing_start(stream);
  hipLaunchKernelGGL((attn_fwd_first_kernel<Et, D>), dim3(B, HG), dim3(kFirstThreads), 0, stream, q, k, v, cu, B,
                   N, H, HPB, gather, ld, c, out, lse);
  timing_stop("attn_fwd_first", ev_attn_fwd_first, stream);
  return hipGetLastError();
}

}  // namespace

FwdList attn_fwd_list(int dt, int D, int max_seq_len, int64_t ld, int32_t H) {
  if (dt == kDtF32) return attn_f32_wave_supported(D, ld, H) ? kFwdListSeq32 : kFwdListPacked128;
  if (attn_fwd_short_supported(dt, D, max_seq_len)) return kFwdListNone;
  return attn_fwd_bf16_supported(D, max_seq_len) && attn_fwd_w64b_supported(D) ? kFwdListSeq128
                                                                                   : kFwdListPacked128;
}

hipError_t launch_attn_fwd(int dt, int D, const void* q, const void* k, const void* v,
                           const int32_t* cu, const int32_t* items, int32_t B, int32_t N, int32_t H,
                           int32_t max_seq_len, int32_t win, int64_t ld, float scale, void* out, float* lse,
                           hipStream_t stream) {
  const bool f16 = dt == kDtF16;
  switch (attn_fwd_list(dt, D, max_seq_len, ld, H)) {
    case kFwdListSeq32:
      return launch_attn_fwd_f32_wave(D, q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream);
    case kFwdListSeq128:
      return launch_attn_fwd_w64b(f16, D, q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream);
    case kFwdListNone:
      return launch_attn_fwd_short(f16, D, q, k, v, cu, B, N, H, win, ld, scale, out, lse, stream);
    case kFwdListPacked128:
      break;
  }
  if (dt != kDtF32 && attn_fwd_bf16_supported(D, max_seq_len))
    return launch_attn_fwd_bf16(f16, D, q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream);
#define PE_FWD_CASE(DD)                                                                                      \
  case DD:                                                                                                  \
    return dt == kDtF32 ? fwd_dispatch<float, DD>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream) \
           : f16        ? fwd_dispatch<_Float16, DD>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream) \
                        : fwd_dispatch<__bf16, DD>(q, k, v, cu, items, B, N, H, win, ld, scale, out, lse, stream);
  switch (D) {
    PE_HEAD_DIMS(PE_FWD_CASE)
    default: return hipErrorInvalidValue;
  }
#undef PE_FWD_CASE
}

hipError_t launch_attn_fwd_first(int dt, int D, const void* q_first, const void* k, const void* v,
                                 const int32_t* cu, int32_t B, int32_t N, int32_t H, int32_t max_seq_len,
                                 int32_t gather, int64_t ld, float scale, void* out_first, float* lse_first,
                                 hipStream_t stream) {
#define PE_FIRST_CASE(DD)                                                                                     \
  case DD:                                                                                                   \
    return dt == kDtF32  ? first_dispatch<float, DD>(q_first, k, v, cu, B, N, H, max_seq_len, gather, ld, scale, out_first,    \
                                                    lse_first, stream)                                           \
           : dt == kDtF16 ? first_dispatch<_Float16, DD>(q_first, k, v, cu, B, N, H, max_seq_len, gather, ld, scale, out_first, \
                                                       lse_first, stream)                                        \
                         : first_dispatch<__bf16, DD>(q_first, k, v, cu, B, N, H, max_seq_len, gather, ld, scale, out_first,    \
                                                     lse_first, stream);
  switch (D) {
    PE_HEAD_DIMS(PE_FIRST_CASE)
    default: return hipErrorInvalidValue;
  }
#undef PE_FIRST_CASE
}

int first_token_slots(int max_seq_len) { return std::max(4, std::min(32, max_seq_len / 16)); }

}  // namespace pe
