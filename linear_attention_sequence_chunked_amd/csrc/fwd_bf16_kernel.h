// Chunkwise gated-delta-rule forward for bfloat16 inputs on MFMA (gfx950): the
// kernel, as a body that a launch of its own (fwd_bf16.hip) or a launch shared
// with other roles (the backward's two walks, bwd_bf16.hip) runs.  The design
// notes are at the top of fwd_bf16.hip.
#pragma once

#include "launch.h"
#include "mfma_common.h"

namespace gdn {
namespace {


using namespace mfma;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
// Ragged batches of up to this many sequences start their longest sequences first.
constexpr int kLongestFirstMax = 128;

// Row stride (elements) of the CP x CP bf16 tiles P^T and Tm^T: 160-byte rows
// at CP = 64 (16-byte aligned for the diagonal blocks' row writes; the
// transpose reads of 4 rows x 32 bytes then fall on distinct banks).
__host__ __device__ constexpr int tile_ld(int cp) { return cp == 64 ? cp + 16 : cp + 8; }

// P^T is written by 8-byte transposed accumulator stores (16 lanes: 16 rows, one
// 8-byte chunk each) and read by 8-byte transpose reads (16 lanes: 4 rows x 4
// chunks), nothing wider, so its 8-byte chunks are swizzled within each 16-column
// tile: chunk j of row i sits at chunk j ^ ((i / 4) % 4) of the tile.  Rows i and
// i + 4 then put the same chunk on different banks, and both access patterns are
// conflict-free.  p_chunk gives the swizzled chunk (in elements) for tile-local
// chunk j (0..3) of row i.
__host__ __device__ constexpr int p_chunk(int j, int i) { return 4 * (j ^ ((i >> 2) & 3)); }

// The fp32 diagonal A blocks are stored transposed, 16 floats per row, with the
// four 16-byte quads of row c permuted: quad u of row c sits at ad_quad(u, c).
// The permutation differs for any two of the rows a 16-byte store serves at once
// (c, c + 4, c + 8, c + 12, and c, c + 2, c + 4, c + 6), so the stores are
// conflict-free.
__host__ __device__ constexpr int ad_quad(int u, int c) { return 4 * ((u ^ ((c >> 1) ^ (c >> 3))) & 3); }

// SQ = false: a states-only layout without the query and P rings (the
// instance with 64 value rows needs that room for its value ring).
template <int KD, int VS, int CP, bool SQ = true>
struct alignas(16) Smem {
  static constexpr int NTB = CP / 16;
  // key and query rows: KD + 16 elements, a stride of 32 bytes modulo 64, which
  // keeps the 16-byte fragment reads (lanes 0-7 and 16-23 served together, rows
  // s and pieces g) on distinct banks: 2x the read rate of an 8-element pad
  static constexpr int LDK = KD + 16;
  static constexpr int LDC = tile_ld(CP);  // CP x CP tiles
  static constexpr int LDA = 24;       // packed 16-wide A^T blocks
  static constexpr int APK = (NTB == 4 ? 96 : 16) * LDA;
  bf16 k[3][CP * LDK];                 // keys [token][channel], padded rows
  bf16 q[2][SQ ? CP * LDK : 8];        // queries, padded rows
  // value slice [token][v]; rows of 96 bytes keep the transpose reads of 8
  // consecutive token rows on distinct banks
  static constexpr int LDV = (VS == 16 || VS == 32) ? 48 : VS + 16;
  bf16 v[2][CP * LDV];
  struct Gates {
    float gl[CP];                      // cumulative log2 gate
    float gam[CP];                     // 2^g
    float beta[CP];
    float bg[CP];                      // beta * gam
    float dn[CP];                      // gam_n / gam
  } gt[3];
  // offsets (in floats) of the gate vectors from gl within one slot
  static constexpr int GAM = CP, BETA = 2 * CP, BG = 3 * CP, DN = 4 * CP;
  bf16 pt[2][SQ ? CP * LDC : 8];                // P^T: pt[i][r]
  bf16 tt[2][CP * LDC];                // Tm^T: tt[j][i]; upper blocks zero
  bf16 ap[2][APK];                     // off-diagonal A^T blocks used by the levels
  // diagonal A blocks, fp32, transposed [c][r]; blocks ADS floats apart so the
  // four blocks read at once by the diagonal solve fall on different banks
  static constexpr int ADS = 256 + 4;
  float ad[NTB * ADS];
  int lens[kLongestFirstMax];          // ragged batch: sequence lengths (start order)
  int pick;
};

// Off-diagonal blocks of Tm = (I + A)^-1 from its diagonal blocks (already in
// tt) and the packed off-diagonal A^T blocks, in two levels of block products:
//   level 1: Tm_10 = -Tm_11 (A_10 Tm_00),  Tm_32 = -Tm_33 (A_32 Tm_22)
//   level 2: Tm_[23][01] = -Tm_[23] (A_[23][01] Tm_[01])
// Two waves share the work: both compute level 1 (identical values, written
// twice), then each computes one 16-column block bj = part of level 2.  The
// inner products A Tm stay in registers: their accumulator tiles become the
// next product's operand (k = their rows) through the permlane conversion, with
// the same bf16 rounding a trip through LDS would give.
template <int CP>
__device__ __forceinline__ void levels_part(bf16* tt, const bf16* ap, int lane, int part) {
  constexpr int NTB = CP / 16;
  constexpr int LDC = tile_ld(CP), LDA = 24;
  if constexpr (NTB == 4) {
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int bi = 2 * pr + 1, bj = 2 * pr;
      const f32x4 X = mma(frag_cols16(ap + 16 * pr * LDA, LDA, 0, 0, lane),
                          frag_rows16(tt, LDC, 16 * bj, 16 * bj, lane), zero4());
      const f32x4 Tij = mma(frag_cols16(tt, LDC, 16 * bi, 16 * bi, lane), acc_pair_to_frag(X, zero4()),
                            zero4());
      store_tile_t(tt, LDC, 16 * bj, 16 * bi, -Tij, lane);
    }
    const int bj = part;
    f32x4 X2[2];
#pragma unroll
    for (int bi = 2; bi < 4; ++bi)
      X2[bi - 2] = mma(frag_cols(ap + (bi == 2 ? 32 : 64) * LDA, LDA, 0, 0, lane),
                       frag_rows(tt, LDC, 16 * bj, 0, lane), zero4());
    const bf16x8 xb = acc_pair_to_frag(X2[0], X2[1]);
#pragma unroll
    for (int bi = 2; bi < 4; ++bi) {
      const f32x4 Tij = mma(frag_cols(tt, LDC, 16 * bi, 32, lane), xb, zero4());
      store_tile_t(tt, LDC, 16 * bj, 16 * bi, -Tij, lane);
    }
  } else {
    if (part != 0) return;
    const f32x4 X = mma(frag_cols16(ap, LDA, 0, 0, lane), frag_rows16(tt, LDC, 0, 0, lane), zero4());
    const f32x4 Tij = mma(frag_cols16(tt, LDC, 16, 16, lane), acc_pair_to_frag(X, zero4()), zero4());
    store_tile_t(tt, LDC, 0, 16, -Tij, lane);
  }
}

// Gram tiles of one chunk for token-block rows R0 and R1 (compile-time, so all
// fragments stay in registers).  TYPE 0 builds A (strictly lower, beta and
// decay applied; diagonal blocks to `ad` in fp32, the off-diagonal blocks the
// solve needs to `ap`), TYPE 1 builds P (lower, decay applied) into the P ring,
// TYPE 2 builds both from one read of the key fragments.  The key fragments of
// rows 0..R1 are read once and reused across tiles.
template <int KD, int CP, int TYPE, int R0, int R1, typename SM>
__device__ __forceinline__ void gram_rows(SM& sm, int c, int lane) {
  constexpr bool DA = TYPE != 1, DP = TYPE != 0;
  constexpr int KS = KD / 32;
  constexpr int LDC = SM::LDC, LDA = SM::LDA;
  const int ls = lane & 15, lg = lane >> 4;
  const int gs = c % 3;
  constexpr int LDK = SM::LDK;
  const lbf16* kr = pin(lds(sm.k[gs]) + rows_lane(LDK, lane));
  const lbf16* qr = pin(lds(sm.q[c % 2]) + rows_lane(LDK, lane));
  const lf32* gl = lds(sm.gt[gs].gl);
  const lf32* g1 = pin(gl + ls);
  const lf32* g4 = pin(gl + 4 * lg);
  constexpr int BOFF = SM::BETA;
  // Every operand and gate value is requested before the first MFMA, gates
  // first and fragments in k-step order, so the first round of MFMAs waits only
  // for its own fragments.
  bf16x8 kf[R1 + 1][KS], af[2][KS];
  f32x4 gr[2], br[2];
  float gi[R1 + 1];
#pragma unroll
  for (int tb = 0; tb <= R1; ++tb) gi[tb] = g1[16 * tb];
#pragma unroll
  for (int ri = 0; ri < 2; ++ri) {
    const int tr = ri == 0 ? R0 : R1;
    gr[ri] = *reinterpret_cast<const lf32x4*>(g4 + 16 * tr);
    if (DA) br[ri] = *reinterpret_cast<const lf32x4*>(g4 + BOFF + 16 * tr);
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int tb = 0; tb <= R1; ++tb) kf[tb][ks] = ld8(kr + 16 * tb * LDK + 32 * ks);
    if (DP) {
#pragma unroll
      for (int ri = 0; ri < 2; ++ri) af[ri][ks] = ld8(qr + 16 * (ri == 0 ? R0 : R1) * LDK + 32 * ks);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // All tiles advance together over the k-steps (independent accumulators); the
  // scheduling barrier after each round keeps that order.
  constexpr int NT0 = R0 + 1, NTILE = R0 + 1 + R1 + 1;
  f32x4 accA[NTILE], accP[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) accA[t] = accP[t] = zero4();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      const int ri = t < NT0 ? 0 : 1;
      const int tr = ri == 0 ? R0 : R1;
      const int tc = ri == 0 ? t : t - NT0;
      if (DA) accA[t] = mma(kf[tr][ks], kf[tc][ks], accA[t]);
      if (DP) accP[t] = mma(af[ri][ks], kf[tc][ks], accP[t]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // Decay 2^(g_r - g_i).  Diagonal tiles: per element, masked before the
  // exponential.  Off-diagonal tiles (every i < r): 2^(g_r - g_ref) 2^(g_ref - g_i)
  // with g_ref the gate of the row block's first token (broadcast from lane 0's
  // column gates), both factors <= 1; the row factor is shared by the row
  // block's tiles.
  float gref[2];
  f32x4 rowf[2];
#pragma unroll
  for (int ri = 0; ri < 2; ++ri) {
    gref[ri] = bits_f(__builtin_amdgcn_readlane(f_bits(gi[ri == 0 ? R0 : R1]), 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) rowf[ri][e] = __builtin_amdgcn_exp2f(gr[ri][e] - gref[ri]);
  }
  lbf16* pw = nullptr;
  lbf16* aw = nullptr;
  lf32* adw = nullptr;
  if (DP) pw = pin(lds(sm.pt[c % 2]) + ls * LDC + p_chunk(lg, ls));  // row 16 tc + ls, chunk lg
  if (DA) {
    aw = pin(lds(sm.ap[c % 2]) + ls * LDA + 4 * lg);
    adw = pin(lds(sm.ad) + ls * 16 + ad_quad(lg, ls));
  }
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int ri = t < NT0 ? 0 : 1;
    const int tr = ri == 0 ? R0 : R1;
    const int tc = ri == 0 ? t : t - NT0;
    const int i = 16 * tc + ls;
    // per-element decay of this tile, shared by A and P (the mask differs on
    // the diagonal: strict for A, inclusive for P)
    f32x4 decA, decP;
    if (tc == tr) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * tr + 4 * lg + e;
        const float d = gr[ri][e] - gi[tc];
        if (DA) decA[e] = __builtin_amdgcn_exp2f(i < r ? d : -INFINITY);
        if (DP) decP[e] = __builtin_amdgcn_exp2f(i <= r ? d : -INFINITY);
      }
    } else {
      const float colf = __builtin_amdgcn_exp2f(gref[ri] - gi[tc]);
#pragma unroll
      for (int e = 0; e < 4; ++e) decA[e] = decP[e] = rowf[ri][e] * colf;
    }
    // accumulator tiles are stored transposed: lane (g, s) writes row s of the
    // transposed tile, 4 consecutive bf16 (or fp32) at column 4g
    if (DP) {
      f32x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = decP[e] * accP[t][e];
      *reinterpret_cast<lds_bf16x4*>(pw + 16 * tc * LDC + 16 * tr) =
          bf16x4{(bf16)val[0], (bf16)val[1], (bf16)val[2], (bf16)val[3]};
    }
    if (DA) {
      f32x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = br[ri][e] * (decA[e] * accA[t][e]);
      if (tc == tr) {
        *reinterpret_cast<lf32x4*>(adw + tr * SM::ADS) = val;  // [c][r]
      } else {
        // packed A^T blocks: (1,0) -> 0, (3,2) -> 16, (2,0..1) -> 32.., (3,0..1) -> 64..
        const int off = tr == 1 ? 0 : (tr == 3 && tc == 2 ? 16 : (tr == 2 ? 32 : 64) + 16 * tc);
        *reinterpret_cast<lds_bf16x4*>(aw + off * LDA) =
            bf16x4{(bf16)val[0], (bf16)val[1], (bf16)val[2], (bf16)val[3]};
      }
    }
  }
}

// WO: the output o is produced.  Without it (states only: o == NULL) queries,
// P, Z and O are skipped entirely.
template <int KD, int VS, int CP, bool WO, bool SQ = true>
__device__ __forceinline__ void
fwd_bf16_body(Smem<KD, VS, CP, SQ>& sm, const int bid, const int nblk,
              const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
              const float* __restrict__ alpha, const float* __restrict__ beta,
              const float* __restrict__ s0, bf16* __restrict__ o, float* __restrict__ s_final,
              float* __restrict__ s_ckpt, bf16* __restrict__ s_ckpt_h, const int* __restrict__ cu,
              int T, int H, int K, int V, int C, int nslice) {
  using SM = Smem<KD, VS, CP, SQ>;
  static_assert(SQ || !WO, "outputs need the query and P rings");
  constexpr int LDC = SM::LDC;
  constexpr int NTB = CP / 16;          // token blocks per chunk tile
  constexpr int NCB = KD / 16;          // key-channel blocks
  constexpr int KS = KD / 32;           // k-steps over key channels
  constexpr int CS = CP / 32;           // k-steps over tokens
  constexpr int NCH = VS / 16;          // chain waves (one per 16 value rows)
  constexpr int W_LEV = NCH;            // levels wave
  constexpr int W_DIAG = NCH + 1;       // diagonal-solve wave
  constexpr int W_G0 = NCH + 2;         // first Gram / staging wave
  constexpr int NG = kWaves - W_G0;     // Gram / staging waves
  // the gates go to the Gram wave whose SIMD partner (the levels wave) is idle
  // while chunks are staged
  constexpr int W_GATE = W_G0 + (NG >= 3 ? 2 : 0);
  static_assert(NG >= 2, "need at least two Gram waves");
  // Issue priority with outputs, 64-token chunks and two chain waves: the Gram
  // waves that build A first, then the chain waves, then the rest (6% faster
  // than equal priorities on the training shape).  Equal priorities are faster
  // for the states-only instance, one chain wave and 32-token chunks.
  constexpr bool kPrio = WO && NTB == 4 && NCH == 2;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ls = lane & 15, lg = lane >> 4;

  // XCD-aware mapping: consecutive workgroup ids go to different XCDs (id mod 8),
  // so give the slices of one stream ids that are equal modulo 8 (same XCD,
  // shared L2).  A dense batch gives each XCD a contiguous run of slices (the
  // heads of one sequence then share the lines of the [B, T, H] gates).  In a
  // ragged batch, when the (stream, head) pairs divide evenly, pair p goes to
  // XCD p mod 8 instead, which spreads long and short sequences over all XCDs.
  int item = bid;
  const bool spread = cu && (nblk / nslice) % 8 == 0;
  if (spread) {
    const int xcd = bid & 7, slot = bid >> 3;
    item = ((slot / nslice) * 8 + xcd) * nslice + slot % nslice;
  } else if ((nblk & 7) == 0) {
    item = (bid & 7) * (nblk >> 3) + (bid >> 3);
  }
  const bool pair_order = spread || (nblk & 7) != 0;  // ids start in pair order
  const int slice = item % nslice;
  const int bh = item / nslice;
  const int h = bh % H;
  int b = bh / H;
  // Ragged batch: the pair started r-th takes a sequence of length rank r / H
  // (longest first, equal lengths in table order), so that the longest chains
  // are not left to start after the short ones.  The ranks come from the
  // clamped table below and form a permutation, so exactly one thread picks.
  const int nseq = nblk / (H * nslice);
  if (cu && pair_order && nseq <= kLongestFirstMax) {
    for (int j = tid; j < nseq; j += kThreads) {
      const int s = min(max(cu[j], 0), T), e = min(max(cu[j + 1], s), T);
      sm.lens[j] = e - s;
    }
    __syncthreads();
    if (tid < nseq) {
      const int lc = sm.lens[tid];
      int rank = 0;
      for (int j = 0; j < nseq; ++j) {
        const int lj = sm.lens[j];
        rank += (lj > lc || (lj == lc && j < tid)) ? 1 : 0;
      }
      if (rank == b) sm.pick = tid;
    }
    __syncthreads();
    b = sm.pick;
  }
  const int v0 = slice * VS;
  const size_t tok_k = (size_t)H * K;
  const size_t tok_v = (size_t)H * V;
  const size_t state_base = ((size_t)b * H + h) * (size_t)V * K + (size_t)v0 * K;
  // This workgroup's sequence: row b of a dense batch, or the packed sequence
  // [cu[b], cu[b+1]) (offsets clamped into [0, T], so a bad table can give wrong
  // results but never an access outside the tensors).
  size_t seq0 = (size_t)b * T;
  int Tn = T;
  if (cu) {
    const int s = min(max(cu[b], 0), T), e = min(max(cu[b + 1], s), T);
    seq0 = s;
    Tn = e - s;
  }
  const int NT = (Tn + C - 1) / C;

  // ---- zero the P and Tm rings: their upper blocks are read as zeros
  for (int i = tid; i < 2 * CP * LDC; i += kThreads) {
    if constexpr (SQ) (&sm.pt[0][0])[i] = (bf16)0.0f;
    (&sm.tt[0][0])[i] = (bf16)0.0f;
  }

  // ---- chain waves: the state slice as S^T accumulator tiles.  Tile cb, lane
  // (g, s), element e holds S[16 vb + s][ch(cb, g) + e] with the key channels in
  // the order ch(cb, g) = 32 (cb / 2) + 8 g + 4 (cb % 2): the pair of tiles
  // (2 ks, 2 ks + 1) then gives lane group g channels 32 ks + 8 g .. + 7 in order,
  // which is the k order of a key-row fragment, so the state packs into the
  // operand of Y = K S^T and Z^T = S Q^T with no data moved between lanes.  The
  // state update's K^T reads fetch the channels in the same order.
  f32x4 S[NCB];
  const int vb = wave;  // value block of a chain wave
  auto chan = [&](int cb) { return 32 * (cb >> 1) + 4 * (cb & 1) + 8 * lg; };
  if (wave < NCH) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      S[cb] = zero4();
      if (s0 && chan(cb) < K)
        S[cb] = *reinterpret_cast<const f32x4*>(&s0[state_base + (size_t)(16 * vb + ls) * K + chan(cb)]);
    }
  }

  // ---- staging registers of the Gram waves (one chunk in flight)
  constexpr int NSL = 64 * NG;                       // staging lanes
  constexpr int KPIECES = CP * KD / 8;               // 16-byte pieces per key/query tile
  constexpr int VPIECES = CP * VS / 8;
  constexpr int KPL = (KPIECES + NSL - 1) / NSL;
  constexpr int VPL = (VPIECES + NSL - 1) / NSL;
  const int sl = tid - 64 * W_G0;                    // staging lane (valid on Gram waves)
  struct StageRegs {
    bf16x8 k[KPL], q[KPL], v[VPL];
    float a, b;
  };

  // Per-piece token row, global offset within a chunk and LDS offset: fixed
  // for a staging lane, so computed once.
  int krow[KPL], kgo[KPL], klo[KPL], vrow[VPL], vgo[VPL], vlo[VPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int p = sl + NSL * j;
    const int r = p / (KD / 8), ch = (p % (KD / 8)) * 8;
    krow[j] = (p < KPIECES && ch < K) ? r : CP;  // CP: never loaded or stored
    kgo[j] = r * (int)tok_k + ch;
    klo[j] = r * SM::LDK + ch;
  }
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int p = sl + NSL * j;
    const int r = p / (VS / 8), ch = (p % (VS / 8)) * 8;
    vrow[j] = p < VPIECES ? r : CP;
    vgo[j] = r * (int)tok_v + ch;
    vlo[j] = r * SM::LDV + ch;
  }

  auto load_chunk = [&](int c, StageRegs& R) {
    const int t0 = c * C;
    const int n = min(C, Tn - t0);
    const bf16* kb = k + (seq0 + t0) * tok_k + (size_t)h * K;
    const bf16* qb = q + (seq0 + t0) * tok_k + (size_t)h * K;
    const bf16* vbp = v ? v + (seq0 + t0) * tok_v + (size_t)h * V + v0 : nullptr;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      R.k[j] = zero8();
      R.q[j] = zero8();
      if (krow[j] < n) {
        R.k[j] = *reinterpret_cast<const bf16x8*>(kb + kgo[j]);
        if constexpr (WO) R.q[j] = *reinterpret_cast<const bf16x8*>(qb + kgo[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      R.v[j] = zero8();
      if (v && vrow[j] < n) R.v[j] = *reinterpret_cast<const bf16x8*>(vbp + vgo[j]);  // no v: zeros
    }
    R.a = 1.0f;
    R.b = 0.0f;
    if (wave == W_GATE && lane < n) {  // one Gram wave holds the gates
      const size_t go = (seq0 + t0 + lane) * H + h;
      R.a = alpha[go];
      R.b = beta[go];
    }
  };

  auto stage_chunk = [&](int c, const StageRegs& R) {
    const int ks = c % 3, qs = c % 2;
    // piece j of a staging lane sits NSL / (KD / 8) token rows below piece 0
    static_assert(NSL % (KD / 8) == 0 && NSL % (VS / 8) == 0, "staging pieces must tile rows");
    lbf16* kst = pin(lds(sm.k[ks]) + klo[0]);
    lbf16* qst = pin(lds(sm.q[qs]) + klo[0]);
    lbf16* vst = pin(lds(sm.v[qs]) + vlo[0]);
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      if (sl + NSL * j < KPIECES) {  // pieces past K are stored as zeros
        *reinterpret_cast<lds_bf16x8*>(kst + j * (NSL / (KD / 8)) * SM::LDK) = R.k[j];
        if constexpr (WO) *reinterpret_cast<lds_bf16x8*>(qst + j * (NSL / (KD / 8)) * SM::LDK) = R.q[j];
      }
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (vrow[j] < CP) *reinterpret_cast<lds_bf16x8*>(vst + j * (NSL / (VS / 8)) * SM::LDV) = R.v[j];
    if (wave == W_GATE) {
      const float la = (lane < CP) ? __builtin_amdgcn_logf(R.a) : 0.0f;  // log2; padding: alpha = 1
      const float bt = (lane < CP) ? R.b : 0.0f;
      const float g = wave_scan(la, lane);
      const float glast = bits_f(__builtin_amdgcn_readlane(f_bits(g), CP - 1));
      if (lane < CP) {
        const float gm = __builtin_amdgcn_exp2f(g);
        sm.gt[ks].gl[lane] = g;
        sm.gt[ks].gam[lane] = gm;
        sm.gt[ks].beta[lane] = bt;
        sm.gt[ks].bg[lane] = bt * gm;
        sm.gt[ks].dn[lane] = __builtin_amdgcn_exp2f(glast - g);
      }
    }
  };

  // Each role runs its own copy of the chunk loop (so the register allocator
  // sees one role's live values at a time); every copy executes exactly two
  // workgroup barriers per iteration, x = -2 .. NT-1.
  if (wave < NCH) {
    // ============================ chain waves ============================
    // Everything that depends on the state stays in registers: the state (as
    // S^T tiles), R and U become MFMA operands through permlane swaps.  Only
    // the chunk's K, Q, V, gates, Tm and P come from LDS.
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
    // the two pipeline-fill iterations (x = -2, -1) have no chain work
    for (int i = 0; i < 4; ++i) lds_barrier();
    for (int x = 0; x < NT; ++x) {
      lds_barrier();
      if (s_ckpt) {  // chunk-start state [B, H, NT, V, K] (for the backward)
        float* dst = s_ckpt + ((((size_t)b * H + h) * NT + x) * V + v0 + 16 * vb + ls) * (size_t)K;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          if (chan(cb) < K) *reinterpret_cast<f32x4*>(dst + chan(cb)) = S[cb];
      }
      if constexpr (!WO) {
        if (s_ckpt_h) {  // the same, rounded to bf16 (the MFMA backward's operand precision)
          bf16* dst = s_ckpt_h + ((((size_t)b * H + h) * NT + x) * V + v0 + 16 * vb + ls) * (size_t)K;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            if (chan(cb) < K)
              *reinterpret_cast<bf16x4*>(dst + chan(cb)) =
                  bf16x4{(bf16)S[cb][0], (bf16)S[cb][1], (bf16)S[cb][2], (bf16)S[cb][3]};
        }
      }
      const int gs = x % 3;
      constexpr int LDK = SM::LDK;
      const lbf16* kr = pin(lds(sm.k[gs]) + rows_lane(LDK, lane));      // K rows
      const lbf16* qr = pin(lds(sm.q[x % 2]) + rows_lane(LDK, lane));   // Q rows
      const lbf16* kc = pin(lds(sm.k[gs]) + cols_lane_tau(LDK, lane, 8));  // K^T by transpose reads
      const lbf16* vc = pin(lds(sm.v[x % 2]) + (4 * lg + (ls >> 2)) * SM::LDV + 16 * vb + 4 * (ls & 3));
      const lf32* g4 = pin(lds(&sm.gt[gs].beta[0]) + 4 * lg);             // per-row gate vectors
      const lf32* g1 = pin(lds(&sm.gt[gs].gam[0]) + ls);                  // per-column gates
      // ---- phase A: Y = K S^T and Z^T = S Q^T (the state operand has k = key
      // channel; as the B operand of Y and the A operand of Z^T it is the same
      // registers).
      // The k-step is the outer loop so the 2 NTB accumulators are independent;
      // fragments of k-step ks + 1 are requested before the MFMAs of ks.
      bf16x8 sbf[KS], ka[2][NTB], qa[2][NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        ka[0][tb] = ld8(kr + 16 * tb * LDK);
        if constexpr (WO) qa[0][tb] = ld8(qr + 16 * tb * LDK);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sbf[ks] = acc_pair_pack(S[2 * ks], S[2 * ks + 1]);
      f32x4 Y[NTB], Z[NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        Y[tb] = zero4();
        Z[tb] = zero4();
      }
      // the V values and gates R needs (one transpose read gives each lane
      // V[16 tb + 4g + e][16 vb + s], e = 0..3); requested after the products
      // (earlier, their reads slow the key and query fragment reads: 1.5%)
      bf16x4 vt[NTB];
      f32x4 bt[NTB], bgv[NTB];
      float gmt[NTB];
      auto load_r_operands = [&]() {
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          vt[tb] = tr4(vc + 16 * tb * SM::LDV);
          bt[tb] = *reinterpret_cast<const lf32x4*>(g4 + 16 * tb);
          bgv[tb] = *reinterpret_cast<const lf32x4*>(g4 + (SM::BG - SM::BETA) + 16 * tb);
          if constexpr (WO) gmt[tb] = g1[16 * tb];  // Z^T columns are tokens
        }
      };
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb) {
            ka[(ks + 1) & 1][tb] = ld8(kr + 16 * tb * LDK + 32 * (ks + 1));
            if constexpr (WO) qa[(ks + 1) & 1][tb] = ld8(qr + 16 * tb * LDK + 32 * (ks + 1));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          Y[tb] = mma(ka[ks & 1][tb], sbf[ks], Y[tb]);   // Y   [token][v]
          if constexpr (WO) Z[tb] = mma(sbf[ks], qa[ks & 1][tb], Z[tb]);   // Z^T [v][token]
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- R = diag(beta) V - diag(beta gam) Y, kept as the U = Tm R operand
      load_r_operands();
      f32x4 R[NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) R[tb][e] = bt[tb][e] * (float)vt[tb][e] - bgv[tb][e] * Y[tb][e];
        if constexpr (WO) Z[tb] = Z[tb] * gmt[tb];
      }
      // R, U and Up become operands with the tokens (their k) in tau order; Tm, P
      // and K^T are read in the same order
      bf16x8 rb[CS];
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) rb[cs] = acc_pair_pack(R[2 * cs], R[2 * cs + 1]);
      // K^T fragments of the state update: the first two tiles with Tm and P,
      // the others one tile ahead of their products
      bf16x8 kt[2][CS];
      auto load_kt = [&](int cb, bf16x8* dst) {
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) dst[cs] = frag_cols_tau_at(kc, LDK, 32 * (cb >> 1) + 4 * (cb & 1), 32 * cs);
      };
      lds_barrier();  // Tm_x is complete after this barrier
      load_kt(0, kt[0]);
      if constexpr (NCB > 1) load_kt(1, kt[1]);
      // ---- phase B: U = Tm R, O = diag(gam) Z + P U, S^T <- gam_n S^T + K^T Up
      const lbf16* tc = pin(lds(sm.tt[x % 2]) + cols_lane_tau(LDC, lane, 4));
      // P^T is swizzled (p_chunk): rows 4g + s/4 (+ multiples of 16), chunk s % 4
      const lbf16* pc = pin(lds(sm.pt[x % 2]) + (4 * lg + (ls >> 2)) * LDC + p_chunk(ls & 3, 4 * lg));
      bf16x8 tf[NTB][CS], pf[NTB][CS];
      f32x4 dnv[NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        dnv[tb] = *reinterpret_cast<const lf32x4*>(g4 + (SM::DN - SM::BETA) + 16 * tb);
#pragma unroll
        for (int cs = 0; cs < CS; ++cs)
          if (32 * cs <= 16 * tb + 15) {  // Tm and P are lower triangular
            tf[tb][cs] = frag_cols_tau_at(tc, LDC, 16 * tb, 32 * cs);
            if constexpr (WO) pf[tb][cs] = frag_cols_tau_at(pc, LDC, 16 * tb, 32 * cs);
          }
      }
      const float gam_n = sm.gt[gs].gam[CP - 1];
      // (no scheduling barrier here: letting the U products start while the later
      // Tm and P fragments arrive measured 0.7% faster)
      f32x4 U[NTB], Up[NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        U[tb] = zero4();
#pragma unroll
        for (int cs = 0; cs < CS; ++cs)
          if (32 * cs <= 16 * tb + 15) U[tb] = mma(tf[tb][cs], rb[cs], U[tb]);
        Up[tb] = U[tb] * dnv[tb];
      }
      bf16x8 ub[CS], upb[CS];
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) {
        ub[cs] = acc_pair_pack(U[2 * cs], U[2 * cs + 1]);
        upb[cs] = acc_pair_pack(Up[2 * cs], Up[2 * cs + 1]);
      }
      // S^T <- gam_n S^T + K^T Up  (A operand: K^T by transpose reads, k = token)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 acc = S[cb] * gam_n;
        bf16x8 cur[CS];
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) cur[cs] = kt[cb & 1][cs];
        if (cb + 2 < NCB) load_kt(cb + 2, kt[cb & 1]);
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) acc = mma(cur[cs], upb[cs], acc);
        S[cb] = acc;
      }
      // O^T = Z^T diag(gam) + U^T P^T: lane (g, s) ends with O[token 16 tb + s]
      // [v 16 vb + 4g .. 4g + 3], stored as one 8-byte write.
      const int t0 = x * C;
      const int n = min(C, Tn - t0);
      bf16* obase = o + (seq0 + t0) * tok_v + (size_t)h * V + v0 + 16 * vb + 4 * lg;
      if (WO && o)  // no output when only states are wanted
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        f32x4 O = Z[tb];
#pragma unroll
        for (int cs = 0; cs < CS; ++cs)
          if (32 * cs <= 16 * tb + 15) O = mma(ub[cs], pf[tb][cs], O);
        const int r = 16 * tb + ls;
        if (r < n)
          *reinterpret_cast<bf16x4*>(obase + (size_t)r * tok_v) = bf16x4{(bf16)O[0], (bf16)O[1], (bf16)O[2], (bf16)O[3]};
      }
    }
  } else if (wave == W_LEV) {
    // ============================ levels wave ============================
    for (int i = 0; i < 4; ++i) lds_barrier();
    for (int x = 0; x < NT; ++x) {
      lds_barrier();
      levels_part<CP>(sm.tt[x % 2], sm.ap[x % 2], lane, 0);
      lds_barrier();
    }
  } else if (wave == W_DIAG) {
    // ============================= diag wave =============================
    for (int x = -2; x < NT; ++x) {
      lds_barrier();
      // phase A: the second half of the off-diagonal solve of chunk x
      if (NTB == 4 && x >= 0) levels_part<CP>(sm.tt[x % 2], sm.ap[x % 2], lane, 1);
      lds_barrier();
      // phase B: diagonal blocks of chunk x + 1
      const int c = x + 1;
      if (c >= 0 && c < NT && lg < NTB) {
        // column j of (I + L_bb)^-1 by forward substitution in fp32;
        // acc[r] carries sum_{i<r} L[r][i] x_i.
        bf16* tt = sm.tt[c % 2];
        const int bb = lg, j = ls;
        const float* Lt = &sm.ad[bb * SM::ADS];  // Lt[c][r] = L[r][c]
        float xv[16], acc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          xv[r] = (r == j) ? 1.0f : ((r < j) ? 0.0f : -acc[r]);
          if (r < 15) {
            f32x4 col[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) col[u] = *reinterpret_cast<const f32x4*>(&Lt[r * 16 + ad_quad(u, r)]);
#pragma unroll
            for (int rr = r + 1; rr < 16; ++rr) acc[rr] = fmaf(col[rr >> 2][rr & 3], xv[r], acc[rr]);
          }
        }
        bf16x8 lo, hi;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          lo[r] = (bf16)xv[r];
          hi[r] = (bf16)xv[8 + r];
        }
        bf16* dst = &tt[(16 * bb + j) * LDC + 16 * bb];
        *reinterpret_cast<bf16x8*>(dst) = lo;
        *reinterpret_cast<bf16x8*>(dst + 8) = hi;
      }
    }
  } else {
    // ========================== Gram / staging waves ==========================
    // Chunk c is loaded into registers one iteration before it is staged in LDS.
    StageRegs R;
    load_chunk(0, R);
    const int gw = wave - W_G0;
    if constexpr (kPrio)
      if (gw >= 2 && gw <= 3) __builtin_amdgcn_s_setprio(2);  // the A waves
    for (int x = -2; x < NT; ++x) {
      lds_barrier();
      {
        const int c = x + 1;  // chunk whose Gram is built now
        // plan: (type, rows) per Gram wave.  type 0: A = K K^T, type 1: P = Q K^T.
        // Four token blocks are split as rows {0, 3} and {1, 2} for balance.  P
        // goes to the Gram waves that share a SIMD with the chain waves and A,
        // whose epilogue is the longer one, to those beside the levels and
        // diagonal waves (2-3% faster than the other way round).
        if (c >= 0 && c < NT) {
          if constexpr (NTB == 4 && !WO && NG == 2) {
            // states only with two Gram waves (64 value rows): both build A
            if (gw == 0) gram_rows<KD, CP, 0, 0, 3>(sm, c, lane);
            else gram_rows<KD, CP, 0, 1, 2>(sm, c, lane);
          } else if constexpr (NTB == 4) {
            switch (gw) {
              case 0: if constexpr (WO) gram_rows<KD, CP, 1, 0, 3>(sm, c, lane); break;
              case 1: if constexpr (WO) gram_rows<KD, CP, 1, 1, 2>(sm, c, lane); break;
              case 2: gram_rows<KD, CP, 0, 0, 3>(sm, c, lane); break;
              case 3: gram_rows<KD, CP, 0, 1, 2>(sm, c, lane); break;
              default: break;
            }
          } else {
            switch (gw) {
              case 0: gram_rows<KD, CP, 0, 0, 1>(sm, c, lane); break;
              case 1: if constexpr (WO) gram_rows<KD, CP, 1, 0, 1>(sm, c, lane); break;
              default: break;
            }
          }
        }
      }
      lds_barrier();
      {
        const int c = x + 2;  // chunk staged now; the registers are reloaded with c + 1
        if (c >= 0 && c < NT) {
          stage_chunk(c, R);
          if (c + 1 < NT) load_chunk(c + 1, R);
        }
      }
    }
  }

  // ---- final state (channel order as above)
  if (wave < NCH && s_final) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      if (chan(cb) < K)
        *reinterpret_cast<f32x4*>(&s_final[state_base + (size_t)(16 * vb + ls) * K + chan(cb)]) = S[cb];
  }
}

// The forward kernel: one workgroup per (stream, value slice).  bid and nblk are
// the workgroup's index and count among the forward's workgroups (a launch that
// also runs other roles passes its own numbering).
template <int KD, int VS, int CP, bool WO>
__global__ void __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                const float* __restrict__ alpha, const float* __restrict__ beta,
                const float* __restrict__ s0, bf16* __restrict__ o, float* __restrict__ s_final,
                float* __restrict__ s_ckpt, bf16* __restrict__ s_ckpt_h, const int* __restrict__ cu,
                int T, int H, int K, int V, int C, int nslice) {
  __shared__ Smem<KD, VS, CP> sm;
  fwd_bf16_body<KD, VS, CP, WO>(sm, blockIdx.x, gridDim.x, q, k, v, alpha, beta, s0, o, s_final,
                                s_ckpt, s_ckpt_h, cu, T, H, K, V, C, nslice);
}

}  // namespace
}  // namespace gdn
