// Chunkwise gated-delta-rule backward for bfloat16 inputs on MFMA (gfx950).
//
// Same reverse mode as bwd.hip (the chunk algebra and its derivatives are
// written out at the top of that file: "Sparse Delta Memory: layer and
// kernels", section "What the layer computes"; operator contract of "OpenGDN
// 0.1.0", section "Core operator reference"), with chunks of C = 64 tokens and
// every matrix product on v_mfma_f32_16x16x32_bf16: bf16 operands, fp32
// accumulation.  Elementwise work, the triangular solve and all reductions are
// fp32.  Each output element has one writer and every sum a fixed order, so
// results are bitwise reproducible.
//
// Launches, all on the caller's stream:
//   (1) prep, one workgroup per chunk: gates, the Gram matrices A = diag(beta) M
//       and P, Tm = (I + A)^-1 in fp32 by 16 x 16 blocks; record = Tm, P
//       (bf16) and the gates (fp32);
//   (2) the two sequential walks, one launch, one workgroup per CU:
//       - the reverse walk, one workgroup per (stream, 32 value rows): the state
//         gradient dS^T lives in MFMA accumulator tiles across chunks (like the
//         forward's state); stores every chunk's end-state gradient dS'_c (bf16);
//       - the bf16 forward kernel's states-only body (fwd_bf16_kernel.h), one
//         workgroup per (stream, 32 value rows): the chunk-start states S_c,
//         rounded to bf16 (the precision (3) reads them in);
//   (3) token gradients, every chunk independent: one persistent workgroup per
//       CU taking the chunks in turn.  The gate gradients are sums of dP o P and
//       dA o M whose terms cancel (strongly so for correlated keys); their P and
//       M are recomputed here in fp32 (exact bf16 products summed in fp32, as
//       prep forms them before rounding) rather than read back as bf16, which
//       halves the error of dalpha in that regime.
//
// Layout conventions of the products in (3): quantities with a token axis and
// a value or channel axis are computed transposed (accumulator rows = value or
// channel, columns = tokens), so per-token scalars are one value per lane and
// the tiles go to LDS as row-major [token][*] with 8-byte writes; an operand
// whose contraction runs over tokens is then read from such an array with
// transpose reads.
#include "fwd_bf16_kernel.h"
#include "launch.h"
#include "mfma_common.h"

#include <atomic>
#include <type_traits>

namespace gdn {
namespace {

using namespace mfma;

constexpr int kC = 64;          // backward chunk (tokens)
constexpr int kLDC = kC + 8;    // row stride of C x C bf16 tiles in LDS
// Per-chunk record: Tm, P as bf16 [C][C] row-major (P lower, Tm unit lower),
// then g (cumulative log2 gate) and beta as fp32 [C].  Padding tokens past a
// sequence's end have alpha = 1 and beta = 0.
constexpr int kRecTm = 0, kRecP = kC * kC * 2;
constexpr int kRecG = 2 * kC * kC * 2, kRecB = kRecG + kC * 4;
constexpr int kRecBytes = kRecB + kC * 4;

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }

// Eight bf16 <- eight fp32 (round to nearest even).
__device__ __forceinline__ bf16x8 to_bf8(const float (&x)[8]) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)x[j];
  return r;
}

__device__ __forceinline__ void store_bf4(bf16* p, f32x4 d) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)d[0], (bf16)d[1], (bf16)d[2], (bf16)d[3]};
}

// ===========================================================================
// (1) prep: one workgroup (4 waves) per (chunk, head, batch).
// The key and query tiles are dead once the Gram is built, so A and Tm take
// their place (A is held in registers until every wave is done with the
// tiles): 36.5 KB at K = 128, so that three workgroups fit in a CU (768 chunks
// in one round on 256 CUs).
template <int KD>
struct alignas(16) PrepSmem {
  static constexpr int LDK = KD + 16;   // 32 bytes modulo 64: conflict-free fragment reads
  union {
    struct {
      bf16 k[kC * LDK], q[kC * LDK];   // [token][channel], read by the Gram only
    } in;
    struct {
      float x[kC][kC + 4];   // Tm (lower); upper blocks hold level scratch
      float a[kC][kC + 4];   // A = diag(beta) M, strictly lower
    } s;
  } u;
  float g[kC], bt[kC];
};

template <int KD>
__global__ void __launch_bounds__(256)
bwd16_prep_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                  const float* __restrict__ alpha, const float* __restrict__ beta,
                  unsigned char* __restrict__ rec, int T, int H) {
  using SM = PrepSmem<KD>;
  constexpr int LDK = SM::LDK;
  constexpr int KS = KD / 32;
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NT = (T + kC - 1) / kC;
  // one-dimensional grid over (chunk, head, batch), chunk fastest
  const int c = blockIdx.x % NT, h = (blockIdx.x / NT) % H, b = blockIdx.x / NT / H;
  const int t0 = c * kC, n = min(kC, T - t0);
  const size_t tok = (size_t)H * KD;
  unsigned char* dst = rec + (((size_t)b * H + h) * NT + c) * kRecBytes;
  bf16* rtm = reinterpret_cast<bf16*>(dst + kRecTm);
  bf16* rp = reinterpret_cast<bf16*>(dst + kRecP);

  // Every global read is issued before the first LDS write, so the chunk's
  // loads overlap instead of waiting one after another: keys and queries (zero
  // rows past the end; NP 16-byte pieces per thread) and, on wave 0, the gates
  // (padding alpha = 1, beta = 0).
  constexpr int NP = kC * KD / 8 / 256;
  bf16x8 kv[NP], qv[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int p = tid + 256 * j, r = p / (KD / 8), c8 = (p % (KD / 8)) * 8;
    kv[j] = zero8();
    qv[j] = zero8();
    if (r < n) {
      const size_t off = ((size_t)b * T + t0 + r) * tok + (size_t)h * KD + c8;
      kv[j] = *reinterpret_cast<const bf16x8*>(k + off);
      qv[j] = *reinterpret_cast<const bf16x8*>(q + off);
    }
  }
  float al = 1.0f, bt = 0.0f;
  if (wave == 0 && lane < n) {
    const size_t go = ((size_t)b * T + t0 + lane) * H + h;
    al = alpha[go];
    bt = beta[go];
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int p = tid + 256 * j, r = p / (KD / 8), c8 = (p % (KD / 8)) * 8;
    *reinterpret_cast<bf16x8*>(&sm.u.in.k[r * LDK + c8]) = kv[j];
    *reinterpret_cast<bf16x8*>(&sm.u.in.q[r * LDK + c8]) = qv[j];
  }
  // gates: g = cumulative log2(alpha) by a wave scan
  if (wave == 0) {
    const float g = wave_scan(__builtin_amdgcn_logf(al), lane);
    sm.g[lane] = g;
    sm.bt[lane] = bt;
    reinterpret_cast<float*>(dst + kRecG)[lane] = g;
    reinterpret_cast<float*>(dst + kRecB)[lane] = bt;
  }
  lds_barrier();

  // Gram tiles, balanced over the waves: waves 0 and 1 build A for token-block
  // rows {0, 3} and {1, 2}, waves 2 and 3 build P for the same rows (five tiles
  // each).  P goes to the record, A (strict) to fp32 LDS over the dead key and
  // query tiles once every wave has passed the barrier after the products;
  // the tiles above the diagonal are written as zeros.
  const int ls = lane & 15, lg = lane >> 4;
  {
    const bool isP = wave >= 2;
    const int ra = (wave & 1) ? 1 : 0, rb = (wave & 1) ? 2 : 3;
    const bf16* ab = isP ? sm.u.in.q : sm.u.in.k;
    // the lane's gates, read once: rows 16 w + 4 lg + e of its two token-block
    // rows, columns 16 tc + ls (no LDS read waits inside the element loop)
    float gr[2][4], br[2][4], gc[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int w = half == 0 ? ra : rb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gr[half][e] = sm.g[16 * w + 4 * lg + e];
        br[half][e] = sm.bt[16 * w + 4 * lg + e];
      }
    }
#pragma unroll
    for (int tc = 0; tc < 4; ++tc) gc[tc] = sm.g[16 * tc + ls];
    float av[2][4][4];   // decayed Gram entries: P, or A = diag(beta) M
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int w = half == 0 ? ra : rb;   // token-block row
#pragma unroll
      for (int tc = 0; tc < 4; ++tc) {
        f32x4 acc = zero4();
        if (tc <= w) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc = mma(frag_rows(ab, LDK, 16 * w, 32 * ks, lane), frag_rows(sm.u.in.k, LDK, 16 * tc, 32 * ks, lane), acc);
        }
        // accumulator: row r = 16 w + 4 lg + e, column i = 16 tc + ls
        const int i = 16 * tc + ls;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * w + 4 * lg + e;
          const float dec = __builtin_amdgcn_exp2f(i <= r ? gr[half][e] - gc[tc] : -INFINITY);
          av[half][tc][e] = isP ? dec * acc[e] : br[half][e] * (i < r ? dec * acc[e] : 0.0f);
        }
      }
    }
    if (isP) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int w = half == 0 ? ra : rb;
#pragma unroll
        for (int tc = 0; tc < 4; ++tc)
#pragma unroll
          for (int e = 0; e < 4; ++e) rp[(16 * w + 4 * lg + e) * kC + 16 * tc + ls] = (bf16)av[half][tc][e];
      }
    }
    lds_barrier();   // the key and query tiles are dead
    if (!isP) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int w = half == 0 ? ra : rb;
#pragma unroll
        for (int tc = 0; tc < 4; ++tc)
#pragma unroll
          for (int e = 0; e < 4; ++e) sm.u.s.a[16 * w + 4 * lg + e][16 * tc + ls] = av[half][tc][e];
      }
    }
  }
  lds_barrier();

  // Tm = (I + A)^-1 in fp32, by 16 x 16 blocks.
  // Diagonal blocks by forward substitution, one lane per (block, column):
  //   x_j = 1, x_r = -sum_{j <= i < r} A[r][i] x_i.
  if (wave == 0) {
    const int bb = lg, j = 16 * bb + ls;
    float xv[16];
    // the block's rows as four 16-byte reads each, row r + 1 requested while
    // row r is substituted
    auto row = [&](int r, f32x4 (&dst)[4]) {
#pragma unroll
      for (int m = 0; m < 4; ++m) dst[m] = *reinterpret_cast<const f32x4*>(&sm.u.s.a[16 * bb + r][16 * bb + 4 * m]);
    };
    f32x4 ra0[4], ra1[4];
    row(1, ra1);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      f32x4 (&cur)[4] = (r & 1) ? ra1 : ra0;
      f32x4 (&nxt)[4] = (r & 1) ? ra0 : ra1;
      if (r >= 1 && r + 1 < 16) row(r + 1, nxt);
      const int rr = 16 * bb + r;
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < r; ++i) s = fmaf(cur[i >> 2][i & 3], xv[i], s);
      xv[r] = rr < j ? 0.0f : (rr == j ? 1.0f : -s);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.u.s.x[16 * bb + r][j] = xv[r];
  }
  lds_barrier();
  // Off-diagonal blocks by levels d = i - j: X_ij = -T_ii (sum_{j <= m < i} A_im T_mj),
  // in fp32 on the matrix cores (16 x 16 x 4 per instruction: lane (s, g) gives
  // the left operand's row s and the right operand's column s at reduction index
  // g, and receives rows 4g .. 4g + 3 of column s).  Wave w takes the pair
  // (j, i) = (w, w + d) of level d.  Step one puts the inner sum into the (j, i)
  // block above the diagonal (scratch), which the same wave then reads back to
  // multiply by the diagonal block; levels are separated by barriers.
  for (int d = 1; d < 4; ++d) {
    if (wave + d < 4) {
      const int j = wave, i = wave + d;
      f32x4 x = zero4();
      for (int m0 = 16 * j; m0 < 16 * i; m0 += 4)
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.u.s.a[16 * i + ls][m0 + lg], sm.u.s.x[m0 + lg][16 * j + ls], x,
                                                 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.s.x[16 * j + 4 * lg + e][16 * i + ls] = x[e];
      // T_ii is lower triangular: its upper entries are zeros
      f32x4 y = zero4();
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4)
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.u.s.x[16 * i + ls][16 * i + k0 + lg],
                                                 sm.u.s.x[16 * j + k0 + lg][16 * i + ls], y, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.s.x[16 * i + 4 * lg + e][16 * j + ls] = -y[e];
    }
    lds_barrier();
  }
  // Tm to the record as bf16, zeros above the diagonal
  for (int p = tid; p < kC * kC / 8; p += 256) {
    const int r = p / (kC / 8), c8 = (p % (kC / 8)) * 8;
    float xr[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) xr[jj] = c8 + jj <= r ? sm.u.s.x[r][c8 + jj] : 0.0f;
    *reinterpret_cast<bf16x8*>(rtm + 8 * p) = to_bf8(xr);
  }
}

// ===========================================================================
// (2) reverse walk: one workgroup per (32 value rows, head, batch).  Waves 0
// and 1 carry dS^T for rows v0 + 16 w .. + 15 (tile cb: lane (g, s) holds
// dS[v0 + 16 w + s][16 cb + 4g + e]); the staging waves load the next chunk (in
// reverse order) into the other LDS slot.
// Per chunk with dS' the gradient of the chunk-end state:
//   W = K dS'^T,  dU = diag(D) W + P^T dO,  dR = Tm^T dU,
//   dS <- gam_n dS' + dO^T diag(gam) Q - dR^T diag(beta gam) K.
constexpr int kLDV = 48;  // [token][16 values] rows of 96 bytes (transpose reads)

template <int KD>
struct alignas(16) WalkSlot {
  static constexpr int LDK = KD + 16;   // 32 bytes modulo 64: conflict-free fragment reads
  bf16 k[kC * LDK], q[kC * LDK];   // [token][channel]
  bf16 tm[kC * kLDC], p[kC * kLDC];
  bf16 dob[kC * kLDV], dog[kC * kLDV];  // dO and diag(gam) dO: [token][32 values]
  float d[kC], nbg[kC];            // D_r = gam_n / gam_r,  -beta_r gam_r
  float gamn[4];
};

// The walk for one (32 value rows, head, batch) item, bid of nblk: waves 0 and 1
// carry the state gradient, the next NSW waves stage the chunks, and any further
// waves only keep the barrier count (every wave reaches each barrier).
template <int KD, int NSW>
__device__ __forceinline__ void
dstate_body(WalkSlot<KD>* slot, const int bid, const int nblk,
            const bf16* __restrict__ q, const bf16* __restrict__ k,
            const bf16* __restrict__ d_o, const float* __restrict__ d_sfinal,
            float* __restrict__ d_s0, const unsigned char* __restrict__ rec,
            bf16* __restrict__ ws_dS, int T, int H, int V) {
  using SL = WalkSlot<KD>;
  constexpr int LDK = SL::LDK;
  constexpr int KS = KD / 32, NCB = KD / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ls = lane & 15, lg = lane >> 4;
  // XCD-aware mapping (one-dimensional grid of B * H * V/32): consecutive
  // workgroup ids go to different XCDs, so the value slices of one (batch, head),
  // which read the same keys, queries and records, get ids equal modulo 8 (same
  // XCD, shared L2)
  int item = bid;
  if ((nblk & 7) == 0) item = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int nsl = V / 32, bh = item / nsl;
  const int v0 = (item - bh * nsl) * 32, h = bh % H, b = bh / H;
  const int NT = (T + kC - 1) / kC;
  const size_t tokk = (size_t)H * KD, tokv = (size_t)H * V;
  const unsigned char* rec_bh = rec + ((size_t)b * H + h) * NT * (size_t)kRecBytes;

  if (wave < 2) {
    const int vw = 16 * wave;   // this wave's value rows within the slot's 32
    const size_t sbase = ((size_t)b * H + h) * (size_t)V * KD + (size_t)(v0 + vw) * KD;
    // ============================== chain wave ==============================
    f32x4 dS[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      dS[cb] = d_sfinal ? *reinterpret_cast<const f32x4*>(&d_sfinal[sbase + (size_t)ls * KD + 16 * cb + 4 * lg])
                        : zero4();
    for (int c = NT - 1; c >= 0; --c) {
      lds_barrier();
      const SL& sl = slot[c & 1];
      // dS' of every chunk, rounded to bf16 (the token-gradient kernel's operand
      // precision)
      bf16* dst = ws_dS + (((size_t)b * H + h) * NT + c) * (size_t)V * KD + (size_t)(v0 + vw + ls) * KD + 4 * lg;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) store_bf4(dst + 16 * cb, dS[cb]);
      bf16x8 sbf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sbf[ks] = acc_pair_to_frag(dS[2 * ks], dS[2 * ks + 1]);
      // W = K dS'^T and P^T dO  ->  dU
      f32x4 dU[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 w = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) w = mma(frag_rows(sl.k, LDK, 16 * tb, 32 * ks, lane), sbf[ks], w);
        f32x4 pd = zero4();
#pragma unroll
        for (int cs = 0; cs < 2; ++cs)
          if (32 * cs + 31 >= 16 * tb)  // P^T is upper triangular
            pd = mma(frag_cols(sl.p, kLDC, 16 * tb, 32 * cs, lane), frag_cols(sl.dob, kLDV, vw, 32 * cs, lane), pd);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(&sl.d[16 * tb + 4 * lg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dU[tb][e] = fmaf(dd[e], w[e], pd[e]);
      }
      bf16x8 duf[2];
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) duf[cs] = acc_pair_to_frag(dU[2 * cs], dU[2 * cs + 1]);
      // dR = Tm^T dU, scaled by -beta gam for the update
      f32x4 dR[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 r = zero4();
#pragma unroll
        for (int cs = 0; cs < 2; ++cs)
          if (32 * cs + 31 >= 16 * tb) r = mma(frag_cols(sl.tm, kLDC, 16 * tb, 32 * cs, lane), duf[cs], r);
        const f32x4 nb = *reinterpret_cast<const f32x4*>(&sl.nbg[16 * tb + 4 * lg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dR[tb][e] = nb[e] * r[e];
      }
      bf16x8 drf[2], gof[2];
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) {
        drf[cs] = acc_pair_to_frag(dR[2 * cs], dR[2 * cs + 1]);
        gof[cs] = frag_cols(sl.dog, kLDV, vw, 32 * cs, lane);
      }
      const float gamn = sl.gamn[0];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 acc = dS[cb] * gamn;
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
          acc = mma(frag_cols(sl.q, LDK, 16 * cb, 32 * cs, lane), gof[cs], acc);
          acc = mma(frag_cols(sl.k, LDK, 16 * cb, 32 * cs, lane), drf[cs], acc);
        }
        dS[cb] = acc;
      }
    }
    if (d_s0)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        *reinterpret_cast<f32x4*>(&d_s0[sbase + (size_t)ls * KD + 16 * cb + 4 * lg]) = dS[cb];
  } else if (wave < 2 + NSW) {
    // ============================= staging waves =============================
    // Chunk c is loaded into registers two iterations before it is written to
    // LDS, in one of two register sets (alternating; the loop is unrolled by
    // two so that each set keeps its registers); 64 NSW staging lanes.  Every
    // load is unconditional (past the end of the sequence a row reads the
    // chunk's first row, past the first chunk the load repeats chunk 0) and the
    // values are zeroed where needed only when staged, so the wait before
    // staging a set leaves the other set's loads in flight.
    constexpr int NSL = 64 * NSW;
    constexpr int NKP = kC * KD / 8;              // 16-byte pieces of a key tile
    constexpr int KPL = NKP / NSL;
    constexpr int NMP = kC * kC / 8;              // pieces of a C x C tile
    constexpr int MPL = NMP / NSL;
    constexpr int DPL = kC * 4 / NSL;             // dO pieces (token, 8 values)
    static_assert(NKP % NSL == 0 && NMP % NSL == 0 && kC * 4 % NSL == 0, "staging pieces");
    const int sl = tid - 128;
    struct Regs {
      bf16x8 k[KPL], q[KPL], tm[MPL], p[MPL], dof[DPL];
      float g[DPL], gl, gn, bt;
    };
    auto load = [&](int c, Regs& R) {
      c = c > 0 ? c : 0;
      const int t0 = c * kC, n = min(kC, T - t0);
      const unsigned char* rc = rec_bh + (size_t)c * kRecBytes;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int p = sl + NSL * j, r = p / (KD / 8), c8 = (p % (KD / 8)) * 8;
        const size_t off = ((size_t)b * T + t0 + (r < n ? r : 0)) * tokk + (size_t)h * KD + c8;
        R.k[j] = *reinterpret_cast<const bf16x8*>(k + off);
        R.q[j] = *reinterpret_cast<const bf16x8*>(q + off);
      }
#pragma unroll
      for (int j = 0; j < MPL; ++j) {
        const int p = sl + NSL * j;
        R.tm[j] = *reinterpret_cast<const bf16x8*>(rc + kRecTm + 16 * p);
        R.p[j] = *reinterpret_cast<const bf16x8*>(rc + kRecP + 16 * p);
      }
      // dO pieces: piece p = sl + NSL j is token p / 4, values 8 (p % 4) .. + 7
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        const int p = sl + NSL * j, dr = p >> 2;
        R.dof[j] = *reinterpret_cast<const bf16x8*>(
            d_o + ((size_t)b * T + t0 + (dr < n ? dr : 0)) * tokv + (size_t)h * V + v0 + 8 * (p & 3));
        R.g[j] = reinterpret_cast<const float*>(rc + kRecG)[dr];
      }
      // gates of token sl (lanes sl >= 64 read token sl - 64 and are not staged);
      // the chunk's last gate is the same for every lane: through a vector
      // register offset it stays a vector load (a scalar load would be waited
      // for with the LDS counter)
      int z = 0;
      asm volatile("" : "+v"(z));
      R.gl = reinterpret_cast<const float*>(rc + kRecG)[sl & (kC - 1)];
      R.gn = reinterpret_cast<const float*>(rc + kRecG)[kC - 1 + z];
      R.bt = reinterpret_cast<const float*>(rc + kRecB)[sl & (kC - 1)];
    };
    auto stage = [&](int c, const Regs& R) {
      SL& s = slot[c & 1];
      const int n = min(kC, T - c * kC);
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int p = sl + NSL * j, r = p / (KD / 8), c8 = (p % (KD / 8)) * 8;
        *reinterpret_cast<bf16x8*>(&s.k[r * LDK + c8]) = r < n ? R.k[j] : zero8();
        *reinterpret_cast<bf16x8*>(&s.q[r * LDK + c8]) = r < n ? R.q[j] : zero8();
      }
#pragma unroll
      for (int j = 0; j < MPL; ++j) {
        const int p = sl + NSL * j, r = p / (kC / 8), c8 = (p % (kC / 8)) * 8;
        *reinterpret_cast<bf16x8*>(&s.tm[r * kLDC + c8]) = R.tm[j];
        *reinterpret_cast<bf16x8*>(&s.p[r * kLDC + c8]) = R.p[j];
      }
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        const int p = sl + NSL * j, dr = p >> 2, c8 = 8 * (p & 3);
        const bf16x8 dof = dr < n ? R.dof[j] : zero8();
        const float gm = __builtin_amdgcn_exp2f(R.g[j]);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = gm * bf2f(dof[e]);
        *reinterpret_cast<bf16x8*>(&s.dob[dr * kLDV + c8]) = dof;
        *reinterpret_cast<bf16x8*>(&s.dog[dr * kLDV + c8]) = to_bf8(x);
      }
      if (sl < kC) {
        s.d[sl] = __builtin_amdgcn_exp2f(R.gn - R.gl);
        s.nbg[sl] = -R.bt * __builtin_amdgcn_exp2f(R.gl);
        if (sl == 0) s.gamn[0] = __builtin_amdgcn_exp2f(R.gn);
      }
    };
    // chunk x_j = NT - 1 - j is staged at step j (step 0 before the loop, step
    // j >= 1 after the chain's j-th barrier) from set j % 2, which is then
    // reloaded with x_{j+2}
    Regs R0, R1;
    load(NT - 1, R0);
    load(NT - 2, R1);
    stage(NT - 1, R0);
    load(NT - 3, R0);
    // (no step's stage or load is conditional, which keeps the wait counts exact)
    auto step = [&](int j, Regs& R) {
      lds_barrier();
      stage(NT - 1 - j, R);
      load(NT - 3 - j, R);
    };
    int j = 1;
    for (; j + 1 <= NT - 1; j += 2) {
      step(j, R1);
      step(j + 1, R0);
    }
    if (j <= NT - 1) step(j, R1);
    lds_barrier();   // the chain's last chunk
  } else {
    // ========================= barrier-only waves =========================
    for (int c = NT - 1; c >= 0; --c) lds_barrier();
  }
}

// (2) both sequential walks of the backward in one launch (neither needs the
// other): workgroups [0, nwalk) run the reverse walk above (waves 2-5 stage,
// 6-7 only keep the barrier count), the rest the forward kernel's states-only
// body with 32 value rows (the chunk-start states, rounded to bf16).  One
// workgroup per CU either way (their LDS is one union).  When nwalk is a
// multiple of 8 both halves keep their XCD-aware numbering (id mod 8 is the
// XCD).
template <int KD>
__global__ void __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd16_walks_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                   const bf16* __restrict__ d_o, const float* __restrict__ alpha,
                   const float* __restrict__ beta, const float* __restrict__ s0,
                   const float* __restrict__ d_sfinal, float* __restrict__ d_s0,
                   const unsigned char* __restrict__ rec, bf16* __restrict__ ws_S,
                   bf16* __restrict__ ws_dS, int T, int H, int V, int nwalk) {
  __shared__ union {
    WalkSlot<KD> slot[2];
    Smem<KD, 32, 64> fwd;
  } u;
  const int bid = blockIdx.x;
  if (bid < nwalk)
    dstate_body<KD, 4>(u.slot, bid, nwalk, q, k, d_o, d_sfinal, d_s0, rec, ws_dS, T, H, V);
  else
    fwd_bf16_body<KD, 32, 64, false>(u.fwd, bid - nwalk, (int)gridDim.x - nwalk, q, k, v, alpha, beta,
                                     s0, nullptr, nullptr, nullptr, ws_S, nullptr, T, H, KD, V, kC,
                                     V / 32);
}

// ===========================================================================
// (3) token gradients: one workgroup (8 waves) per CU, each taking (chunk, head,
// batch) items in turn.  Per item the value axis is walked in slices of VSL
// columns; dP, dA and the S / dS' parts of dQ and dK accumulate in registers
// across slices.
template <int KD, int VD>
struct alignas(16) LocalSmem {
  static constexpr int VSL = 32;                    // value slice
  // rows of 32 bytes modulo 64 for the 16-byte fragment reads (lanes 0-7 and
  // 16-23 are served together): keys, queries, S, dS' and the slice tiles
  static constexpr int LDK = KD + 16, LDW = VSL + 16;
  bf16 k[kC * LDK], q[kC * LDK];       // [token][channel]
  bf16 tm[kC * kLDC], p[kC * kLDC];    // Tm, P [row][col]
  union {
    struct {
      bf16 s[VSL * LDK], ds[VSL * LDK];  // slice rows of S and dS' [value][channel]
      bf16 dob[kC * LDW];                // dO slice [token][value]
      bf16 rb[kC * LDW], ub[kC * LDW], dub[kC * LDW], drb[kC * LDW];  // R, U, dU, dR [token][value]
    } sl;
    struct {
      bf16 dpe[kC * kLDC], dae[kC * kLDC];  // (dP o E), (dA o beta E) [row][col]
      float xp[kC][kC + 4], xa[kC][kC + 4]; // dP o P and dA o M, [row][col]
    } fin;
  } u;
  alignas(16) float g[kC];
  float bt[kC];
  float red[4][16][16];                // per-token row sums of the slice tiles
  float dgs[kC], dbs[kC], dus[kC];     // per-token gate gradients, D_r U_r.W_r
  float dot[8];                        // <dS', S> partials per wave
};

template <int KD, int VD>
__global__ void __launch_bounds__(512)
bwd16_local_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                   const bf16* __restrict__ v, const bf16* __restrict__ d_o,
                   const float* __restrict__ alpha, const bf16* __restrict__ ws_S,
                   const bf16* __restrict__ ws_dS, const unsigned char* __restrict__ rec,
                   bf16* __restrict__ dq, bf16* __restrict__ dk, bf16* __restrict__ dv,
                   float* __restrict__ dalpha, float* __restrict__ dbeta, int B, int T, int H) {
  using SM = LocalSmem<KD, VD>;
  constexpr int LDK = SM::LDK, LDW = SM::LDW, VSL = SM::VSL;
  constexpr int KS = KD / 32, VKS = VSL / 32;
  constexpr int NVB = VSL / 16;            // value blocks per slice
  constexpr int NCB = KD / 16;             // channel blocks
  constexpr int NST = NVB * 4 / 8;         // slice tiles (value block, token block) per wave
  constexpr int NQT = NCB * 4 / 8;         // dQ / dK tiles per wave
  static_assert(NST >= 1 && NQT >= 1, "shape too small for 8 waves");
  __shared__ SM sm;
  // the lane indices are re-made opaque at every item (below), so that the
  // compiler keeps each item's per-lane addresses next to their use instead of
  // hoisting them all out of the item loop (which exceeds the register file)
  int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int ls = lane & 15, lg = lane >> 4;
  const int NT = (T + kC - 1) / kC;
  const size_t tokk = (size_t)H * KD, tokv = (size_t)H * VD;
  // Items are (chunk, head, batch), chunk fastest; the grid holds at most one
  // workgroup per CU and each workgroup takes items blockIdx.x, + gridDim.x, ...
  // so that the next item's operands are requested while this one is computed.
  const int items = NT * H * B;
  struct Item {
    int c, h, b, t0, n;
    size_t ck;                  // element offset of the item's [V, K] states
    const unsigned char* rc;    // the item's record
  };
  auto item_of = [&](int it) {
    Item I;
    I.c = it % NT;
    I.h = (it / NT) % H;
    I.b = it / NT / H;
    I.t0 = I.c * kC;
    I.n = min(kC, T - I.t0);
    I.ck = (((size_t)I.b * H + I.h) * NT + I.c) * (size_t)VD * KD;
    I.rc = rec + (((size_t)I.b * H + I.h) * NT + I.c) * kRecBytes;
    return I;
  };

  // ---- slice operands travel through registers, so the next slice is
  // requested while the current one is computed: S and dS' pieces (bf16), dO
  // pieces, and the V values of this wave's tiles
  constexpr int SP = VSL * KD / 8, SPL = (SP + 511) / 512;
  constexpr int OP = kC * VSL / 8, OPL = (OP + 511) / 512;
  struct SliceRegs {
    bf16x8 s[SPL], d[SPL];
    bf16x8 o[OPL];
    bf16x4 v[NST];
  };
  auto load_slice = [&](const Item& I, int vs0, SliceRegs& R) {
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const int p = tid + 512 * j, r = p / (KD / 8), c8 = (p % (KD / 8)) * 8;
      if (p < SP) {
        R.s[j] = *reinterpret_cast<const bf16x8*>(ws_S + I.ck + (size_t)(vs0 + r) * KD + c8);
        R.d[j] = *reinterpret_cast<const bf16x8*>(ws_dS + I.ck + (size_t)(vs0 + r) * KD + c8);
      }
    }
#pragma unroll
    for (int j = 0; j < OPL; ++j) {
      const int p = tid + 512 * j, r = p / (VSL / 8), c8 = (p % (VSL / 8)) * 8;
      R.o[j] = zero8();
      if (p < OP && r < I.n)
        R.o[j] = *reinterpret_cast<const bf16x8*>(d_o + ((size_t)I.b * T + I.t0 + r) * tokv + (size_t)I.h * VD + vs0 + c8);
    }
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int t = wave + 8 * u, vb = t % NVB, tk = 16 * (t / NVB) + ls;
      const bf16 z = (bf16)0.0f;
      R.v[u] = bf16x4{z, z, z, z};
      if (tk < I.n)
        R.v[u] = *reinterpret_cast<const bf16x4*>(v + ((size_t)I.b * T + I.t0 + tk) * tokv + (size_t)I.h * VD + vs0 + 16 * vb + 4 * lg);
    }
  };
  float dot = 0.0f;   // <dS', S> partial of the current item
  auto stage_slice = [&](const SliceRegs& R) {
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const int p = tid + 512 * j, r = p / (KD / 8), c8 = (p % (KD / 8)) * 8;
      if (p < SP) {
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf(bf2f(R.d[j][e]), bf2f(R.s[j][e]), dot);
        *reinterpret_cast<bf16x8*>(&sm.u.sl.s[r * LDK + c8]) = R.s[j];
        *reinterpret_cast<bf16x8*>(&sm.u.sl.ds[r * LDK + c8]) = R.d[j];
      }
    }
#pragma unroll
    for (int j = 0; j < OPL; ++j) {
      const int p = tid + 512 * j, r = p / (VSL / 8), c8 = (p % (VSL / 8)) * 8;
      if (p < OP) *reinterpret_cast<bf16x8*>(&sm.u.sl.dob[r * LDW + c8]) = R.o[j];
    }
  };
  // ---- chunk operands: keys, queries, Tm, P, gates, through registers so that
  // the next item's are requested while this one is computed
  constexpr int KP = kC * KD / 8, KPL = (KP + 511) / 512;
  static_assert(kC * kC / 8 == 512, "one C x C piece per thread");
  struct ChunkRegs {
    bf16x8 kv[KPL], qv[KPL], tv, pv;
    float gv, bv;
  };
  auto load_chunk = [&](const Item& I, ChunkRegs& C) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int p = tid + 512 * j, r = p / (KD / 8), c8 = (p % (KD / 8)) * 8;
      C.kv[j] = C.qv[j] = zero8();
      if (p < KP && r < I.n) {
        const size_t off = ((size_t)I.b * T + I.t0 + r) * tokk + (size_t)I.h * KD + c8;
        C.kv[j] = *reinterpret_cast<const bf16x8*>(k + off);
        C.qv[j] = *reinterpret_cast<const bf16x8*>(q + off);
      }
    }
    C.tv = *reinterpret_cast<const bf16x8*>(I.rc + kRecTm + 16 * tid);
    C.pv = *reinterpret_cast<const bf16x8*>(I.rc + kRecP + 16 * tid);
    // every thread reads a gate (threads past the chunk a valid duplicate), so
    // no load sits under a branch
    C.gv = reinterpret_cast<const float*>(I.rc + kRecG)[tid & (kC - 1)];
    C.bv = reinterpret_cast<const float*>(I.rc + kRecB)[tid & (kC - 1)];
  };
  auto stage_chunk = [&](const ChunkRegs& C) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int p = tid + 512 * j, r = p / (KD / 8), c8 = (p % (KD / 8)) * 8;
      if (p < KP) {
        *reinterpret_cast<bf16x8*>(&sm.k[r * LDK + c8]) = C.kv[j];
        *reinterpret_cast<bf16x8*>(&sm.q[r * LDK + c8]) = C.qv[j];
      }
    }
    const int r = tid / (kC / 8), c8 = (tid % (kC / 8)) * 8;
    *reinterpret_cast<bf16x8*>(&sm.tm[r * kLDC + c8]) = C.tv;
    *reinterpret_cast<bf16x8*>(&sm.p[r * kLDC + c8]) = C.pv;
    if (tid < kC) {
      sm.g[tid] = C.gv;
      sm.bt[tid] = C.bv;
    }
  };

  int it = blockIdx.x;
  Item I = item_of(it);
  ChunkRegs CR;
  SliceRegs R;
  load_chunk(I, CR);
  load_slice(I, 0, R);
  for (;;) {
    asm volatile("" : "+v"(tid), "+v"(lane), "+v"(ls), "+v"(lg));
    const int h = I.h, b = I.b, t0 = I.t0, n = I.n;
    // the next item (this one again after the last: its loads are then unused but
    // keep every load unconditional, so the wait counts stay exact)
    const int nx = it + (int)gridDim.x;
    const bool more = nx < items;
    const Item J = item_of(more ? nx : it);
    stage_chunk(CR);
    dot = 0.0f;

    // per-wave accumulators
    // slice tiles: t = wave + 8 u -> value block t % NVB, token block t / NVB
    float rs_oz[NST], rs_uw[NST], rs_db[NST], rs_ry[NST];   // per-lane row-sum partials
#pragma unroll
    for (int u = 0; u < NST; ++u) rs_oz[u] = rs_uw[u] = rs_db[u] = rs_ry[u] = 0.0f;
    // dP^T / dA^T tiles: job j = wave + 8 u < 20 (10 upper (i, r) block pairs each)
    f32x4 pa[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) pa[u] = zero4();
    // dQ^T / dK^T tiles: t = wave + 8 u -> channel block t % NCB, token block t / NCB
    f32x4 aq[NQT], ak1[NQT], ak2[NQT];
#pragma unroll
    for (int u = 0; u < NQT; ++u) aq[u] = ak1[u] = ak2[u] = zero4();

    for (int vs0 = 0; vs0 < VD; vs0 += VSL) {
      __syncthreads();
      stage_slice(R);
      bf16x4 vcur[NST];
#pragma unroll
      for (int u = 0; u < NST; ++u) vcur[u] = R.v[u];
      {
        const bool last = vs0 + VSL >= VD;
        load_slice(last ? J : I, last ? 0 : vs0 + VSL, R);
      }
      __syncthreads();

      // ---- (a) Y^T = S K^T, Z^T = S Q^T, W^T = dS' K^T; R^T = beta V^T - beta gam Y^T
      f32x4 YT[NST], WT[NST], VT[NST];
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const int t = wave + 8 * u, vb = t % NVB, tb = t / NVB;
        f32x4 y = zero4(), z = zero4(), w = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 sa = frag_rows(sm.u.sl.s, LDK, 16 * vb, 32 * ks, lane);
          const bf16x8 da = frag_rows(sm.u.sl.ds, LDK, 16 * vb, 32 * ks, lane);
          const bf16x8 kb = frag_rows(sm.k, LDK, 16 * tb, 32 * ks, lane);
          y = mma(sa, kb, y);
          z = mma(sa, frag_rows(sm.q, LDK, 16 * tb, 32 * ks, lane), z);
          w = mma(da, kb, w);
        }
        // lane: values vs0 + 16 vb + 4 lg + e, token tk = 16 tb + ls
        const int tk = 16 * tb + ls;
        const float gm = __builtin_amdgcn_exp2f(sm.g[tk]), bt = sm.bt[tk];
        const f32x4 vv = f32x4{bf2f(vcur[u][0]), bf2f(vcur[u][1]), bf2f(vcur[u][2]), bf2f(vcur[u][3])};
        const bf16x4 ov = *reinterpret_cast<const bf16x4*>(&sm.u.sl.dob[tk * LDW + 16 * vb + 4 * lg]);
        f32x4 r;
        float oz = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r[e] = bt * vv[e] - bt * gm * y[e];
          oz = fmaf(bf2f(ov[e]), z[e], oz);
        }
        rs_oz[u] += oz;
        store_tile_t(sm.u.sl.rb, LDW, 16 * tb, 16 * vb, r, lane);
        YT[u] = y;
        WT[u] = w;
        VT[u] = vv;
      }
      __syncthreads();
      // ---- (b) U^T = R^T Tm^T,  dU^T = diag(D) W^T + dO^T P
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const int t = wave + 8 * u, vb = t % NVB, tb = t / NVB;
        f32x4 uu = zero4(), du = zero4();
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
          if (32 * cs <= 16 * tb + 15)  // Tm lower
            uu = mma(frag_cols(sm.u.sl.rb, LDW, 16 * vb, 32 * cs, lane), frag_rows(sm.tm, kLDC, 16 * tb, 32 * cs, lane), uu);
          if (32 * cs + 31 >= 16 * tb)  // P lower: rows r >= i
            du = mma(frag_cols(sm.u.sl.dob, LDW, 16 * vb, 32 * cs, lane), frag_cols(sm.p, kLDC, 16 * tb, 32 * cs, lane), du);
        }
        const int tk = 16 * tb + ls;
        const float dd = __builtin_amdgcn_exp2f(sm.g[kC - 1] - sm.g[tk]);
        float uw = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          du[e] = fmaf(dd, WT[u][e], du[e]);
          uw = fmaf(uu[e], WT[u][e], uw);
        }
        rs_uw[u] += uw;
        store_tile_t(sm.u.sl.ub, LDW, 16 * tb, 16 * vb, uu, lane);
        store_tile_t(sm.u.sl.dub, LDW, 16 * tb, 16 * vb, du, lane);
      }
      __syncthreads();
      // ---- (c) dR^T = dU^T Tm;  dV = diag(beta) dR
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const int t = wave + 8 * u, vb = t % NVB, tb = t / NVB;
        f32x4 dr = zero4();
#pragma unroll
        for (int cs = 0; cs < 2; ++cs)
          if (32 * cs + 31 >= 16 * tb)  // Tm[i][r] with i >= r
            dr = mma(frag_cols(sm.u.sl.dub, LDW, 16 * vb, 32 * cs, lane), frag_cols(sm.tm, kLDC, 16 * tb, 32 * cs, lane), dr);
        const int tk = 16 * tb + ls;
        const float gm = __builtin_amdgcn_exp2f(sm.g[tk]), bt = sm.bt[tk];
        float db = 0.0f, ry = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          db = fmaf(dr[e], VT[u][e] - gm * YT[u][e], db);
          ry = fmaf(dr[e], YT[u][e], ry);
        }
        rs_db[u] += db;
        rs_ry[u] += ry;
        if (tk < n) store_bf4(dv + ((size_t)b * T + t0 + tk) * tokv + (size_t)h * VD + vs0 + 16 * vb + 4 * lg, dr * bt);
        store_tile_t(sm.u.sl.drb, LDW, 16 * tb, 16 * vb, dr, lane);
      }
      __syncthreads();
      // ---- (d) dP^T += U dO^T,  dA^T -= U dR^T   (upper (i, r) blocks, i <= r)
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int j = wave + 8 * u;
        if (j < 20) {
          const int jt = j % 10;
          const int rbk = jt < 1 ? 0 : (jt < 3 ? 1 : (jt < 6 ? 2 : 3));   // r block
          const int ibk = jt - rbk * (rbk + 1) / 2;                        // i block <= r block
          const bf16* bsrc = j < 10 ? sm.u.sl.dob : sm.u.sl.drb;
#pragma unroll
          for (int ks = 0; ks < VKS; ++ks)
            pa[u] = mma(frag_rows(sm.u.sl.ub, LDW, 16 * ibk, 32 * ks, lane), frag_rows(bsrc, LDW, 16 * rbk, 32 * ks, lane), pa[u]);
        }
      }
      // ---- (e) dQ^T += S^T dO^T,  dK^T += dS'^T U^T (part 1), S^T dR^T (part 2)
#pragma unroll
      for (int u = 0; u < NQT; ++u) {
        const int t = wave + 8 * u, cb = t % NCB, tb = t / NCB;
#pragma unroll
        for (int ks = 0; ks < VKS; ++ks) {
          const bf16x8 st = frag_cols(sm.u.sl.s, LDK, 16 * cb, 32 * ks, lane);
          aq[u] = mma(st, frag_rows(sm.u.sl.dob, LDW, 16 * tb, 32 * ks, lane), aq[u]);
          ak1[u] = mma(frag_cols(sm.u.sl.ds, LDK, 16 * cb, 32 * ks, lane), frag_rows(sm.u.sl.ub, LDW, 16 * tb, 32 * ks, lane), ak1[u]);
          ak2[u] = mma(st, frag_rows(sm.u.sl.drb, LDW, 16 * tb, 32 * ks, lane), ak2[u]);
        }
      }
    }
    // the next item's chunk operands, requested now so that they arrive during
    // this item's final products (requested at the item's start instead, they
    // hold 26 more registers through the slice loop and gained nothing)
    load_chunk(J, CR);
    // per-token row sums of the slice tiles: reduce over the four lane groups
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      float x[4] = {rs_oz[u], rs_uw[u], rs_db[u], rs_ry[u]};
#pragma unroll
      for (int qn = 0; qn < 4; ++qn) {
        x[qn] += __shfl_xor(x[qn], 16);
        x[qn] += __shfl_xor(x[qn], 32);
      }
      const int t = wave + 8 * u;
      if (lg == 0)
#pragma unroll
        for (int qn = 0; qn < 4; ++qn) sm.red[qn][t][ls] = x[qn];
    }
    // <dS', S>: wave partial
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);
    if (lane == 0) sm.dot[wave] = dot;
    __syncthreads();   // every slice array is dead from here

    // ---- (f) dP o E, dA o beta E to LDS (bf16, [r][i]); dP o P and dA o M (fp32,
    // with P and M recomputed in fp32 from the key and query tiles)
    for (int p = tid; p < kC * kC / 8; p += 512) {   // zero the tiles no job writes
      const int r = p / (kC / 8), c8 = (p % (kC / 8)) * 8;
      *reinterpret_cast<bf16x8*>(&sm.u.fin.dpe[r * kLDC + c8]) = zero8();
      *reinterpret_cast<bf16x8*>(&sm.u.fin.dae[r * kLDC + c8]) = zero8();
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int j = wave + 8 * u;
      if (j < 20) {
        const int jt = j % 10;
        const int rbk = jt < 1 ? 0 : (jt < 3 ? 1 : (jt < 6 ? 2 : 3));
        const int ibk = jt - rbk * (rbk + 1) / 2;
        // lane: i = 16 ibk + 4 lg + e, r = 16 rbk + ls
        const int r = 16 * rbk + ls;
        const float gr = sm.g[r], br = sm.bt[r];
        // gates of the lane's four i, read before the products (no LDS waits
        // inside the element loop)
        const f32x4 gi = *reinterpret_cast<const f32x4*>(&sm.g[16 * ibk + 4 * lg]);
        // Gram tile in the same layout: G[i][r] = k_i . q_r (dP jobs) or
        // k_i . k_r (dA jobs), exact bf16 products summed in fp32
        const bf16* gsrc = j < 10 ? sm.q : sm.k;
        f32x4 gram = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          gram = mma(frag_rows(sm.k, LDK, 16 * ibk, 32 * ks, lane), frag_rows(gsrc, LDK, 16 * rbk, 32 * ks, lane), gram);
        f32x4 val, prod;
        if (j < 10) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * ibk + 4 * lg + e;
            const float ee = __builtin_amdgcn_exp2f(i <= r ? gr - gi[e] : -INFINITY);
            const float dp = i <= r ? pa[u][e] : 0.0f;
            val[e] = dp * ee;
            prod[e] = dp * (ee * gram[e]);   // dP o P, P = E o (Q K^T)
          }
          store_tile_t(sm.u.fin.dpe, kLDC, 16 * rbk, 16 * ibk, val, lane);
          *reinterpret_cast<f32x4*>(&sm.u.fin.xp[r][16 * ibk + 4 * lg]) = prod;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * ibk + 4 * lg + e;
            const float ee = __builtin_amdgcn_exp2f(i < r ? gr - gi[e] : -INFINITY);
            const float da = i < r ? -pa[u][e] : 0.0f;
            val[e] = da * br * ee;
            prod[e] = da * (ee * gram[e]);   // dA o M, M = E o (K K^T), strictly lower
          }
          store_tile_t(sm.u.fin.dae, kLDC, 16 * rbk, 16 * ibk, val, lane);
          *reinterpret_cast<f32x4*>(&sm.u.fin.xa[r][16 * ibk + 4 * lg]) = prod;
        }
      }
    }
    __syncthreads();
    // ---- (g) dQ^T = diag(gam) S^T dO^T + K^T (dP o E)^T
    //          dK^T = D dS'^T U^T - beta gam S^T dR^T + Q^T (dP o E) + K^T (dA o bE)^T + K^T (dA o bE)
#pragma unroll
    for (int u = 0; u < NQT; ++u) {
      const int t = wave + 8 * u, cb = t % NCB, tb = t / NCB;
      const int tk = 16 * tb + ls;
      const float gm = __builtin_amdgcn_exp2f(sm.g[tk]);
      const float dd = __builtin_amdgcn_exp2f(sm.g[kC - 1] - sm.g[tk]);
      const float bg = sm.bt[tk] * gm;
      f32x4 xq = aq[u] * gm;
      f32x4 xk = ak1[u] * dd - ak2[u] * bg;
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) {
        const bf16x8 kt = frag_cols(sm.k, LDK, 16 * cb, 32 * cs, lane);
        if (32 * cs <= 16 * tb + 15) {   // (dP o E)[t][i], (dA o bE)[t][i]: i <= t
          xq = mma(kt, frag_rows(sm.u.fin.dpe, kLDC, 16 * tb, 32 * cs, lane), xq);
          xk = mma(kt, frag_rows(sm.u.fin.dae, kLDC, 16 * tb, 32 * cs, lane), xk);
        }
        if (32 * cs + 31 >= 16 * tb) {   // (dP o E)[r][t], (dA o bE)[r][t]: r >= t
          xk = mma(frag_cols(sm.q, LDK, 16 * cb, 32 * cs, lane), frag_cols(sm.u.fin.dpe, kLDC, 16 * tb, 32 * cs, lane), xk);
          xk = mma(kt, frag_cols(sm.u.fin.dae, kLDC, 16 * tb, 32 * cs, lane), xk);
        }
      }
      if (tk < n) {
        const size_t off = ((size_t)b * T + t0 + tk) * tokk + (size_t)h * KD + 16 * cb + 4 * lg;
        store_bf4(dq + off, xq);
        store_bf4(dk + off, xk);
      }
    }
    // ---- (h) per-token gate gradients: eight lanes per token split the row and
    // column sums of dP o P and dA o M by index mod 8 and combine them with three
    // shuffles (fixed order).  The sums skip the diagonal (dP o P's diagonal term
    // would enter both and cancel; dA o M's diagonal is zero).
    {
      const int r = tid >> 3, q8 = tid & 7;
      float sp = 0.0f, sa = 0.0f, cp = 0.0f, ca = 0.0f;
      // row sums over i = q8 + 8 m < r, column sums over rr = rr0 + 8 m < C: all
      // reads issued first (clamped indices), then added in order where valid
      const int rr0 = r + 1 + ((q8 - r - 1) & 7);
      float vxp[8], vxa[8], wxp[8], wxa[8], wbt[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int i = min(q8 + 8 * m, kC - 1), rr = min(rr0 + 8 * m, kC - 1);
        vxp[m] = sm.u.fin.xp[r][i];
        vxa[m] = sm.u.fin.xa[r][i];
        wxp[m] = sm.u.fin.xp[rr][r];
        wxa[m] = sm.u.fin.xa[rr][r];
        wbt[m] = sm.bt[rr];
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (q8 + 8 * m < r) {
          sp += vxp[m];
          sa += vxa[m];
        }
        if (rr0 + 8 * m < kC) {
          cp += wxp[m];
          ca += wbt[m] * wxa[m];
        }
      }
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) {
        sp += __shfl_xor(sp, m);
        sa += __shfl_xor(sa, m);
        cp += __shfl_xor(cp, m);
        ca += __shfl_xor(ca, m);
      }
      if (q8 == 0) {
        const int tb = r / 16, s = r % 16;
        float oz = 0.0f, uw = 0.0f, db = 0.0f, ry = 0.0f;
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
          oz += sm.red[0][tb * NVB + vb][s];
          uw += sm.red[1][tb * NVB + vb][s];
          db += sm.red[2][tb * NVB + vb][s];
          ry += sm.red[3][tb * NVB + vb][s];
        }
        const float gm = __builtin_amdgcn_exp2f(sm.g[r]), br = sm.bt[r];
        const float dd = __builtin_amdgcn_exp2f(sm.g[kC - 1] - sm.g[r]);
        sm.dgs[r] = gm * oz - br * gm * ry + (sp - cp) + (br * sa - ca);
        sm.dbs[r] = db + sa;
        sm.dus[r] = dd * uw;   // zero past the end (U rows are zero there)
      }
    }
    __syncthreads();
    if (wave == 0) {
      // d ln alpha_t = sum_{t <= r < n} dg_r (a scan over the reversed tokens, with
      // gam_last <dS', S> on the last real token) + sum_{r < t} D_r U_r.W_r (an
      // exclusive scan): the U.W terms reach token t only through the gates of
      // tokens before it, and summing them so, rather than as the chunk total minus
      // a suffix, keeps small gates free of cancellation
      float dsum = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) dsum += sm.dot[w];
      float dg = lane < n ? sm.dgs[lane] : 0.0f;
      if (lane == n - 1) dg += __builtin_amdgcn_exp2f(sm.g[kC - 1]) * dsum;
      const float suf = __shfl(wave_scan(__shfl(dg, 63 - lane), lane), 63 - lane);
      // exclusive scan: shift by one token first (inclusive minus own would cancel)
      const float pre = wave_scan(lane > 0 ? sm.dus[lane - 1] : 0.0f, lane);
      if (lane < n) {
        const size_t go = ((size_t)b * T + t0 + lane) * H + h;
        dalpha[go] = (suf + pre) / alpha[go];
        dbeta[go] = sm.dbs[lane];
      }
    }
    if (!more) break;
    it = nx;
    I = J;
    __syncthreads();   // this item's reads of the chunk operands and sums are done
  }
}

template <typename F>
hipError_t with_kd(int K, F&& f) {
  switch (K) {
    case 32: return f(std::integral_constant<int, 32>());
    case 64: return f(std::integral_constant<int, 64>());
    case 128: return f(std::integral_constant<int, 128>());
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool bwd_bf16_supported(int K, int V) {
  return (K == 32 || K == 64 || K == 128) && (V == 32 || V == 64 || V == 128);
}

size_t bwd_bf16_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V) {
  const int64_t NT = (T + kC - 1) / kC;
  return (size_t)(2 * B * H * NT * V * K * 2 + B * H * NT * (int64_t)kRecBytes);
}

namespace {

// Compute units of the device a stream belongs to (the persistent token-gradient
// grid is one workgroup per CU), queried once per device and cached; 256 (an
// MI355X) if the query fails.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus(hipStream_t stream) {
  int dev = -1;
  if (stream) {
    hipDevice_t d;
    if (hipStreamGetDevice(stream, &d) == hipSuccess) dev = static_cast<int>(d);
  } else if (hipGetDevice(&dev) != hipSuccess) {
    dev = -1;
  }
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int nc = 0;
  if (dev < 0 || hipDeviceGetAttribute(&nc, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      nc <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev < kMaxDevices) g_cus[dev].store(nc, std::memory_order_relaxed);
  return nc;
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (!bwd_bf16_supported(a.K, a.V)) return hipErrorInvalidValue;
  const int NT = (a.T + kC - 1) / kC;
  // workspace: chunk-start states and state gradients (bf16), then the records
  bf16* ws_S = reinterpret_cast<bf16*>(a.workspace);
  bf16* ws_dS = ws_S + (size_t)a.B * a.H * NT * a.V * a.K;
  unsigned char* rec = reinterpret_cast<unsigned char*>(ws_dS + (size_t)a.B * a.H * NT * a.V * a.K);
  const bf16* q = static_cast<const bf16*>(a.q);
  const bf16* k = static_cast<const bf16*>(a.k);
  const bf16* v = static_cast<const bf16*>(a.v);
  const bf16* d_o = static_cast<const bf16*>(a.d_o);
  const int cus = device_cus(stream);
  const long items_local = (long)NT * a.H * a.B;
  const int grid_local = (int)(items_local < cus ? items_local : cus);
  auto run = [&](auto kc) -> hipError_t {
    constexpr int KD = decltype(kc)::value;
    // the records first, with the whole GPU; then the two sequential walks in
    // one launch (one workgroup per CU each, side by side); then the token
    // gradients.  All three on the caller's stream.
    hipLaunchKernelGGL((bwd16_prep_kernel<KD>), dim3(NT * a.H * a.B), dim3(256), 0, stream, q, k, a.alpha,
                       a.beta, rec, a.T, a.H);
    hipError_t r;
    if ((r = hipGetLastError()) != hipSuccess) return r;
    const int nwalk = a.B * a.H * (a.V / 32);
    hipLaunchKernelGGL((bwd16_walks_kernel<KD>), dim3(2 * nwalk), dim3(512), 0, stream, q, k, v, d_o,
                       a.alpha, a.beta, a.s0, a.d_sfinal, a.d_s0, rec, ws_S, ws_dS, a.T, a.H, a.V, nwalk);
    if ((r = hipGetLastError()) != hipSuccess) return r;
    auto local = [&](auto vc) -> hipError_t {
      constexpr int VD = decltype(vc)::value;
      // one workgroup per CU (the kernel's LDS allows no more), each walking
      // items blockIdx.x, + gridDim.x, ...
      hipLaunchKernelGGL((bwd16_local_kernel<KD, VD>), dim3(grid_local), dim3(512), 0, stream, q, k, v,
                         d_o, a.alpha, ws_S, ws_dS, rec, static_cast<bf16*>(a.dq), static_cast<bf16*>(a.dk),
                         static_cast<bf16*>(a.dv), a.dalpha, a.dbeta, a.B, a.T, a.H);
      return hipGetLastError();
    };
    switch (a.V) {
      case 32: return local(std::integral_constant<int, 32>());
      case 64: return local(std::integral_constant<int, 64>());
      case 128: return local(std::integral_constant<int, 128>());
    }
    return hipErrorInvalidValue;
  };
  return with_kd(a.K, run);
}

}  // namespace gdn
