// Chunkwise gated-delta-rule forward for float32 inputs on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulation).
//
// The chunk algebra is that of the extended-WY / UT decomposition ("Sparse Delta
// Memory: layer and kernels", "What the layer computes"; "OpenGDN 0.1.0", "Core
// operator reference").  Per chunk of n <= C tokens, with g the cumulative log2
// gate (g_r = sum_{i<=r} log2 alpha_i) and gam = 2^g:
//
//   A_ri = beta_r 2^(g_r - g_i) k_r.k_i   (i < r)      Tm = (I + A)^-1
//   P_ri = 2^(g_r - g_i) q_r.k_i          (i <= r)
//   X = K S^T,  Z = Q S^T,  R = diag(beta) (V - diag(gam) X),  U = Tm R
//   O = diag(gam) Z + P U
//   S^T <- 2^g_n S^T + (diag(dn) K)^T U,  dn_t = 2^(g_n - g_t)
//
// The pages split the work the same way: a phase that handles all chunks at once
// and never sees the state (here a launch over (chunk, head) that writes gates,
// Tm and P as a record), then the sequential walk over chunks (here a launch
// over (sequence, head, 16 value rows)).  With fp32 operands the matrix cores
// run at the vector rate, so arithmetic, not memory, bounds this path; doing
// the state-independent half once per chunk, rather than once per value slice
// inside the walk, is what keeps the arithmetic down.
//
// Operand layout of the 16x16x4 product: lane (g = lane / 16, s = lane % 16)
// supplies A[s][g] and B[g][s]; the accumulator gives lane (g, s) rows
// 4g .. 4g + 3 of column s.  mma16 runs four of them with lane (g, s) holding a
// float4 A[s][4g .. 4g + 3] and B[4g .. 4g + 3][s], product j taking element j of
// both, which contracts over 16 k in all.  An accumulator tile is then, as it
// stands, the right operand of a 16-deep product whose left operand rows are read
// as float4s: no data moves between lanes anywhere in this file.
//
// Every exponent is a difference g_r - g_i with r >= i (or g_n - g_t), so it is
// <= 0 and never overflows; masked entries are never exponentiated.  Sums run in
// a fixed order, so results are bitwise reproducible.
#include <mutex>
#include <type_traits>

#include "f32_mfma.h"
#include "launch.h"
#include "mfma_common.h"

namespace gdn {
namespace {

using namespace f32mfma;

// ---------------------------------------------------------------------------
// Launch 1: per (chunk, head) record.  256 threads.
template <int KD, int C>
__global__ void __launch_bounds__(256)
f32_record_kernel(const float* __restrict__ q, const float* __restrict__ k,
                  const float* __restrict__ alpha, const float* __restrict__ beta,
                  float* __restrict__ rec, float* __restrict__ fact, const int* __restrict__ cu, int B,
                  int T, int H, int NT) {
  constexpr int NB = C / 16;
  constexpr int LK = KD + 4;            // K rows in LDS: 16 lanes of a float4 read hit 16 bank quads
  constexpr int LC = C + 4;
  constexpr int KQ = KD / 16;
  constexpr int LKT = LK > LC ? LK : LC;
  __shared__ __attribute__((aligned(16))) float sKT[C * LKT];  // K tile, later Tm
  __shared__ __attribute__((aligned(16))) float sA[C * LC];
  __shared__ __attribute__((aligned(16))) float sg[C], sb[C];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s = lane & 15, g = lane >> 4;
  const int h = blockIdx.x % H, slot = blockIdx.x / H;
  int b, c;
  size_t seq0;
  int Tn;
  if (!cu) {
    b = slot / NT;
    c = slot - b * NT;
    seq0 = (size_t)b * T;
    Tn = T;
  } else {
    // the sequence whose slot range holds this slot: the last b with base(b) <= slot
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (clampi(cu[mid], 0, T) / C + mid <= slot) lo = mid; else hi = mid - 1;
    }
    b = lo;
    int s0, e0;
    packed_seq(cu, b, T, s0, e0);
    c = slot - (s0 / C + b);
    seq0 = s0;
    Tn = e0 - s0;
    if (c < 0) return;
  }
  const int t0 = c * C;
  if (t0 >= Tn) return;
  const int n = min(C, Tn - t0);
  float* R = rec + ((size_t)slot * H + h) * Rec<C>::kFloats;
  const size_t row0 = (seq0 + t0) * H + h;   // token row of the chunk's first token
  // the backward's factors of this chunk (dense batches only): M, P, Tm as C x C
  // row-major, then the cumulative natural-log gate, gam and beta
  float* Fc = fact ? fact + (((size_t)b * H + h) * NT + c) * (3 * C * C + 3 * C) : nullptr;

  // every global read of the chunk (K tile, gates, the P waves' query rows) is
  // requested before the first LDS write
  constexpr int NKP = C * (KD / 4), KP = (NKP + 255) / 256;
  f32x4 kx[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const int i = min(tid + 256 * j, NKP - 1), r = i / (KD / 4), c4 = i - r * (KD / 4);
    kx[j] = ld4(k + (row0 + (size_t)(r < n ? r : 0) * H) * KD + 4 * c4);
  }
  const bool live = lane < n;
  const float av = alpha[row0 + (size_t)(live ? lane : 0) * H];
  const float bv = beta[row0 + (size_t)(live ? lane : 0) * H];
  // Gram tasks: waves 0, 1 build A, waves 2, 3 P; each takes row blocks
  // {w % 2, NB - 1 - w % 2} (two for NB = 4) so that both do 5 of the 10 blocks.
  const bool pkind = w >= 2;
  const int I0 = w & 1;
  f32x4 qa[2][KQ];
  if (pkind) {
#pragma unroll
    for (int ri = 0; ri < 2; ++ri) {
      const int I = ri == 0 ? I0 : NB - 1 - I0;
      const int r = 16 * I + s;
      const bool ok = (ri == 0 ? I0 < NB : NB == 4) && r < n;
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq)
        qa[ri][kq] = ok ? ld4(q + (row0 + (size_t)r * H) * KD + 16 * kq + 4 * g) : zero4f();
    }
  }
  // K tile to LDS (rows past the chunk end are zero)
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const int i = tid + 256 * j, r = i / (KD / 4), c4 = i - r * (KD / 4);
    if (i < NKP) st4(sKT + r * LK + 4 * c4, r < n ? kx[j] : zero4f());
  }
  // cumulative log2 gates (padded tokens add log2 1 = 0) and beta
  if (w == 0) {
    const float gc = mfma::wave_scan(live ? log2f(av) : 0.0f, lane);
    if (lane < C) {
      sg[lane] = gc;
      sb[lane] = live ? bv : 0.0f;
    }
  }
  __syncthreads();

#pragma unroll
  for (int ri = 0; ri < 2; ++ri) {
    const int I = ri == 0 ? I0 : NB - 1 - I0;
    if (ri == 0 ? I0 >= NB : NB != 4) continue;
    f32x4 a[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
      a[kq] = pkind ? qa[ri][kq] : ld4(sKT + (16 * I + s) * LK + 16 * kq + 4 * g);
    for (int J = 0; J <= I; ++J) {
      f32x4 acc = zero4f();
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) acc = mma16(a[kq], ld4(sKT + (16 * J + s) * LK + 16 * kq + 4 * g), acc);
      const int j = 16 * J + s;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * I + 4 * g + e;
        if (pkind) {
          const float p = j <= i ? exp2f(sg[i] - sg[j]) * acc[e] : 0.0f;
          R[Rec<C>::kP + Rec<C>::at(I, J, 4 * g + e, s)] = p;
          if (Fc) Fc[C * C + i * C + j] = p;
        } else {
          const float m = j < i ? exp2f(sg[i] - sg[j]) * acc[e] : 0.0f;
          sA[i * LC + j] = sb[i] * m;
          if (Fc) Fc[i * C + j] = m;
        }
      }
    }
  }
  __syncthreads();   // A complete; the K tile is dead from here on

  float* sT = sKT;
  // diagonal blocks of Tm by forward substitution: wave w inverts block w, lane
  // s < 16 builds column s
  if (w < NB) {
    float t[16];
    const float* ab = sA + 16 * w * LC + 16 * w;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = s == r ? 1.0f : 0.0f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc = fmaf(-ab[r * LC + i], t[i], acc);
      t[r] = acc;
    }
    if (lane < 16) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[(16 * w + r) * LC + 16 * w + s] = t[r];
    }
  }
  __syncthreads();
  // off-diagonal blocks, one block diagonal at a time:
  // Tm_IJ = -Tm_II sum_{M=J}^{I-1} A_IM Tm_MJ
#pragma unroll
  for (int d = 1; d < NB; ++d) {
    const int J = w, I = w + d;
    if (I < NB) {
      f32x4 x = zero4f();
      for (int M = J; M < I; ++M) {
        const f32x4 am = ld4(sA + (16 * I + s) * LC + 16 * M + 4 * g);
        f32x4 tb;
#pragma unroll
        for (int j = 0; j < 4; ++j) tb[j] = sT[(16 * M + 4 * g + j) * LC + 16 * J + s];
        x = mma16(am, tb, x);
      }
      const f32x4 y = mma16(ld4(sT + (16 * I + s) * LC + 16 * I + 4 * g), x, zero4f());
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(16 * I + 4 * g + e) * LC + 16 * J + s] = -y[e];
    }
    __syncthreads();
  }
  // Tm diag(beta) (lower blocks) and the gate factors to the record.  Padded
  // tokens have log2 alpha = 0, so g_{C-1} = g_{n-1}.
  for (int i = tid; i < record_blocks(C) * 64; i += 256) {
    const int blk = i >> 6, r = (i >> 2) & 15, c4 = i & 3;
    const int I = blk >= 6 ? 3 : blk >= 3 ? 2 : blk >= 1 ? 1 : 0, J = blk - I * (I + 1) / 2;
    st4(R + Rec<C>::kTm + Rec<C>::at(I, J, r, 4 * c4),
        ld4(sT + (16 * I + r) * LC + 16 * J + 4 * c4) * ld4(sb + 16 * J + 4 * c4));
  }
  if (tid < C) {
    const float gl = sg[C - 1];
    R[Rec<C>::kGam + tid] = exp2f(sg[tid]);
    R[Rec<C>::kDn + tid] = exp2f(gl - sg[tid]);
    if (tid < 4) R[Rec<C>::kGn + tid] = tid == 0 ? exp2f(gl) : 0.0f;
  }
  if (Fc) {
    // the blocks above the diagonal of M and P are zero; Tm with the rows and
    // columns past the chunk end zero (the layout of the scalar prep's factors)
    for (int i = tid; i < C * C; i += 256) {
      const int r = i / C, j = i - r * C;
      if (j / 16 > r / 16) {
        Fc[i] = 0.0f;
        Fc[C * C + i] = 0.0f;
      }
      Fc[2 * C * C + i] = r < n && j < n && j / 16 <= r / 16 ? sT[r * LC + j] : 0.0f;
    }
    if (tid < C) {
      const bool live = tid < n;
      Fc[3 * C * C + tid] = live ? sg[tid] * 0.69314718055994531f : 0.0f;
      Fc[3 * C * C + C + tid] = live ? exp2f(sg[tid]) : 0.0f;
      Fc[3 * C * C + 2 * C + tid] = sb[tid];
    }
  }
}

// ---------------------------------------------------------------------------
// Launch 2: the walk over chunks.  One workgroup per (sequence, head, 16 NG
// value rows): NG groups of NB = C / 16 waves, group j owning value rows
// v0 + 16 j .. + 15.  Within a group, wave w owns token rows 16w .. 16w + 15 of
// every chunk for X, Z, R', U and O, and state tiles kappa = w, w + NB, ...
// (16 key channels each) for the update.  The state slice lives in the owners'
// accumulators and, for the X and Z products, in the group's LDS.  The chunk's
// key and query tiles are staged once per workgroup in LDS (keys double
// buffered), loaded with whole-row pieces two chunks ahead; the groups share
// them.
//
// WO: outputs wanted (q and o used); HV: values given (else V = 0); CK: chunk-start
// states to s_ckpt [B, H, NT, V, K].  No global load sits under a branch, so
// the compiler's wait counts stay exact across the loop, and loaded values are
// used as loaded (a select would make the load wait at once).  Rows past the
// chunk end read the chunk's first row instead: their X, Z and R' rows are finite
// junk that meets only zeros -- the record's Tm diag(beta) has zero columns there
// (beta = 0) and identity-times-beta rows, so those rows of U are exactly 0 and
// the state update adds 0 for them, and their O rows are not stored.  Blocks
// right of the diagonal block are loaded as the diagonal block and skipped by the
// products.
template <int KD, int C, int NG, bool WO, bool HV, bool CK>
__global__ void __launch_bounds__(64 * NG * (C / 16), 1)
f32_chain_kernel(const float* __restrict__ q, const float* __restrict__ k,
                 const float* __restrict__ v, const float* __restrict__ s0, float* __restrict__ o,
                 float* __restrict__ s_final, float* __restrict__ s_ckpt,
                 const float* __restrict__ rec, const int* __restrict__ cu, int B, int T, int H,
                 int V, int NT) {
  constexpr int NB = C / 16;
  constexpr int NTH = 64 * NG * NB;
  constexpr int KQ = KD / 16;             // key-channel tiles
  constexpr int NKT = (KQ + NB - 1) / NB; // state tiles per wave (upper bound)
  constexpr int LS = KD + 4;
  constexpr int LC = C + 4;
  constexpr int TP = C * KD / 4;          // float4 pieces of a key (query) tile
  constexpr int PPT = (TP + NTH - 1) / NTH;
  struct Grp {
    float sS[16 * LS];                    // S[v][k]
    float sR[16 * LC];                    // R'^T[v][t]
    float sU[16 * LC];                    // U^T[v][t]
    float sUd[16 * LC];                   // (diag(dn) U)^T[v][t]
  };
  __shared__ __attribute__((aligned(16))) float sK[2][C * LS];   // K [t][k]
  __shared__ __attribute__((aligned(16))) float sQ[WO ? C * LS : 4];
  __shared__ __attribute__((aligned(16))) Grp grp[NG];

  const int tid = threadIdx.x, lane = tid & 63, wg = tid >> 6;
  // group, token block.  The odd groups take their token blocks in reverse, so
  // that the two waves of a SIMD (wave i and i + NB share one) hold blocks w and
  // NB - 1 - w: the lower-triangular U and O products cost a block-row w wave
  // w + 1 steps, and each SIMD then carries NB + 1 of them.
  const int gi = wg / NB, w = (gi & 1) ? NB - 1 - (wg - gi * NB) : wg - gi * NB;
  const int s = lane & 15, g = lane >> 4;
  Grp& G = grp[gi];
  // workgroups of one (sequence, head) share an XCD (dispatch is round-robin
  // over the 8 XCDs), so its records and key rows are fetched into one L2
  const int nvs = V / (16 * NG), streams = B * H;
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int stream = xcd + 8 * (jx / nvs);
  if (stream >= streams) return;
  const int v0 = 16 * NG * (jx - (jx / nvs) * nvs) + 16 * gi;
  const int b = stream / H, h = stream - b * H;

  size_t seq0;
  int Tn, slot0;
  if (!cu) {
    seq0 = (size_t)b * T;
    Tn = T;
    slot0 = b * NT;
  } else {
    int s_, e_;
    packed_seq(cu, b, T, s_, e_);
    seq0 = s_;
    Tn = e_ - s_;
    slot0 = s_ / C + b;
  }
  const int nch = (Tn + C - 1) / C;
  const size_t sbase = ((size_t)b * H + h) * (size_t)V * KD + (size_t)(v0 + s) * KD;

  f32x4 S[NKT];
#pragma unroll
  for (int m = 0; m < NKT; ++m) {
    const int kap = w + NB * m;
    S[m] = (s0 && kap < KQ) ? ld4(s0 + sbase + 16 * kap + 4 * g) : zero4f();
    if (kap < KQ) st4(G.sS + s * LS + 16 * kap + 4 * g, S[m]);
  }

  auto rec_of = [&](int cc) { return rec + ((size_t)(slot0 + cc) * H + h) * Rec<C>::kFloats; };
  auto row_of = [&](int cc) { return (seq0 + (size_t)cc * C) * H + h; };
  auto n_of = [&](int cc) { return min(C, Tn - cc * C); };

  // key / query tiles: piece p = tid + NTH j is row p / (KD / 4), channels
  // 4 (p % (KD / 4)) .. + 3, so a wave reads whole 512-byte rows
  f32x4 kreg[PPT], qreg[PPT];
  auto tile_off = [&](int cc, int j) {
    const int n = n_of(cc);
    const int p = tid + NTH * j, r = p / (KD / 4), c4 = p - r * (KD / 4);
    const bool ok = p < TP && r < n;
    return (row_of(cc) + (size_t)(ok ? r : 0) * H) * KD + 4 * (ok ? c4 : 0);
  };
  auto load_k = [&](int cc) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) kreg[j] = ld4(k + tile_off(cc, j));
  };
  auto load_q = [&](int cc) {
    if (WO)
#pragma unroll
      for (int j = 0; j < PPT; ++j) qreg[j] = ld4(q + tile_off(cc, j));
  };
  auto stage_k = [&](int cc) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j, r = p / (KD / 4), c4 = p - r * (KD / 4);
      if (p < TP) st4(sK[cc & 1] + r * LS + 4 * c4, kreg[j]);
    }
  };
  auto stage_q = [&](int cc) {
    if (WO)
#pragma unroll
      for (int j = 0; j < PPT; ++j) {
        const int p = tid + NTH * j, r = p / (KD / 4), c4 = p - r * (KD / 4);
        if (p < TP) st4(sQ + r * LS + 4 * c4, qreg[j]);
      }
  };
  // per-wave operands of one chunk, in two alternating sets
  struct Ops {
    f32x4 vv, gw, dn;              // values, gam and dn of rows 16w + 4g + e
    f32x4 tmr[NB], pr[NB];         // Tm diag(beta) / P rows 16w + s (U, O)
    float gn;                      // 2^g_n
  };
  auto load_ops = [&](int cc, Ops& d) {
    const int n = n_of(cc);
    const size_t r0 = row_of(cc);
    if (HV) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * w + 4 * g + e;
        d.vv[e] = v[(r0 + (size_t)(t < n ? t : 0) * H) * V + v0 + s];
      }
    }
    const float* Rc = rec_of(cc);
    d.gw = ld4(Rc + Rec<C>::kGam + 16 * w + 4 * g);
    d.dn = ld4(Rc + Rec<C>::kDn + 16 * w + 4 * g);
    // 2^g_n is the same for every lane: through a vector register offset it stays
    // a vector load (a scalar load is waited for with the LDS counter, which the
    // next LDS barrier drains)
    int z = 0;
    asm volatile("" : "+v"(z));
    d.gn = Rc[Rec<C>::kGn + z];
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      const int o4 = Rec<C>::at(w, J <= w ? J : w, s, 4 * g);
      d.tmr[J] = ld4(Rc + Rec<C>::kTm + o4);
      if (WO) d.pr[J] = ld4(Rc + Rec<C>::kP + o4);
    }
  };
  Ops opa, opb;
  opa.vv = opb.vv = zero4f();
  // output rows of the previous chunk, stored one chunk late
  f32x4 Oprev = zero4f();
  size_t oprev = 0;
  auto store_o = [&](size_t r0, int n, bool check) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * w + 4 * g + e;
      if (!check || t < n) o[(r0 + (size_t)t * H) * V + v0 + s] = Oprev[e];
    }
  };
  if (nch > 0) {
    load_k(0);
    load_q(0);
    stage_k(0);
    stage_q(0);
    load_k(nch > 1 ? 1 : 0);
    load_q(nch > 1 ? 1 : 0);
    load_ops(0, opa);
  }
  __syncthreads();

  // One chunk with operands cur, loading chunk c + 1's into nxt and chunk c + 2's
  // key / query tiles (past the end the loads repeat the last chunk: no load is
  // conditional).  TAIL: the last, partial chunk.  gfx9 counts loads and stores
  // in one counter and a wait for a load while a store is pending waits for
  // everything, so the previous chunk's output rows are stored right after this
  // chunk's one real wait (for cur), and every wait finds its loads issued a
  // chunk earlier.  The empty asm statements take the consumer's results and
  // clobber memory, so that a consumer is done before the loads that reuse its
  // registers are issued.
  auto body = [&](int c, auto tail, Ops& cur, Ops& nxt) {
    constexpr bool TAIL = decltype(tail)::value;
    const int cn = c + 1 < nch ? c + 1 : c;
    const int cn2 = c + 2 < nch ? c + 2 : nch - 1;
    const float* kt = sK[c & 1];
    if (CK) {
#pragma unroll
      for (int m = 0; m < NKT; ++m) {
        const int kap = w + NB * m;
        if (kap < KQ)
          st4(s_ckpt + (((size_t)b * H + h) * nch + c) * (size_t)V * KD + (size_t)(v0 + s) * KD +
                  16 * kap + 4 * g, S[m]);
      }
    }

    // the next chunk's operands go to the other set, whose last reader was the
    // previous chunk: issued first, they overlap the products below
    load_ops(cn, nxt);

    // X = K S^T and Z = Q S^T for this wave's 16 token rows
    f32x4 X = zero4f(), Z = zero4f();
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
      const f32x4 bs = ld4(G.sS + s * LS + 16 * kq + 4 * g);
      X = mma16(ld4(kt + (16 * w + s) * LS + 16 * kq + 4 * g), bs, X);
      if (WO) Z = mma16(ld4(sQ + (16 * w + s) * LS + 16 * kq + 4 * g), bs, Z);
    }
    // R' = V - diag(gam) X (beta is in the record's Tm); Z <- diag(gam) Z
    f32x4 Rv = cur.vv - cur.gw * X;
    Z *= cur.gw;
    asm volatile("" : "+v"(Rv), "+v"(Z) : : "memory");
    if (WO && c > 0) store_o(oprev, C, false);
    st4(G.sR + s * LC + 16 * w + 4 * g, Rv);
    // chunk c + 1's keys to the other key buffer (its last reader, chunk c - 1's
    // state update, finished before the previous barrier) ahead of this barrier;
    // the registers are reloaded with chunk c + 2's
    stage_k(c + 1);
    load_k(cn2);
    mfma::lds_barrier();

    // chunk c + 1's queries to LDS (Q(c) is dead); the registers are reloaded
    // with chunk c + 2's
    stage_q(c + 1);
    load_q(cn2);

    // U = Tm diag(beta) R' (rows of this block; lower block-triangular)
    f32x4 U = zero4f();
#pragma unroll
    for (int J = 0; J < NB; ++J)
      if (J <= w) U = mma16(cur.tmr[J], ld4(G.sR + s * LC + 16 * J + 4 * g), U);
    st4(G.sU + s * LC + 16 * w + 4 * g, U);
    st4(G.sUd + s * LC + 16 * w + 4 * g, U * cur.dn);
    mfma::lds_barrier();

    // O = diag(gam) Z + P U
    if (WO) {
      f32x4 O = Z;
#pragma unroll
      for (int J = 0; J < NB; ++J)
        if (J <= w) O = mma16(cur.pr[J], ld4(G.sU + s * LC + 16 * J + 4 * g), O);
      Oprev = O;
      oprev = row_of(c);
      if (TAIL) store_o(oprev, n_of(c), true);
    }
    // S^T <- 2^g_n S^T + K^T (diag(dn) U) for the owned tiles
#pragma unroll
    for (int m = 0; m < NKT; ++m) {
      const int kap = w + NB * m;
      if (kap >= KQ) continue;
      f32x4 acc = S[m] * cur.gn;
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        f32x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = kt[(16 * J + 4 * g + e) * LS + 16 * kap + s];
        acc = mma16(a, ld4(G.sUd + s * LC + 16 * J + 4 * g), acc);
      }
      S[m] = acc;
      st4(G.sS + s * LS + 16 * kap + 4 * g, acc);
    }
    mfma::lds_barrier();
  };
  const int nfull = Tn / C;
  int c = 0;
  for (; c + 1 < nfull; c += 2) {
    body(c, std::false_type(), opa, opb);
    body(c + 1, std::false_type(), opb, opa);
  }
  const bool odd = c < nfull;       // one full chunk left, its operands in opa
  if (odd) body(c++, std::false_type(), opa, opb);
  if (c < nch) {
    if (odd) body(c, std::true_type(), opb, opa);
    else body(c, std::true_type(), opa, opb);
  } else if (WO && nch > 0) {
    store_o(oprev, C, false);       // the last chunk was full
  }

  if (s_final) {
#pragma unroll
    for (int m = 0; m < NKT; ++m) {
      const int kap = w + NB * m;
      if (kap < KQ) st4(s_final + sbase + 16 * kap + 4 * g, S[m]);
    }
  }
}

// Two value groups per workgroup (32 rows) while that still leaves at least
// 128 workgroups, else one (16 rows, twice the workgroups).
template <int KD, int C, bool WO, bool HV, bool CK>
hipError_t launch_chain(const FwdArgs& a, float* rec, int NT, hipStream_t stream) {
  const long groups = ((long)a.B * a.H + 7) / 8;
  if (a.V % 32 == 0 && (long)a.B * a.H * (a.V / 32) >= 128) {
    hipLaunchKernelGGL((f32_chain_kernel<KD, C, 2, WO, HV, CK>), dim3(8 * groups * (a.V / 32)),
                       dim3(128 * (C / 16)), 0, stream, static_cast<const float*>(a.q),
                       static_cast<const float*>(a.k), static_cast<const float*>(a.v), a.s0,
                       static_cast<float*>(a.o), a.s_final, a.s_ckpt, rec, a.cu_seqlens, a.B, a.T,
                       a.H, a.V, NT);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((f32_chain_kernel<KD, C, 1, WO, HV, CK>), dim3(8 * groups * (a.V / 16)),
                     dim3(64 * (C / 16)), 0, stream, static_cast<const float*>(a.q),
                     static_cast<const float*>(a.k), static_cast<const float*>(a.v), a.s0,
                     static_cast<float*>(a.o), a.s_final, a.s_ckpt, rec, a.cu_seqlens, a.B, a.T,
                     a.H, a.V, NT);
  return hipGetLastError();
}

template <int KD, int C>
hipError_t launch_kc(const FwdArgs& a, float* rec, hipStream_t stream) {
  const int NT = (a.T + C - 1) / C;
  const long slots = a.cu_seqlens ? (long)(a.T / C) + a.B + 1 : (long)a.B * NT;
  hipLaunchKernelGGL((f32_record_kernel<KD, C>), dim3(slots * a.H), dim3(256), 0, stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k), a.alpha,
                     a.beta, rec, a.cu_seqlens ? nullptr : a.factors, a.cu_seqlens, a.B, a.T, a.H, NT);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.o && a.v && !a.s_ckpt) return launch_chain<KD, C, true, true, false>(a, rec, NT, stream);
  if (a.o) return hipErrorInvalidValue;   // outputs are computed with values and no checkpoints
  if (a.v)
    return a.s_ckpt ? launch_chain<KD, C, false, true, true>(a, rec, NT, stream)
                    : launch_chain<KD, C, false, true, false>(a, rec, NT, stream);
  if (a.s_ckpt) return hipErrorInvalidValue;
  return launch_chain<KD, C, false, false, false>(a, rec, NT, stream);
}

template <int KD>
hipError_t launch_k(const FwdArgs& a, float* rec, hipStream_t stream) {
  if (a.chunk == 16) return launch_kc<KD, 16>(a, rec, stream);
  if (a.chunk == 32) return launch_kc<KD, 32>(a, rec, stream);
  return launch_kc<KD, 64>(a, rec, stream);
}

// Library-owned stream-ordered pool for the records, one per device.  Its
// release threshold is raised so that freed records stay reserved for the next
// call instead of going back to the driver at every synchronisation.
constexpr int kMaxPoolDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pool[kMaxPoolDevices];

hipError_t record_pool(hipStream_t stream, hipMemPool_t* out) {
  int dev = -1;
  hipError_t e;
  if (stream) {
    hipDevice_t d;
    if ((e = hipStreamGetDevice(stream, &d)) != hipSuccess) return e;
    dev = static_cast<int>(d);
  } else if ((e = hipGetDevice(&dev)) != hipSuccess) {
    return e;
  }
  if (dev < 0 || dev >= kMaxPoolDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (!g_pool[dev]) {
    hipMemPoolProps p = {};
    p.allocType = hipMemAllocationTypePinned;
    p.handleTypes = hipMemHandleTypeNone;
    p.location.type = hipMemLocationTypeDevice;
    p.location.id = dev;
    hipMemPool_t pool = nullptr;
    if ((e = hipMemPoolCreate(&pool, &p)) != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;
    if ((e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep)) != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return e;
    }
    g_pool[dev] = pool;
  }
  *out = g_pool[dev];
  return hipSuccess;
}

}  // namespace

size_t fwd_f32_record_bytes(const FwdArgs& a) {
  const int C = a.chunk;
  const long NT = (a.T + C - 1) / C;
  const long slots = a.cu_seqlens ? (long)(a.T / C) + a.B + 1 : (long)a.B * NT;
  return (size_t)slots * a.H * (size_t)record_floats(C) * sizeof(float);
}

bool fwd_f32_mfma_supported(int K, int V, int chunk) {
  return (K == 16 || K == 32 || K == 64 || K == 128) && V > 0 && V % 16 == 0 && V <= 128 &&
         (chunk == 16 || chunk == 32 || chunk == 64);
}

hipError_t launch_fwd_f32_records(const FwdArgs& a, float* rec, hipStream_t stream) {
  if (!fwd_f32_mfma_supported(a.K, a.V, a.chunk) || !rec) return hipErrorInvalidValue;
  if (a.K == 16) return launch_k<16>(a, rec, stream);
  if (a.K == 32) return launch_k<32>(a, rec, stream);
  if (a.K == 64) return launch_k<64>(a, rec, stream);
  return launch_k<128>(a, rec, stream);
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (!fwd_f32_mfma_supported(a.K, a.V, a.chunk)) return launch_fwd_f32_scalar(a, stream);
  hipMemPool_t pool;
  hipError_t e = record_pool(stream, &pool);
  if (e != hipSuccess) return e;
  void* rec = nullptr;
  if ((e = hipMallocFromPoolAsync(&rec, fwd_f32_record_bytes(a), pool, stream)) != hipSuccess) return e;
  e = launch_fwd_f32_records(a, static_cast<float*>(rec), stream);
  const hipError_t f = hipFreeAsync(rec, stream);
  return e != hipSuccess ? e : f;
}

}  // namespace gdn
