// The float32 walk over chunks of the forward (the state recurrence of the
// extended-WY / UT chunk form, "Sparse Delta Memory: layer and kernels", "What
// the layer computes"), on the fp32 matrix cores.  Shared by the forward launch
// (fwd_f32_mfma.hip) and the backward's walks launch (bwd_f32_mfma.hip), which
// runs it for the chunk-start states beside the reverse walk.
#pragma once

#include "f32_mfma.h"
#include "mfma_common.h"

namespace gdn {
namespace f32mfma {

// ---------------------------------------------------------------------------
// The walk over chunks.  One workgroup per (sequence, head, 16 NG
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
//
// The walk is a device function over a caller-declared LDS block (ChainLds) and
// a block index, so that one launch can run it beside the backward's reverse
// walk (bwd_f32_mfma.hip); f32_chain_kernel is the plain launch of it.
template <int KD, int C, int NG, bool WO>
struct ChainLds {
  static constexpr int LS = KD + 4;
  static constexpr int LC = C + 4;
  struct Grp {
    float sS[16 * LS];                    // S[v][k]
    float sR[16 * LC];                    // R'^T[v][t]
    float sU[16 * LC];                    // U^T[v][t]
    float sUd[16 * LC];                   // (diag(dn) U)^T[v][t]
  };
  alignas(16) float sK[2][C * LS];        // K [t][k]
  alignas(16) float sQ[WO ? C * LS : 4];
  alignas(16) Grp grp[NG];
};

template <int KD, int C, int NG, bool WO, bool HV, bool CK>
__device__ __forceinline__ void chain_walk(ChainLds<KD, C, NG, WO>& L, int bid,
                                           const float* __restrict__ q, const float* __restrict__ k,
                                           const float* __restrict__ v, const float* __restrict__ s0,
                                           float* __restrict__ o, float* __restrict__ s_final,
                                           float* __restrict__ s_ckpt, const float* __restrict__ rec,
                                           const int* __restrict__ cu, int B, int T, int H, int V,
                                           int NT) {
  constexpr int NB = C / 16;
  constexpr int NTH = 64 * NG * NB;
  constexpr int KQ = KD / 16;             // key-channel tiles
  constexpr int NKT = (KQ + NB - 1) / NB; // state tiles per wave (upper bound)
  constexpr int LS = KD + 4;
  constexpr int LC = C + 4;
  constexpr int TP = C * KD / 4;          // float4 pieces of a key (query) tile
  constexpr int PPT = (TP + NTH - 1) / NTH;
  using Grp = typename ChainLds<KD, C, NG, WO>::Grp;
  auto& sK = L.sK;
  auto& sQ = L.sQ;
  auto& grp = L.grp;

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
  const int xcd = bid & 7, jx = bid >> 3;
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

}  // namespace f32mfma
}  // namespace gdn
