// Float32 backward, the reverse walk over chunks on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32).  With dS' the gradient of a chunk's end state
// (the derivation is in the header of bwd.hip), per chunk, chunks in reverse:
//
//   W = K dS'^T,  dU = diag(D) W + P^T dO,  dR = Tm^T dU
//   dS (chunk start) = gam_n dS' + dO^T diag(gam) Q - dR^T diag(beta gam) K
//
// storing every chunk's dS' for the token-gradient launch.  It reads the records
// the matrix-core forward's chunk-parallel launch wrote for the state recompute
// (fwd_f32_mfma.hip): with Tm diag(beta) in the record, Tm_b^T dU = diag(beta) dR
// is what the update needs.  Layouts and lane conventions are those of the
// forward's walk (f32_mfma.h): the state gradient lives as dS'^T tiles in the
// owners' accumulators; P^T and Tm_b^T operands are column reads of the record's
// blocks in LDS, the Q and K operands of the update column reads of the chunk's
// tiles.
#include <type_traits>

#include "f32_chain.h"
#include "f32_mfma.h"
#include "launch.h"
#include "mfma_common.h"

namespace gdn {
namespace {

using namespace f32mfma;

// One workgroup per (batch, head, 16 NG value rows), NG groups of NB = C / 16
// waves; wave w of a group owns token rows 16w .. 16w + 15 (W, dU, dR) and
// state-gradient tiles w, w + NB, ... (16 key channels each).  Chunk c - 1's
// key and query tiles, record and dO rows are staged in LDS (double buffers)
// while chunk c is walked, from registers loaded one chunk earlier; no load sits
// under a branch (rows past the end read the chunk's first row; their dO rows
// are staged as zeros, and the record's zero P columns and beta = 0 keep the
// other junk rows out of dR and the update).
//
// The walk is a device function over a caller-declared LDS block (DstateLds) and
// a block index; f32_dstate_kernel launches it alone, f32_walks_kernel beside the
// forward walk that recomputes the chunk-start states.
template <int KD, int C, int NG>
struct DstateLds {
  static constexpr int LS = KD + 4;
  static constexpr int LC = C + 4;
  struct Grp {
    float sS[16 * LS];                       // dS' [v][k]
    float sdO[2][16 * LC];                   // dO^T [v][t]
    float sdU[16 * LC];                      // dU^T [v][t]
    float sdR[16 * LC];                      // (-beta gam dR)^T [v][t]
  };
  alignas(16) float sK[2][C * LS];
  alignas(16) float sQ[2][C * LS];
  alignas(16) float sRec[2][Rec<C>::kFloats];
  alignas(16) Grp grp[NG];
};

template <int KD, int C, int NG>
__device__ __forceinline__ void dstate_walk(DstateLds<KD, C, NG>& L, int bid,
                                            const float* __restrict__ q,
                                            const float* __restrict__ k,
                                            const float* __restrict__ d_o,
                                            const float* __restrict__ d_sfinal,
                                            float* __restrict__ d_s0, const float* __restrict__ rec,
                                            float* __restrict__ ws_dS, int B, int T, int H, int V) {
  constexpr int NB = C / 16;
  constexpr int NTH = 64 * NG * NB;
  constexpr int KQ = KD / 16;
  constexpr int NKT = (KQ + NB - 1) / NB;
  constexpr int LS = KD + 4;
  constexpr int LC = C + 4;
  constexpr int TP = C * KD / 4;             // float4 pieces of a key (query) tile
  constexpr int PPT = (TP + NTH - 1) / NTH;
  constexpr int RF = Rec<C>::kFloats;
  static_assert(RF % 4 == 0, "record pieces");
  constexpr int RP = RF / 4;                 // float4 pieces of a record
  constexpr int RPT = (RP + NTH - 1) / NTH;
  using Grp = typename DstateLds<KD, C, NG>::Grp;
  auto& sK = L.sK;
  auto& sQ = L.sQ;
  auto& sRec = L.sRec;
  auto& grp = L.grp;

  const int tid = threadIdx.x, lane = tid & 63, wg = tid >> 6;
  const int gi = wg / NB, w = wg - gi * NB;
  const int s = lane & 15, g = lane >> 4;
  Grp& G = grp[gi];
  // the workgroups of one (batch, head) share an XCD, so its records and tiles
  // are fetched into one L2
  const int nvs = V / (16 * NG), streams = B * H;
  const int xcd = bid & 7, jx = bid >> 3;
  const int stream = xcd + 8 * (jx / nvs);
  if (stream >= streams) return;
  const int v0 = 16 * NG * (jx - (jx / nvs) * nvs) + 16 * gi;
  const int b = stream / H, h = stream - b * H;
  const int NT = (T + C - 1) / C;
  const size_t sbase = ((size_t)b * H + h) * (size_t)V * KD + (size_t)(v0 + s) * KD;

  auto rec_of = [&](int cc) { return rec + ((size_t)(b * NT + cc) * H + h) * RF; };
  auto row_of = [&](int cc) { return ((size_t)b * T + (size_t)cc * C) * H + h; };
  auto n_of = [&](int cc) { return min(C, T - cc * C); };

  f32x4 S[NKT];                              // dS'^T tiles
#pragma unroll
  for (int m = 0; m < NKT; ++m) {
    const int kap = w + NB * m;
    S[m] = (d_sfinal && kap < KQ) ? ld4(d_sfinal + sbase + 16 * kap + 4 * g) : zero4f();
    if (kap < KQ) st4(G.sS + s * LS + 16 * kap + 4 * g, S[m]);
  }

  f32x4 kreg[PPT], qreg[PPT], rreg[RPT];
  float dor[4];
  auto load_next = [&](int cc) {
    const int n = n_of(cc);
    const size_t r0 = row_of(cc);
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j, r = p / (KD / 4), c4 = p - r * (KD / 4);
      const bool ok = p < TP && r < n;
      const size_t off = (r0 + (size_t)(ok ? r : 0) * H) * KD + 4 * (ok ? c4 : 0);
      kreg[j] = ld4(k + off);
      qreg[j] = ld4(q + off);
    }
    const float* R = rec_of(cc);
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int p = tid + NTH * j;
      rreg[j] = ld4(R + 4 * (p < RP ? p : 0));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * w + 4 * g + e;
      dor[e] = d_o[(r0 + (size_t)(t < n ? t : 0) * H) * V + v0 + s];
    }
  };
  // into buffer `buf` the chunk whose row count is n
  auto stage = [&](int buf, int n) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j, r = p / (KD / 4), c4 = p - r * (KD / 4);
      if (p < TP) {
        st4(sK[buf] + r * LS + 4 * c4, kreg[j]);
        st4(sQ[buf] + r * LS + 4 * c4, qreg[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int p = tid + NTH * j;
      if (p < RP) st4(sRec[buf] + 4 * p, rreg[j]);
    }
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = 16 * w + 4 * g + e < n ? dor[e] : 0.0f;
    st4(G.sdO[buf] + s * LC + 16 * w + 4 * g, x);
  };

  if (NT > 0) {
    load_next(NT - 1);
    stage((NT - 1) & 1, n_of(NT - 1));
    load_next(NT > 1 ? NT - 2 : 0);
  }
  __syncthreads();

  for (int c = NT - 1; c >= 0; --c) {
    const float* kt = sK[c & 1];
    const float* qt = sQ[c & 1];
    const float* rc = sRec[c & 1];
    const float* dot = G.sdO[c & 1];
    // dS' of this chunk for the token gradients
#pragma unroll
    for (int m = 0; m < NKT; ++m) {
      const int kap = w + NB * m;
      if (kap < KQ)
        st4(ws_dS + (((size_t)b * H + h) * NT + c) * (size_t)V * KD + (size_t)(v0 + s) * KD +
                16 * kap + 4 * g, S[m]);
    }
    // W = K dS'^T (rows 16w + s of the chunk)
    f32x4 W = zero4f();
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
      W = mma16(ld4(kt + (16 * w + s) * LS + 16 * kq + 4 * g), ld4(G.sS + s * LS + 16 * kq + 4 * g), W);
    // dU = diag(D) W + P^T dO: P^T[16w + s][16J + k] = P block (J, w) [k][s]
    f32x4 dU = ld4(rc + Rec<C>::kDn + 16 * w + 4 * g) * W;
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      if (J < w) continue;
      f32x4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = rc[Rec<C>::kP + Rec<C>::at(J, w, 4 * g + e, s)];
      dU = mma16(a, ld4(dot + s * LC + 16 * J + 4 * g), dU);
    }
    st4(G.sdU + s * LC + 16 * w + 4 * g, dU);
    mfma::lds_barrier();

    // chunk c - 1 into the other buffers (whose last reader was chunk c + 1;
    // after the last chunk the staging lands in the unused buffer), then the
    // registers take chunk c - 2
    stage((c + 1) & 1, n_of(c > 0 ? c - 1 : 0));
    load_next(c > 1 ? c - 2 : 0);

    // diag(beta) dR = (Tm diag(beta))^T dU, scaled to -beta gam dR for the update
    f32x4 dR = zero4f();
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      if (J < w) continue;
      f32x4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = rc[Rec<C>::kTm + Rec<C>::at(J, w, 4 * g + e, s)];
      dR = mma16(a, ld4(G.sdU + s * LC + 16 * J + 4 * g), dR);
    }
    st4(G.sdR + s * LC + 16 * w + 4 * g, -(ld4(rc + Rec<C>::kGam + 16 * w + 4 * g) * dR));
    mfma::lds_barrier();

    // dS'^T <- gam_n dS'^T + Q^T diag(gam) dO + K^T (-beta gam dR), owned tiles;
    // the right operands are the same for every tile, so they are read once, and
    // the new tiles go to LDS after all of the products
    const float gn = rc[Rec<C>::kGn];
    f32x4 gdv[NB], drv[NB];
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      gdv[J] = ld4(dot + s * LC + 16 * J + 4 * g) * ld4(rc + Rec<C>::kGam + 16 * J + 4 * g);
      drv[J] = ld4(G.sdR + s * LC + 16 * J + 4 * g);
    }
#pragma unroll
    for (int m = 0; m < NKT; ++m) {
      const int kap = w + NB * m;
      if (kap >= KQ) continue;
      f32x4 acc = S[m] * gn;
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        f32x4 aq, ak;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          aq[e] = qt[(16 * J + 4 * g + e) * LS + 16 * kap + s];
          ak[e] = kt[(16 * J + 4 * g + e) * LS + 16 * kap + s];
        }
        acc = mma16(aq, gdv[J], acc);
        acc = mma16(ak, drv[J], acc);
      }
      S[m] = acc;
    }
#pragma unroll
    for (int m = 0; m < NKT; ++m) {
      const int kap = w + NB * m;
      if (kap < KQ) st4(G.sS + s * LS + 16 * kap + 4 * g, S[m]);
    }
    mfma::lds_barrier();
  }

  if (d_s0) {
#pragma unroll
    for (int m = 0; m < NKT; ++m) {
      const int kap = w + NB * m;
      if (kap < KQ) st4(d_s0 + sbase + 16 * kap + 4 * g, S[m]);
    }
  }
}

template <int KD, int C, int NG>
__global__ void __launch_bounds__(64 * NG * (C / 16), 1)
f32_dstate_kernel(const float* __restrict__ q, const float* __restrict__ k,
                  const float* __restrict__ d_o, const float* __restrict__ d_sfinal,
                  float* __restrict__ d_s0, const float* __restrict__ rec,
                  float* __restrict__ ws_dS, int B, int T, int H, int V) {
  __shared__ DstateLds<KD, C, NG> lds;
  dstate_walk<KD, C, NG>(lds, blockIdx.x, q, k, d_o, d_sfinal, d_s0, rec, ws_dS, B, T, H, V);
}

// Both sequential walks of the backward in one launch, each at two value groups
// (32 value rows) per workgroup: blocks [0, nd) walk the chunks in reverse for
// the state gradients, blocks [nd, nd + nf) walk them forward for the chunk-start
// states (checkpoints, no outputs).  The two are independent given the records,
// and neither fills the chip at the shapes the backward is used on, so running
// them side by side takes about the longer of the two instead of their sum.  nd
// is a multiple of 8, so both keep their XCD-aware block mapping.  The LDS is
// the union of the two walks' blocks.
template <int KD, int C>
__global__ void __launch_bounds__(128 * (C / 16), 1)
f32_walks_kernel(const float* __restrict__ q, const float* __restrict__ k,
                 const float* __restrict__ v, const float* __restrict__ s0,
                 float* __restrict__ s_ckpt, const float* __restrict__ d_o,
                 const float* __restrict__ d_sfinal, float* __restrict__ d_s0,
                 const float* __restrict__ rec, float* __restrict__ ws_dS, int B, int T, int H,
                 int V, int NT, int nd) {
  __shared__ union Lds {
    ChainLds<KD, C, 2, false> fwd;
    DstateLds<KD, C, 2> rev;
  } lds;
  const int bid = blockIdx.x;
  if (bid < nd)
    dstate_walk<KD, C, 2>(lds.rev, bid, q, k, d_o, d_sfinal, d_s0, rec, ws_dS, B, T, H, V);
  else
    chain_walk<KD, C, 2, false, true, true>(lds.fwd, bid - nd, q, k, v, s0, nullptr, nullptr,
                                            s_ckpt, rec, nullptr, B, T, H, V, NT);
}

// ---------------------------------------------------------------------------
// Token gradients of one chunk on the fp32 matrix cores: one workgroup (four
// waves) per (chunk, head, batch).  The value axis is walked in rounds of four
// 16-wide slices, wave w taking slice 4 rho + w of round rho; per slice (with S
// and dS' the chunk's start state and end-state gradient, the slice's rows):
//
//   Y = K S^T, Z = Q S^T, W = K dS'^T, R = diag(beta) V - diag(beta gam) Y
//   U = Tm R, dU = diag(D) W + P^T dO, dR = Tm^T dU, dV = diag(beta) dR
//   dP += dO U^T, dA -= dR U^T
//
// and the per-token sums of the gate gradients.  The round's slice tiles (S,
// dS', dO, U, dR) then stay in LDS for all four waves, and wave w adds every
// slice's share of
//
//   dQ += diag(gam) dO S,  dK += diag(D) U dS' - diag(beta gam) dR S
//
// to the key-channel tiles it owns (w, w + 4, ...), so dQ and dK need no
// reduction across waves; the waves' partial dP, dA and sums are added in wave
// order through LDS, and the owners finish dQ and dK with the chunk's
// token-axis products:
//
//   dQ += (dP o E) K,  dK += (dP o E)^T Q + (dA o bE) K + (dA o bE)^T K.
//
// The factors (M, P, Tm, gates) are the float32 prep's; the gate gradients use
// its cancellation-free sums (bwd.hip): the pair terms of token t run over
// i < t <= r only.  Rows past the chunk end are staged as zeros, with zero
// gates and factors, so they add nothing anywhere.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// sum over the 16 lanes of a lane group, in a fixed order; every lane ends with it
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m, 16);
  return x;
}

template <int KD, int C>
__global__ void __launch_bounds__(256, 1)
f32_local_kernel(const float* __restrict__ q, const float* __restrict__ k,
                 const float* __restrict__ v, const float* __restrict__ d_o,
                 const float* __restrict__ alpha, const float* __restrict__ ws_S,
                 const float* __restrict__ ws_dS, const float* __restrict__ ws_F,
                 float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
                 float* __restrict__ dalpha, float* __restrict__ dbeta, int T, int H, int V) {
  constexpr int NB = C / 16;
  constexpr int KQ = KD / 16;
  constexpr int LK = KD + 4, LCC = C + 4, LV = 16 + 4;
  constexpr int NW = 4;
  constexpr int NBL = NB * (NB + 1) / 2;       // lower token blocks
  constexpr int NKO = (KQ + NW - 1) / NW;      // key-channel tiles a wave owns
  static_assert(C <= 64, "one lane per token in the gate scans");
  struct WaveArea {                             // one slice's tiles
    float S[16 * LK], dS[16 * LK];              // [v][k]
    float dO[C * LV], U[C * LV], dR[C * LV];    // [t][v]
  };
  struct Red {                                  // after the value walk
    float dP[C * LCC], dA[C * LCC];             // [r][i]
    float X[C * LCC];                           // pair terms of the gate sums
    float pP[NW][C * LCC], pA[NW][C * LCC];     // the waves' partial dP, dA
    float pdb[NW][C], pdg[NW][C], puw[NW][C];   // the waves' per-token sums
  };
  union Area {
    WaveArea wave[NW];
    Red red;
  };
  __shared__ __attribute__((aligned(16))) float sK[C * LK], sQ[C * LK];
  __shared__ __attribute__((aligned(16))) float sM[C * LCC], sP[C * LCC], sT[C * LCC];
  __shared__ __attribute__((aligned(16))) Area area;
  __shared__ float sg[C], sgam[C], sb[C], sD[C];
  __shared__ float sdb[C], sdg[C], sdu[C], sxr[C], sdot[NW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s = lane & 15, g = lane >> 4;
  const int NT = (T + C - 1) / C;
  const int c = blockIdx.x % NT, h = (blockIdx.x / NT) % H, b = blockIdx.x / NT / H;
  const int t0 = c * C, n = min(C, T - t0);
  const size_t ck = (((size_t)b * H + h) * NT + c) * (size_t)V * KD;
  const size_t row0 = ((size_t)b * T + t0) * H + h;   // token row of the chunk's first token

  // key / query tiles (rows past the end zero), the prep's factors and gates:
  // every load is issued before the first LDS write
  {
    constexpr int NKP = C * (KD / 4), KP = (NKP + 255) / 256;
    static_assert(C * C % 256 == 0, "whole factor pieces per thread");
    f32x4 kx[KP], qx[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      const int i = min(tid + 256 * j, NKP - 1), r = i / (KD / 4), c4 = i - r * (KD / 4);
      const size_t off = (row0 + (size_t)(r < n ? r : 0) * H) * KD + 4 * c4;
      kx[j] = ld4(k + off);
      qx[j] = ld4(q + off);
    }
    const float* F = ws_F + (((size_t)b * H + h) * NT + c) * (3 * C * C + 3 * C);
    constexpr int FP = C * C / 256;
    float fm[FP], fp[FP], ft[FP];
#pragma unroll
    for (int j = 0; j < FP; ++j) {
      fm[j] = F[tid + 256 * j];
      fp[j] = F[C * C + tid + 256 * j];
      ft[j] = F[2 * C * C + tid + 256 * j];
    }
    const int tg = tid & (C - 1);
    const float gl = F[3 * C * C + n - 1], gt = F[3 * C * C + tg];
    const float gam = F[3 * C * C + C + tg], bet = F[3 * C * C + 2 * C + tg];
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      const int i = tid + 256 * j, r = i / (KD / 4), c4 = i - r * (KD / 4);
      if (i < NKP) {
        st4(sK + r * LK + 4 * c4, r < n ? kx[j] : zero4f());
        st4(sQ + r * LK + 4 * c4, r < n ? qx[j] : zero4f());
      }
    }
#pragma unroll
    for (int j = 0; j < FP; ++j) {
      const int i = tid + 256 * j, r = i / C, jj = i - r * C;
      sM[r * LCC + jj] = fm[j];
      sP[r * LCC + jj] = fp[j];
      sT[r * LCC + jj] = ft[j];
    }
    if (tid < C) {
      const bool ok = tid < n;
      sg[tid] = gt;
      sgam[tid] = ok ? gam : 0.0f;
      sb[tid] = ok ? bet : 0.0f;
      sD[tid] = ok ? expf(gl - gt) : 0.0f;
    }
  }
  __syncthreads();

  f32x4 aQ[NB][NKO], aK[NB][NKO], aP[NBL], aA[NBL];
#pragma unroll
  for (int I = 0; I < NB; ++I)
#pragma unroll
    for (int m = 0; m < NKO; ++m) aQ[I][m] = aK[I][m] = zero4f();
#pragma unroll
  for (int i = 0; i < NBL; ++i) aP[i] = aA[i] = zero4f();
  float pdb[NB][4], poz[NB][4], pry[NB][4], puw[NB][4];
#pragma unroll
  for (int I = 0; I < NB; ++I)
#pragma unroll
    for (int e = 0; e < 4; ++e) pdb[I][e] = poz[I][e] = pry[I][e] = puw[I][e] = 0.0f;
  float pdot = 0.0f;

  WaveArea& A = area.wave[w];
  const int nsl = V / 16;
  for (int sl0 = 0; sl0 < nsl; sl0 += NW) {
    // ---- this wave's slice (a wave past the last slice loads the last one
    // again, so that no load sits under a branch, and adds nothing)
    const bool act = sl0 + w < nsl;
    const int v0 = 16 * min(sl0 + w, nsl - 1);
    {
      constexpr int SPL = 16 * KD / 4 / 64;     // float4 pieces per lane of 16 state rows
      constexpr int OPL = (C * 4 + 63) / 64;    // float4 pieces per lane of the dO columns
      f32x4 sx[SPL], dx[SPL], ox[OPL];
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const int p = lane + 64 * j, r = p / (KD / 4), c4 = p - r * (KD / 4);
        sx[j] = ld4(ws_S + ck + (size_t)(v0 + r) * KD + 4 * c4);
        dx[j] = ld4(ws_dS + ck + (size_t)(v0 + r) * KD + 4 * c4);
      }
#pragma unroll
      for (int j = 0; j < OPL; ++j) {
        const int p = min(lane + 64 * j, C * 4 - 1), r = p >> 2, c4 = p & 3;
        ox[j] = ld4(d_o + (row0 + (size_t)(r < n ? r : 0) * H) * V + v0 + 4 * c4);
      }
      float vv[NB][4];
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * I + 4 * g + e;
          vv[I][e] = v[(row0 + (size_t)(t < n ? t : 0) * H) * V + v0 + s];
        }
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const int p = lane + 64 * j, r = p / (KD / 4), c4 = p - r * (KD / 4);
        if (act) pdot += (sx[j][0] * dx[j][0] + sx[j][1] * dx[j][1]) + (sx[j][2] * dx[j][2] + sx[j][3] * dx[j][3]);
        st4(A.S + r * LK + 4 * c4, sx[j]);
        st4(A.dS + r * LK + 4 * c4, dx[j]);
      }
#pragma unroll
      for (int j = 0; j < OPL; ++j) {
        const int p = lane + 64 * j, r = p >> 2, c4 = p & 3;
        if (p < C * 4) st4(A.dO + r * LV + 4 * c4, r < n ? ox[j] : zero4f());
      }
      wave_lds_sync();

      // Y, Z, W
      f32x4 Y[NB], Z[NB], Wt[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        Y[I] = Z[I] = Wt[I] = zero4f();
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) {
          const f32x4 ak = ld4(sK + (16 * I + s) * LK + 16 * kq + 4 * g);
          const f32x4 bs = ld4(A.S + s * LK + 16 * kq + 4 * g);
          Y[I] = mma16(ak, bs, Y[I]);
          Z[I] = mma16(ld4(sQ + (16 * I + s) * LK + 16 * kq + 4 * g), bs, Z[I]);
          Wt[I] = mma16(ak, ld4(A.dS + s * LK + 16 * kq + 4 * g), Wt[I]);
        }
      }
      // R, U = Tm R
      f32x4 R[NB], U[NB], dU[NB], dR[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * I + 4 * g + e;
          const float x = t < n ? vv[I][e] : 0.0f;
          vv[I][e] = x;
          R[I][e] = sb[t] * x - sb[t] * sgam[t] * Y[I][e];
        }
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        U[I] = zero4f();
#pragma unroll
        for (int J = 0; J <= I; ++J) U[I] = mma16(ld4(sT + (16 * I + s) * LCC + 16 * J + 4 * g), R[J], U[I]);
      }
      // dU = diag(D) W + P^T dO, dR = Tm^T dU
#pragma unroll
      for (int I = 0; I < NB; ++I) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dU[I][e] = sD[16 * I + 4 * g + e] * Wt[I][e];
#pragma unroll
        for (int J = I; J < NB; ++J) {
          f32x4 a, bo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = sP[(16 * J + 4 * g + e) * LCC + 16 * I + s];
            bo[e] = A.dO[(16 * J + 4 * g + e) * LV + s];
          }
          dU[I] = mma16(a, bo, dU[I]);
        }
      }
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        dR[I] = zero4f();
#pragma unroll
        for (int J = I; J < NB; ++J) {
          f32x4 a;
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] = sT[(16 * J + 4 * g + e) * LCC + 16 * I + s];
          dR[I] = mma16(a, dU[J], dR[I]);
        }
      }
      // dV, the per-token partial sums, U and dR to LDS
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * I + 4 * g + e;
          if (act) {
            if (t < n) dv[(row0 + (size_t)t * H) * V + v0 + s] = sb[t] * dR[I][e];
            pdb[I][e] += dR[I][e] * (vv[I][e] - sgam[t] * Y[I][e]);
            poz[I][e] += A.dO[t * LV + s] * Z[I][e];
            pry[I][e] += dR[I][e] * Y[I][e];
            puw[I][e] += U[I][e] * Wt[I][e];
          }
          A.U[t * LV + s] = U[I][e];
          A.dR[t * LV + s] = dR[I][e];
        }
      wave_lds_sync();
      // dP += dO U^T, dA += dR U^T (negated at the end), lower blocks
      if (act) {
#pragma unroll
        for (int I = 0; I < NB; ++I)
#pragma unroll
          for (int J = 0; J <= I; ++J) {
            const int blk = I * (I + 1) / 2 + J;
            const f32x4 bu = ld4(A.U + (16 * J + s) * LV + 4 * g);
            aP[blk] = mma16(ld4(A.dO + (16 * I + s) * LV + 4 * g), bu, aP[blk]);
            aA[blk] = mma16(ld4(A.dR + (16 * I + s) * LV + 4 * g), bu, aA[blk]);
          }
      }
    }
    __syncthreads();   // the round's slice tiles are complete
    // ---- dQ += diag(gam) dO S;  dK += diag(D) U dS' - diag(beta gam) dR S, over
    // the round's slices, for the key-channel tiles this wave owns
    for (int x = 0; x < NW && sl0 + x < nsl; ++x) {
      const WaveArea& X = area.wave[x];
      // the slice's S and dS' columns of the owned tiles serve every token block
      f32x4 bs[NKO], bd[NKO];
#pragma unroll
      for (int m = 0; m < NKO; ++m) {
        const int kq = min(w + NW * m, KQ - 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bs[m][e] = X.S[(4 * g + e) * LK + 16 * kq + s];
          bd[m][e] = X.dS[(4 * g + e) * LK + 16 * kq + s];
        }
      }
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        const int r = 16 * I + s;
        const f32x4 ao = ld4(X.dO + r * LV + 4 * g) * sgam[r];
        const f32x4 au = ld4(X.U + r * LV + 4 * g) * sD[r];
        const f32x4 ar = ld4(X.dR + r * LV + 4 * g) * (-sb[r] * sgam[r]);
#pragma unroll
        for (int m = 0; m < NKO; ++m) {
          if (w + NW * m < KQ) {
            aQ[I][m] = mma16(ao, bs[m], aQ[I][m]);
            aK[I][m] = mma16(ar, bs[m], mma16(au, bd[m], aK[I][m]));
          }
        }
      }
    }
    __syncthreads();   // the slice tiles may be overwritten
  }

  // per-token sums: over the 16 lanes of a group, then over the waves
#pragma unroll
  for (int I = 0; I < NB; ++I)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pdb[I][e] = group_sum(pdb[I][e]);
      poz[I][e] = group_sum(poz[I][e]);
      pry[I][e] = group_sum(pry[I][e]);
      puw[I][e] = group_sum(puw[I][e]);
    }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) pdot += __shfl_xor(pdot, m, 64);
  // the waves' partials to their own slots, then added in wave order
  Red& RD = area.red;
#pragma unroll
  for (int I = 0; I < NB; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      const int blk = I * (I + 1) / 2 + J;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int o2 = (16 * I + 4 * g + e) * LCC + 16 * J + s;
        RD.pP[w][o2] = aP[blk][e];
        RD.pA[w][o2] = aA[blk][e];
      }
    }
  if (s == 0) {
#pragma unroll
    for (int I = 0; I < NB; ++I)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * g + e;
        RD.pdb[w][t] = pdb[I][e];
        RD.pdg[w][t] = sgam[t] * poz[I][e] - sb[t] * sgam[t] * pry[I][e];
        RD.puw[w][t] = puw[I][e];
      }
  }
  if (lane == 0) sdot[w] = pdot;
  __syncthreads();
  // masks and signs: dP lower (j <= r), dA = -(dR U^T) strictly lower; the pair
  // terms X[r][j] = dP[r][j] P[r][j] + dA[r][j] beta_r M[r][j] (j < r)
  for (int i = tid; i < C * C; i += 256) {
    const int r = i / C, j = i - r * C;
    const int o = r * LCC + j;
    if (r >= n || j > r) {
      RD.dP[o] = 0.0f;
      RD.dA[o] = 0.0f;
      RD.X[o] = 0.0f;
    } else {
      float dp = RD.pP[0][o], da = RD.pA[0][o];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) {
        dp += RD.pP[ww][o];
        da += RD.pA[ww][o];
      }
      da = j == r ? 0.0f : -da;
      RD.dP[o] = dp;
      RD.dA[o] = da;
      RD.X[o] = j < r ? fmaf(da, sb[r] * sM[o], dp * sP[o]) : 0.0f;
    }
  }
  if (tid < C) {
    const int t = tid;
    float db = RD.pdb[0][t], dg = RD.pdg[0][t], du = sD[t] * RD.puw[0][t];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) {
      db += RD.pdb[ww][t];
      dg += RD.pdg[ww][t];
      du = fmaf(sD[t], RD.puw[ww][t], du);
    }
    sdb[t] = db;
    sdg[t] = dg;
    sdu[t] = du;
  }
  __syncthreads();
  // sxr[t] = sum over i < t <= r of X[r][i]: suffix sums down each column (one
  // thread per column), then the part of row t left of the diagonal (one
  // thread per row); and the row sums of dA o M for dbeta
  if (tid < C) {
    float acc = 0.0f;
    for (int r = C - 1; r > tid; --r) {
      acc += RD.X[r * LCC + tid];
      RD.X[r * LCC + tid] = acc;
    }
  }
  __syncthreads();
  if (tid < C) {
    const int t = tid;
    float sx = 0.0f, db = 0.0f;
    for (int i = 0; i < t; ++i) {
      sx += RD.X[t * LCC + i];
      db = fmaf(RD.dA[t * LCC + i], sM[t * LCC + i], db);
    }
    sxr[t] = sx;
    sdb[t] += db;
  }
  __syncthreads();
  // (dP o E) and (dA o beta E) in place
  for (int i = tid; i < C * C; i += 256) {
    const int r = i / C, j = i - r * C;
    if (r < n && j <= r) {
      const float e = expf(sg[r] - sg[j]);
      RD.dP[r * LCC + j] *= e;
      RD.dA[r * LCC + j] *= sb[r] * e;
    }
  }
  __syncthreads();
  // dQ += (dP o E) K;  dK += (dP o E)^T Q + (dA o bE) K + (dA o bE)^T K on the
  // owned key-channel tiles
#pragma unroll
  for (int m = 0; m < NKO; ++m) {
    const int kq = w + NW * m;
    if (kq >= KQ) continue;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 accq = aQ[I][m], acck = aK[I][m];
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        f32x4 bk, bq;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bk[e] = sK[(16 * J + 4 * g + e) * LK + 16 * kq + s];
          bq[e] = sQ[(16 * J + 4 * g + e) * LK + 16 * kq + s];
        }
        if (J <= I) {
          accq = mma16(ld4(RD.dP + (16 * I + s) * LCC + 16 * J + 4 * g), bk, accq);
          acck = mma16(ld4(RD.dA + (16 * I + s) * LCC + 16 * J + 4 * g), bk, acck);
        }
        if (J >= I) {
          f32x4 pt, at;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pt[e] = RD.dP[(16 * J + 4 * g + e) * LCC + 16 * I + s];
            at[e] = RD.dA[(16 * J + 4 * g + e) * LCC + 16 * I + s];
          }
          acck = mma16(pt, bq, acck);
          acck = mma16(at, bk, acck);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * g + e;
        if (t < n) {
          dq[(row0 + (size_t)t * H) * KD + 16 * kq + s] = accq[e];
          dk[(row0 + (size_t)t * H) * KD + 16 * kq + s] = acck[e];
        }
      }
    }
  }
  // gate gradients (the cancellation-free sums of bwd.hip), one lane per token:
  // d ln alpha_t = sum_{r >= t} dg_r (with gam_last <dS', S> on the last token)
  // + sxr_t + sum_{r < t} D_r U_r.W_r
  if (w == 0) {
    float dot = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) dot += sdot[ww];
    float dg = lane < n ? sdg[lane] : 0.0f;
    if (lane == n - 1) dg += sgam[n - 1] * dot;
    const float suf = __shfl(mfma::wave_scan(__shfl(dg, 63 - lane), lane), 63 - lane);
    const float pre = mfma::wave_scan(lane > 0 && lane - 1 < n ? sdu[lane - 1] : 0.0f, lane);
    if (lane < n) {
      const size_t go = row0 + (size_t)lane * H;
      dalpha[go] = (suf + sxr[lane] + pre) / alpha[go];
      dbeta[go] = sdb[lane];
    }
  }
}

template <int KD, int C>
hipError_t launch_kc(const BwdArgs& a, const float* rec, float* ws_dS, hipStream_t stream) {
  const long groups = ((long)a.B * a.H + 7) / 8;
  const float* q = static_cast<const float*>(a.q);
  const float* k = static_cast<const float*>(a.k);
  const float* d_o = static_cast<const float*>(a.d_o);
  if (a.V % 32 == 0 && (long)a.B * a.H * (a.V / 32) >= 128)
    hipLaunchKernelGGL((f32_dstate_kernel<KD, C, 2>), dim3(8 * groups * (a.V / 32)),
                       dim3(128 * (C / 16)), 0, stream, q, k, d_o, a.d_sfinal, a.d_s0, rec, ws_dS,
                       a.B, a.T, a.H, a.V);
  else
    hipLaunchKernelGGL((f32_dstate_kernel<KD, C, 1>), dim3(8 * groups * (a.V / 16)),
                       dim3(64 * (C / 16)), 0, stream, q, k, d_o, a.d_sfinal, a.d_s0, rec, ws_dS,
                       a.B, a.T, a.H, a.V);
  return hipGetLastError();
}

template <int KD, int C>
hipError_t launch_walks_kc(const BwdArgs& a, const float* rec, float* ws_S, float* ws_dS,
                           hipStream_t stream) {
  const long groups = ((long)a.B * a.H + 7) / 8;
  const int nd = (int)(8 * groups * (a.V / 32));
  const int NT = (a.T + C - 1) / C;
  hipLaunchKernelGGL((f32_walks_kernel<KD, C>), dim3(2 * nd), dim3(128 * (C / 16)), 0, stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), a.s0, ws_S, static_cast<const float*>(a.d_o),
                     a.d_sfinal, a.d_s0, rec, ws_dS, a.B, a.T, a.H, a.V, NT, nd);
  return hipGetLastError();
}

template <int KD>
hipError_t launch_k(const BwdArgs& a, int C, const float* rec, float* ws_dS, hipStream_t stream) {
  if (C == 16) return launch_kc<KD, 16>(a, rec, ws_dS, stream);
  return launch_kc<KD, 32>(a, rec, ws_dS, stream);
}

template <int KD>
hipError_t launch_local_k(const BwdArgs& a, int C, const float* ws_S, const float* ws_dS,
                          const float* ws_F, hipStream_t stream) {
  const int NT = (a.T + C - 1) / C;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(NT * a.H * a.B), dim3(256), 0, stream,
                       static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.v), static_cast<const float*>(a.d_o), a.alpha,
                       ws_S, ws_dS, ws_F, static_cast<float*>(a.dq), static_cast<float*>(a.dk),
                       static_cast<float*>(a.dv), a.dalpha, a.dbeta, a.T, a.H, a.V);
    return hipGetLastError();
  };
  if (C == 16) return go(f32_local_kernel<KD, 16>);
  return go(f32_local_kernel<KD, 32>);
}

}  // namespace

hipError_t launch_bwd_f32_local(const BwdArgs& a, int chunk, const float* ws_S, const float* ws_dS,
                                const float* ws_F, hipStream_t stream) {
  if ((chunk != 16 && chunk != 32) || a.V % 16 != 0) return hipErrorInvalidValue;
  switch (a.K) {
    case 16: return launch_local_k<16>(a, chunk, ws_S, ws_dS, ws_F, stream);
    case 32: return launch_local_k<32>(a, chunk, ws_S, ws_dS, ws_F, stream);
    case 64: return launch_local_k<64>(a, chunk, ws_S, ws_dS, ws_F, stream);
    case 128: return launch_local_k<128>(a, chunk, ws_S, ws_dS, ws_F, stream);
  }
  return hipErrorInvalidValue;
}

bool bwd_f32_walks_supported(int K, int V, int chunk) {
  return (K == 16 || K == 32 || K == 64 || K == 128) && V > 0 && V % 32 == 0 && V <= 128 &&
         (chunk == 16 || chunk == 32);
}

hipError_t launch_bwd_f32_walks(const BwdArgs& a, int chunk, const float* rec, float* ws_S,
                                float* ws_dS, hipStream_t stream) {
  if (!bwd_f32_walks_supported(a.K, a.V, chunk)) return hipErrorInvalidValue;
  auto by_c = [&](auto kc) -> hipError_t {
    constexpr int KD = decltype(kc)::value;
    if (chunk == 16) return launch_walks_kc<KD, 16>(a, rec, ws_S, ws_dS, stream);
    return launch_walks_kc<KD, 32>(a, rec, ws_S, ws_dS, stream);
  };
  switch (a.K) {
    case 16: return by_c(std::integral_constant<int, 16>());
    case 32: return by_c(std::integral_constant<int, 32>());
    case 64: return by_c(std::integral_constant<int, 64>());
    case 128: return by_c(std::integral_constant<int, 128>());
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_f32_dstate(const BwdArgs& a, int chunk, const float* rec, float* ws_dS,
                                 hipStream_t stream) {
  if ((chunk != 16 && chunk != 32) || a.V % 16 != 0) return hipErrorInvalidValue;
  switch (a.K) {
    case 16: return launch_k<16>(a, chunk, rec, ws_dS, stream);
    case 32: return launch_k<32>(a, chunk, rec, ws_dS, stream);
    case 64: return launch_k<64>(a, chunk, rec, ws_dS, stream);
    case 128: return launch_k<128>(a, chunk, rec, ws_dS, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
