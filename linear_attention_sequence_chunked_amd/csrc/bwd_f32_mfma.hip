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
template <int KD, int C, int NG>
__global__ void __launch_bounds__(64 * NG * (C / 16), 1)
f32_dstate_kernel(const float* __restrict__ q, const float* __restrict__ k,
                  const float* __restrict__ d_o, const float* __restrict__ d_sfinal,
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
  struct Grp {
    float sS[16 * LS];                       // dS' [v][k]
    float sdO[2][16 * LC];                   // dO^T [v][t]
    float sdU[16 * LC];                      // dU^T [v][t]
    float sdR[16 * LC];                      // (-beta gam dR)^T [v][t]
  };
  __shared__ __attribute__((aligned(16))) float sK[2][C * LS];
  __shared__ __attribute__((aligned(16))) float sQ[2][C * LS];
  __shared__ __attribute__((aligned(16))) float sRec[2][RF];
  __shared__ __attribute__((aligned(16))) Grp grp[NG];

  const int tid = threadIdx.x, lane = tid & 63, wg = tid >> 6;
  const int gi = wg / NB, w = wg - gi * NB;
  const int s = lane & 15, g = lane >> 4;
  Grp& G = grp[gi];
  // the workgroups of one (batch, head) share an XCD, so its records and tiles
  // are fetched into one L2
  const int nvs = V / (16 * NG), streams = B * H;
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
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

    // dS'^T <- gam_n dS'^T + Q^T diag(gam) dO + K^T (-beta gam dR), owned tiles
    const float gn = rc[Rec<C>::kGn];
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
        const f32x4 gd = ld4(dot + s * LC + 16 * J + 4 * g) * ld4(rc + Rec<C>::kGam + 16 * J + 4 * g);
        acc = mma16(aq, gd, acc);
        acc = mma16(ak, ld4(G.sdR + s * LC + 16 * J + 4 * g), acc);
      }
      S[m] = acc;
      st4(G.sS + s * LS + 16 * kap + 4 * g, acc);
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

template <int KD>
hipError_t launch_k(const BwdArgs& a, int C, const float* rec, float* ws_dS, hipStream_t stream) {
  if (C == 16) return launch_kc<KD, 16>(a, rec, ws_dS, stream);
  return launch_kc<KD, 32>(a, rec, ws_dS, stream);
}

}  // namespace

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
