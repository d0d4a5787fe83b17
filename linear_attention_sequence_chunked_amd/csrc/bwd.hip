// Chunkwise gated-delta-rule backward: reverse mode of the forward in
// fwd_f32.hip / fwd_bf16.hip for the loss <o, dO> + <S_final, dS_final>.
//
// The chunk form of the forward ("Sparse Delta Memory: layer and kernels",
// section "What the layer computes"; operator contract of "OpenGDN 0.1.0",
// section "Core operator reference"), for a chunk of n tokens with start state S:
//
//   g = cumsum(ln alpha), gam = e^g, D = e^(g_last - g)
//   M_ri = e^(g_r - g_i) k_r.k_i (i < r),  A = diag(beta) M,  Tm = (I + A)^-1
//   P_ri = e^(g_r - g_i) q_r.k_i (i <= r)
//   Y = K S^T, Z = Q S^T, R = diag(beta) V - diag(beta gam) Y, U = Tm R
//   O = diag(gam) Z + P U,  S' = gam_last S + U^T diag(D) K
//
// differentiated by hand.  With dS' the gradient of the chunk-end state:
//
//   W  = K dS'^T,  dU = diag(D) W + P^T dO,  dR = Tm^T dU
//   dS (chunk start) = gam_last dS' + dO^T diag(gam) Q - dR^T diag(beta gam) K
//   dP = tril(dO U^T),  dA = strict_tril(-dR U^T)
//   dQ = diag(gam) dO S + (dP o E) K                       (E_ri = e^(g_r - g_i))
//   dK = diag(D) U dS' - diag(beta gam) dR S + (dP o E)^T Q + (dA o bE) K + (dA o bE)^T K
//   dV = diag(beta) dR
//   dbeta_r = dR_r.(v_r - gam_r Y_r) + sum_i dA_ri M_ri
//   dg_r = gam_r dO_r.Z_r - beta_r gam_r dR_r.Y_r
//          + sum_i (dP o P)_ri - sum_i (dP o P)_ir + sum_i (dA o A)_ri - sum_i (dA o A)_ir
//   dg_last += gam_last <dS', S> + sum_r D_r U_r.W_r
//   d ln alpha_t = sum_{r >= t} dg_r,   dalpha_t = d ln alpha_t / alpha_t
//
// which is summed here in an equal form without cancellation:
//   d ln alpha_t = sum_{r >= t} (gam_r dO_r.Z_r - beta_r gam_r dR_r.Y_r)
//                + sum_{r >= t} sum_{i < t} ((dP o P)_ri + (dA o A)_ri)
//                + sum_{r < t} D_r U_r.W_r + gam_last <dS', S>
// (every (dP o P + dA o A)_ri with i and r both >= t enters the suffix twice
// with opposite signs, and the U.W terms, the derivative through
// D_r = e^(g_last - g_r), reach token t only for r < t; with small gates
// d ln alpha_t is tiny next to those terms, and the chunk total minus a suffix
// would lose it to rounding).
//
// Four steps: (1) the forward kernel of the input dtype recomputes the
// chunk-start states into the workspace; (2a) every chunk builds its
// state-independent factors M, P, Tm and gates in parallel (for float32 inputs
// the chunk-parallel launch of (1)'s matrix-core forward writes them); (2b) a
// reverse walk over the chunks carries dS and stores each chunk's dS'; (3)
// every chunk computes its token gradients independently.  Float32 inputs run
// (1), (2b) and (3) on the fp32 matrix cores (fwd_f32_mfma.hip,
// bwd_f32_mfma.hip); bfloat16 inputs with K or V = 16 take the scalar kernels
// of this file.
// All arithmetic is fp32 in a fixed order (bitwise reproducible); inputs and the
// dq, dk, dv outputs have the dtype of q.  The backward chunk is at most 32
// tokens (chunk size changes results only by rounding).
#include "launch.h"

#include <hip/hip_bf16.h>

#include <type_traits>

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kBwdC = 32;   // backward chunk (tokens)

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__hip_bfloat16 x) { return __bfloat162float(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __hip_bfloat16 from_f32<__hip_bfloat16>(float x) {
  return __float2bfloat16(x);  // round to nearest even
}

// Gates of one chunk into LDS: g (cumulative natural-log gate, summed in token
// order), gam = e^g, beta.  Leaves a barrier behind.
__device__ __forceinline__ void load_gates(const float* alpha, const float* beta, float* sg,
                                           float* sgam, float* sb, int b, int h, int T, int H,
                                           int t0, int n, int tid) {
  if (tid < n) {
    const size_t go = ((size_t)b * T + t0 + tid) * H + h;
    sg[tid] = logf(alpha[go]);
    sb[tid] = beta[go];
  }
  __syncthreads();
  if (tid == 0) {
    float acc = 0.0f;
    for (int r = 0; r < n; ++r) {
      acc += sg[r];
      sg[r] = acc;
    }
  }
  __syncthreads();
  if (tid < n) sgam[tid] = expf(sg[tid]);
  __syncthreads();
}

// M (strictly lower, decayed K K^T, no beta), P (lower, decayed Q K^T) and
// Tm = (I + diag(beta) M)^-1 by forward substitution (one column per thread).
// Key/query rows have leading dimension LK (K + 1: threads reading different
// rows hit different banks); the C x C results have leading dimension C.
// Leaves a barrier behind.
__device__ __forceinline__ void chunk_mats(const float* sq, const float* sk, const float* sg,
                                           const float* sb, float* sM, float* sP, float* sT,
                                           int n, int C, int K, int LK, int tid) {
  for (int i = tid; i < C * C; i += kThreads) {
    const int r = i / C, j = i - r * C;
    float m = 0.0f, p = 0.0f;
    if (r < n && j <= r) {
      float dk = 0.0f, dq = 0.0f;
      for (int c = 0; c < K; ++c) {
        dk = fmaf(sk[r * LK + c], sk[j * LK + c], dk);
        dq = fmaf(sq[r * LK + c], sk[j * LK + c], dq);
      }
      const float e = expf(sg[r] - sg[j]);
      if (j < r) m = e * dk;
      p = e * dq;
    }
    sM[i] = m;
    sP[i] = p;
  }
  __syncthreads();
  if (tid < n) {
    const int j = tid;
    for (int r = 0; r < j; ++r) sT[r * C + j] = 0.0f;
    sT[j * C + j] = 1.0f;
    for (int r = j + 1; r < n; ++r) {
      float s = 0.0f;
      for (int i = j; i < r; ++i) s = fmaf(sb[r] * sM[r * C + i], sT[i * C + j], s);
      sT[r * C + j] = -s;
    }
  }
  __syncthreads();
}

// Per-chunk factor record in the workspace: M, P, Tm (C x C each), then g, gam,
// beta (C each).
__host__ __device__ constexpr int factor_floats(int C) { return 3 * C * C + 3 * C; }

// Copy a chunk's factor record into LDS (M skipped when sM is null).  Leaves a
// barrier behind.
__device__ __forceinline__ void load_factors(const float* f, float* sM, float* sP, float* sT,
                                             float* sg, float* sgam, float* sb, int C, int tid) {
  const int CC = C * C;
  for (int i = tid; i < CC; i += kThreads) {
    if (sM) sM[i] = f[i];
    sP[i] = f[CC + i];
    sT[i] = f[2 * CC + i];
  }
  if (tid < C) {
    sg[tid] = f[3 * CC + tid];
    sgam[tid] = f[3 * CC + C + tid];
    sb[tid] = f[3 * CC + 2 * C + tid];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// (2a) State-independent factors of every chunk, in parallel: one workgroup per
// (chunk, head, batch).
template <typename TIn>
__global__ void __launch_bounds__(kThreads)
bwd_prep_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                const float* __restrict__ alpha, const float* __restrict__ beta,
                float* __restrict__ ws_F, int T, int H, int K, int C) {
  extern __shared__ float lds[];
  const int LK = K + 1;
  float* sq = lds;                 // [C][LK]
  float* sk = sq + C * LK;         // [C][LK]
  float* sM = sk + C * LK;         // [C][C]
  float* sP = sM + C * C;
  float* sT = sP + C * C;
  float* sg = sT + C * C;          // [C]
  float* sgam = sg + C;
  float* sb = sgam + C;
  const int tid = threadIdx.x;
  const int NT = (T + C - 1) / C;
  // one-dimensional grid over (chunk, head, batch), chunk fastest
  const int c = blockIdx.x % NT, h = (blockIdx.x / NT) % H, b = blockIdx.x / NT / H;
  const int t0 = c * C;
  const int n = min(C, T - t0);
  for (int i = tid; i < n * K; i += kThreads) {
    const int r = i / K, e = i - r * K;
    const size_t off = (((size_t)b * T + t0 + r) * H + h) * (size_t)K + e;
    sq[r * LK + e] = to_f32(q[off]);
    sk[r * LK + e] = to_f32(k[off]);
  }
  load_gates(alpha, beta, sg, sgam, sb, b, h, T, H, t0, n, tid);
  chunk_mats(sq, sk, sg, sb, sM, sP, sT, n, C, K, LK, tid);
  float* f = ws_F + (((size_t)b * H + h) * NT + c) * factor_floats(C);
  const int CC = C * C;
  for (int i = tid; i < CC; i += kThreads) {
    const int r = i / C, j = i - r * C;
    const bool in = r < n && j < n;  // rows and columns past the tail are zero
    f[i] = sM[i];
    f[CC + i] = sP[i];
    f[2 * CC + i] = in ? sT[i] : 0.0f;
  }
  if (tid < C) {
    f[3 * CC + tid] = tid < n ? sg[tid] : 0.0f;
    f[3 * CC + C + tid] = tid < n ? sgam[tid] : 0.0f;
    f[3 * CC + 2 * C + tid] = tid < n ? sb[tid] : 0.0f;
  }
}

// ---------------------------------------------------------------------------
// (2b) Reverse walk: one workgroup per (batch, head, value slice of VS rows).
// Stores dS' of every chunk to ws_dS [B, H, NT, V, K] and the gradient of the
// initial state.
// Eight consecutive elements as floats (16 bytes of bf16 or 32 bytes of fp32).
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const __hip_bfloat16* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename TIn, int K>
__global__ void __launch_bounds__(kThreads)
bwd_dstate_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ d_o,
                  const float* __restrict__ d_sfinal, float* __restrict__ d_s0,
                  const float* __restrict__ ws_F, float* __restrict__ ws_dS, int T, int H,
                  int V, int C, int VS) {
  extern __shared__ float lds[];
  const int LK = K + 1, LV = VS + 1;  // padded rows: no bank conflicts across rows
  float* sq = lds;                 // [C][LK]
  float* sk = sq + C * LK;         // [C][LK]
  float* sdo = sk + C * LK;        // [C][LV]  diag(gam) dO
  float* sP = sdo + C * LV;        // [C][C]
  float* sT = sP + C * C;          // [C][C]
  float* sdU = sT + C * C;         // [C][LV]
  float* sdR = sdU + C * LV;       // [C][LV]  -diag(beta gam) dR
  float* sdS = sdR + C * LV;       // [VS][LK]
  float* sg = sdS + VS * LK;       // [C]
  float* sgam = sg + C;
  float* sb = sgam + C;

  const int tid = threadIdx.x;
  // one-dimensional grid over (value slice, head, batch), value slice fastest
  const int nvs = V / VS;
  const int v0 = (blockIdx.x % nvs) * VS;
  const int h = (blockIdx.x / nvs) % H;
  const int b = blockIdx.x / nvs / H;
  const int NT = (T + C - 1) / C;
  const size_t state_base = ((size_t)b * H + h) * (size_t)V * K + (size_t)v0 * K;

  // Registers of the next chunk's inputs: they are requested while the current
  // chunk is computed.  Pieces of 8 elements: q/k rows (KP8 per thread), the dO
  // slice, and the chunk's P, Tm and gates.
  constexpr int KP8 = kBwdC * 128 / 8 / kThreads;   // 2
  float nq[KP8][8], nk[KP8][8], ndo[2], nP[4], nT[4], ng[3];
  auto fetch = [&](int c) {
    const int t0 = c * C, n = min(C, T - t0);
#pragma unroll
    for (int u = 0; u < KP8; ++u) {
      const int piece = tid + u * kThreads, r = piece / (K / 8), e8 = (piece % (K / 8)) * 8;
      if (r < n) {
        const size_t off = (((size_t)b * T + t0 + r) * H + h) * (size_t)K + e8;
        load8(q + off, nq[u]);
        load8(k + off, nk[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + u * kThreads, r = i / VS, e = i - r * VS;
      ndo[u] = r < n ? to_f32(d_o[(((size_t)b * T + t0 + r) * H + h) * (size_t)V + v0 + e]) : 0.0f;
    }
    const float* f = ws_F + (((size_t)b * H + h) * NT + c) * factor_floats(C);
    const int CC = C * C;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + u * kThreads;
      nP[u] = i < CC ? f[CC + i] : 0.0f;
      nT[u] = i < CC ? f[2 * CC + i] : 0.0f;
    }
    if (tid < C) {
      ng[0] = f[3 * CC + tid];
      ng[1] = f[3 * CC + C + tid];
      ng[2] = f[3 * CC + 2 * C + tid];
    }
  };

  for (int i = tid; i < VS * K; i += kThreads)
    sdS[(i / K) * LK + i % K] = d_sfinal ? d_sfinal[state_base + i] : 0.0f;
  fetch(NT - 1);

  for (int c = NT - 1; c >= 0; --c) {
    const int t0 = c * C;
    const int n = min(C, T - t0);
    __syncthreads();
    float* dst = ws_dS + ((((size_t)b * H + h) * NT + c) * V + v0) * (size_t)K;
    for (int i = tid; i < VS * K; i += kThreads) dst[i] = sdS[(i / K) * LK + i % K];
    // stage the fetched chunk
#pragma unroll
    for (int u = 0; u < KP8; ++u) {
      const int piece = tid + u * kThreads, r = piece / (K / 8), e8 = (piece % (K / 8)) * 8;
      if (r < n) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          sq[r * LK + e8 + j] = nq[u][j];
          sk[r * LK + e8 + j] = nk[u][j];
        }
      }
    }
    const int CC = C * C;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + u * kThreads;
      if (i < CC) {
        sP[i] = nP[u];
        sT[i] = nT[u];
      }
    }
    if (tid < C) {
      sg[tid] = ng[0];
      sgam[tid] = ng[1];
      sb[tid] = ng[2];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + u * kThreads, r = i / VS, e = i - r * VS;
      if (r < C) sdo[r * LV + e] = ndo[u];
    }
    if (c > 0) fetch(c - 1);  // overlaps the arithmetic below
    const float glast = sg[n - 1];
    __syncthreads();
    // dU = diag(D) K dS'^T + P^T dO
    for (int i = tid; i < n * VS; i += kThreads) {
      const int r = i / VS, e = i - r * VS;
      float w = 0.0f;
      for (int j = 0; j < K; ++j) w = fmaf(sk[r * LK + j], sdS[e * LK + j], w);
      float acc = expf(glast - sg[r]) * w;
      for (int rr = r; rr < n; ++rr) acc = fmaf(sP[rr * C + r], sdo[rr * LV + e], acc);
      sdU[r * LV + e] = acc;
    }
    __syncthreads();
    // dR = Tm^T dU, kept scaled by -beta gam; dO scaled by gam (for the update)
    for (int i = tid; i < n * VS; i += kThreads) {
      const int r = i / VS, e = i - r * VS;
      float acc = 0.0f;
      for (int rr = r; rr < n; ++rr) acc = fmaf(sT[rr * C + r], sdU[rr * LV + e], acc);
      sdR[r * LV + e] = -sb[r] * sgam[r] * acc;
    }
    __syncthreads();
    for (int i = tid; i < n * VS; i += kThreads) {
      const int r = i / VS, e = i - r * VS;
      sdo[r * LV + e] *= sgam[r];
    }
    __syncthreads();
    // dS <- gam_last dS + dO^T diag(gam) Q - dR^T diag(beta gam) K.  A thread
    // owns one channel j and the rows e = e0, e0 + 2, ..: q and k of token r are
    // read once for all of them.
    const float gam_last = sgam[n - 1];
    {
      const int j = tid % K, e0 = tid / K, es = kThreads / K;
      float acc[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) acc[u] = (e0 + u * es < VS) ? gam_last * sdS[(e0 + u * es) * LK + j] : 0.0f;
      for (int r = 0; r < n; ++r) {
        const float qv = sq[r * LK + j], kv = sk[r * LK + j];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + u * es;
          if (e < VS) acc[u] = fmaf(sdR[r * LV + e], kv, fmaf(sdo[r * LV + e], qv, acc[u]));
        }
      }
      __syncthreads();  // every thread has read the old dS
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (e0 + u * es < VS) sdS[(e0 + u * es) * LK + j] = acc[u];
    }
  }
  __syncthreads();
  if (d_s0)
    for (int i = tid; i < VS * K; i += kThreads) d_s0[state_base + i] = sdS[(i / K) * LK + i % K];
}

// ---------------------------------------------------------------------------
// (3) Token gradients of one chunk: one workgroup per (chunk, head, batch).
// dQ and dK accumulate in registers (QPT elements per thread), dP and dA in
// LDS; the value axis is walked in slices of VS.
constexpr int kBwdVS = 32;  // value slice of the local kernel
constexpr int kQPT = kBwdC * 128 / kThreads;

template <typename TIn, int K>
__global__ void __launch_bounds__(kThreads)
bwd_local_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
                 const TIn* __restrict__ d_o, const float* __restrict__ alpha,
                 const float* __restrict__ beta, const float* __restrict__ ws_S,
                 const float* __restrict__ ws_dS, const float* __restrict__ ws_F,
                 TIn* __restrict__ dq, TIn* __restrict__ dk,
                 TIn* __restrict__ dv, float* __restrict__ dalpha, float* __restrict__ dbeta,
                 int T, int H, int V, int C) {
  constexpr int VS = kBwdVS;
  const int LK = K + 1;            // padded rows: no bank conflicts across rows
  constexpr int LV = VS + 1;
  extern __shared__ float lds[];
  float* sq = lds;                 // [C][LK]
  float* sk = sq + C * LK;         // [C][LK]
  float* sM = sk + C * LK;         // [C][C]
  float* sP = sM + C * C;
  float* sT = sP + C * C;
  float* sdP = sT + C * C;
  float* sdA = sdP + C * C;
  float* sv = sdA + C * C;         // [C][LV] slices
  float* sdo = sv + C * LV;
  float* sY = sdo + C * LV;
  float* sZ = sY + C * LV;
  float* sW = sZ + C * LV;
  float* sU = sW + C * LV;         // R, then U
  float* sdU = sU + C * LV;
  float* sdR = sdU + C * LV;
  float* sS = sdR + C * LV;        // [VS][LK]
  float* sdS = sS + VS * LK;       // [VS][LK]
  float* sg = sdS + VS * LK;       // [C]
  float* sgam = sg + C;
  float* sb = sgam + C;
  float* sdb = sb + C;             // dbeta accumulator
  float* sdg = sdb + C;            // dg accumulator
  float* sdu = sdg + C;            // D_r U_r.W_r accumulator
  float* sxr = sdu + C;            // cross sums of dP o P + dA o A per token
  float* sred = sxr + C;           // [kThreads] reduction scratch

  const int tid = threadIdx.x;
  const int NT = (T + C - 1) / C;
  // one-dimensional grid over (chunk, head, batch), chunk fastest
  const int c = blockIdx.x % NT;
  const int h = (blockIdx.x / NT) % H;
  const int b = blockIdx.x / NT / H;
  const int t0 = c * C;
  const int n = min(C, T - t0);
  const size_t ck = (((size_t)b * H + h) * NT + c) * (size_t)V * K;

  for (int i = tid; i < n * K; i += kThreads) {
    const int r = i / K, e = i - r * K;
    const size_t off = (((size_t)b * T + t0 + r) * H + h) * (size_t)K + e;
    sq[r * LK + e] = to_f32(q[off]);
    sk[r * LK + e] = to_f32(k[off]);
  }
  if (tid < C) {
    sdb[tid] = 0.0f;
    sdg[tid] = 0.0f;
    sdu[tid] = 0.0f;
  }
  for (int i = tid; i < C * C; i += kThreads) {
    sdP[i] = 0.0f;
    sdA[i] = 0.0f;
  }
  load_factors(ws_F + (((size_t)b * H + h) * NT + c) * factor_floats(C), sM, sP, sT, sg, sgam, sb,
               C, tid);
  const float glast = sg[n - 1];
  const float gam_last = sgam[n - 1];

  float aq[kQPT], ak[kQPT];
#pragma unroll
  for (int j = 0; j < kQPT; ++j) aq[j] = ak[j] = 0.0f;
  float sdot = 0.0f;  // <dS', S>, per-thread partial

  for (int v0 = 0; v0 < V; v0 += VS) {
    const int vs = min(VS, V - v0);
    __syncthreads();
    for (int i = tid; i < n * vs; i += kThreads) {
      const int r = i / vs, e = i - r * vs;
      const size_t off = (((size_t)b * T + t0 + r) * H + h) * (size_t)V + v0 + e;
      sv[r * LV + e] = to_f32(v[off]);
      sdo[r * LV + e] = to_f32(d_o[off]);
    }
    for (int i = tid; i < vs * K; i += kThreads) {
      const int e = i / K, j = i - e * K;
      sS[e * LK + j] = ws_S[ck + (size_t)v0 * K + i];
      sdS[e * LK + j] = ws_dS[ck + (size_t)v0 * K + i];
    }
    __syncthreads();
    // Y = K S^T, Z = Q S^T, W = K dS'^T;  R = diag(beta) V - diag(beta gam) Y
    for (int i = tid; i < n * vs; i += kThreads) {
      const int r = i / vs, e = i - r * vs;
      float y = 0.0f, z = 0.0f, w = 0.0f;
      for (int j = 0; j < K; ++j) {
        const float kk = sk[r * LK + j];
        y = fmaf(kk, sS[e * LK + j], y);
        z = fmaf(sq[r * LK + j], sS[e * LK + j], z);
        w = fmaf(kk, sdS[e * LK + j], w);
      }
      sY[r * LV + e] = y;
      sZ[r * LV + e] = z;
      sW[r * LV + e] = w;
      sdR[r * LV + e] = sb[r] * sv[r * LV + e] - sb[r] * sgam[r] * y;  // R (temporary)
    }
    __syncthreads();
    // U = Tm R;  <dS', S> partials
    for (int i = tid; i < n * vs; i += kThreads) {
      const int r = i / vs, e = i - r * vs;
      float u = 0.0f;
      for (int j = 0; j <= r; ++j) u = fmaf(sT[r * C + j], sdR[j * LV + e], u);
      sU[r * LV + e] = u;
    }
    for (int i = tid; i < vs * K; i += kThreads) {
      const int e = i / K, j = i - e * K;
      sdot = fmaf(sdS[e * LK + j], sS[e * LK + j], sdot);
    }
    __syncthreads();
    // dU = diag(D) W + P^T dO
    for (int i = tid; i < n * vs; i += kThreads) {
      const int r = i / vs, e = i - r * vs;
      float acc = expf(glast - sg[r]) * sW[r * LV + e];
      for (int rr = r; rr < n; ++rr) acc = fmaf(sP[rr * C + r], sdo[rr * LV + e], acc);
      sdU[r * LV + e] = acc;
    }
    __syncthreads();
    // dR = Tm^T dU
    for (int i = tid; i < n * vs; i += kThreads) {
      const int r = i / vs, e = i - r * vs;
      float acc = 0.0f;
      for (int rr = r; rr < n; ++rr) acc = fmaf(sT[rr * C + r], sdU[rr * LV + e], acc);
      sdR[r * LV + e] = acc;
    }
    __syncthreads();
    // dP += dO U^T (lower), dA -= dR U^T (strictly lower): each element has one owner
    for (int i = tid; i < C * C; i += kThreads) {
      const int r = i / C, j = i - r * C;
      if (r < n && j <= r) {
        float p = 0.0f, a = 0.0f;
        for (int e = 0; e < vs; ++e) {
          p = fmaf(sdo[r * LV + e], sU[j * LV + e], p);
          a = fmaf(sdR[r * LV + e], sU[j * LV + e], a);
        }
        sdP[i] += p;
        if (j < r) sdA[i] -= a;
      }
    }
    // dQ += diag(gam) dO S;  dK += diag(D) U dS' - diag(beta gam) dR S
#pragma unroll
    for (int jj = 0; jj < kQPT; ++jj) {
      const int i = tid + jj * kThreads;
      const int r = i / K, j = i - r * K;
      if (r < n) {
        float zq = 0.0f, zu = 0.0f, zr = 0.0f;
        for (int e = 0; e < vs; ++e) {
          const float s = sS[e * LK + j];
          zq = fmaf(sdo[r * LV + e], s, zq);
          zu = fmaf(sU[r * LV + e], sdS[e * LK + j], zu);
          zr = fmaf(sdR[r * LV + e], s, zr);
        }
        aq[jj] = fmaf(sgam[r], zq, aq[jj]);
        ak[jj] = fmaf(expf(glast - sg[r]), zu, ak[jj]);
        ak[jj] = fmaf(-sb[r] * sgam[r], zr, ak[jj]);
      }
    }
    // dV = diag(beta) dR
    for (int i = tid; i < n * vs; i += kThreads) {
      const int r = i / vs, e = i - r * vs;
      dv[(((size_t)b * T + t0 + r) * H + h) * (size_t)V + v0 + e] = from_f32<TIn>(sb[r] * sdR[r * LV + e]);
    }
    // per-token sums over this slice
    if (tid < n) {
      const int r = tid;
      float db = 0.0f, oz = 0.0f, ry = 0.0f, uw = 0.0f;
      for (int e = 0; e < vs; ++e) {
        const float y = sY[r * LV + e], dr = sdR[r * LV + e];
        db = fmaf(dr, sv[r * LV + e] - sgam[r] * y, db);
        oz = fmaf(sdo[r * LV + e], sZ[r * LV + e], oz);
        ry = fmaf(dr, y, ry);
        uw = fmaf(sU[r * LV + e], sW[r * LV + e], uw);
      }
      sdb[r] += db;
      sdg[r] += sgam[r] * oz - sb[r] * sgam[r] * ry;
      sdu[r] = fmaf(expf(glast - sg[r]), uw, sdu[r]);
    }
  }
  __syncthreads();
  // (dP o E) and beta (dA o E) in place, dg and dbeta terms of P and A: token t
  // sums the pairs i < t <= r (rows r >= t, columns i < t) in a fixed order
  if (tid < n) {
    const int t = tid;
    float s = 0.0f, db = 0.0f;
    for (int r = t; r < n; ++r) {
      const float br = sb[r];
      for (int i = 0; i < t; ++i) {
        s = fmaf(sdP[r * C + i], sP[r * C + i], s);
        s = fmaf(sdA[r * C + i], br * sM[r * C + i], s);
      }
    }
    for (int i = 0; i < t; ++i) db = fmaf(sdA[t * C + i], sM[t * C + i], db);
    sxr[t] = s;
    sdb[t] += db;
  }
  // reduction of the <dS', S> partials (fixed order)
  sred[tid] = gam_last * sdot;
  __syncthreads();
  for (int i = tid; i < C * C; i += kThreads) {
    const int r = i / C, j = i - r * C;
    if (r < n && j <= r) {
      const float e = expf(sg[r] - sg[j]);
      sdP[i] *= e;
      sdA[i] *= sb[r] * e;
    }
  }
  for (int st = kThreads / 2; st > 0; st >>= 1) {
    if (tid < st) sred[tid] += sred[tid + st];
    __syncthreads();
  }
  // dQ += (dP o E) K;  dK += (dP o E)^T Q + (dA o bE) K + (dA o bE)^T K
#pragma unroll
  for (int jj = 0; jj < kQPT; ++jj) {
    const int i = tid + jj * kThreads;
    const int r = i / K, j = i - r * K;
    if (r < n) {
      float zq = 0.0f, zk = 0.0f;
      for (int ii = 0; ii <= r; ++ii) zq = fmaf(sdP[r * C + ii], sk[ii * LK + j], zq);
      for (int rr = r; rr < n; ++rr) zk = fmaf(sdP[rr * C + r], sq[rr * LK + j], zk);
      for (int ii = 0; ii < r; ++ii) zk = fmaf(sdA[r * C + ii], sk[ii * LK + j], zk);
      for (int rr = r + 1; rr < n; ++rr) zk = fmaf(sdA[rr * C + r], sk[rr * LK + j], zk);
      const size_t off = (((size_t)b * T + t0 + r) * H + h) * (size_t)K + j;
      dq[off] = from_f32<TIn>(aq[jj] + zq);
      dk[off] = from_f32<TIn>(ak[jj] + zk);
    }
  }
  if (tid == 0) {
    sdg[n - 1] += sred[0];
    // prefix sums of the U.W terms (sdg's slots hold the results in place)
    float pre = 0.0f;
    for (int r = 0; r < n; ++r) {
      const float du = sdu[r];
      sdu[r] = pre;  // sum_{r' < r}
      pre += du;
    }
    float acc = 0.0f;  // suffix sums of the per-token terms (gam_last <dS', S> on the last)
    for (int r = n - 1; r >= 0; --r) {
      acc += sdg[r];
      const size_t go = ((size_t)b * T + t0 + r) * H + h;
      dalpha[go] = (acc + sxr[r] + sdu[r]) / alpha[go];
      dbeta[go] = sdb[r];
    }
  }
}

// Calls f with std::integral_constant<int, K> for K in {16, 32, 64, 128}.
template <typename F>
hipError_t with_k(int K, F&& f) {
  switch (K) {
    case 16: return f(std::integral_constant<int, 16>());
    case 32: return f(std::integral_constant<int, 32>());
    case 64: return f(std::integral_constant<int, 64>());
    case 128: return f(std::integral_constant<int, 128>());
  }
  return hipErrorInvalidValue;
}

template <typename TIn>
hipError_t set_lds_limit(const void* fn) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

template <typename TIn>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const int C = a.chunk < kBwdC ? a.chunk : kBwdC;
  const int NT = (a.T + C - 1) / C;
  float* ws_S = a.workspace;
  float* ws_dS = ws_S + (size_t)a.B * a.H * NT * a.V * a.K;
  float* ws_F = ws_dS + (size_t)a.B * a.H * NT * a.V * a.K;
  hipError_t e;

  // (1) chunk-start states
  FwdArgs f;
  f.q = a.q;
  f.k = a.k;
  f.v = a.v;
  f.alpha = a.alpha;
  f.beta = a.beta;
  f.s0 = a.s0;
  f.o = nullptr;
  f.s_final = nullptr;
  f.B = a.B;
  f.T = a.T;
  f.H = a.H;
  f.K = a.K;
  f.V = a.V;
  f.chunk = C;
  float* ws_R = ws_F + (size_t)a.B * a.H * NT * factor_floats(C);  // float32: the records
  bool walked = false;  // float32: (1) and (2b) ran in one launch
  if constexpr (sizeof(TIn) == 4) {
    // float32: the matrix-core forward in its states-only mode, its per-chunk
    // records after the factors in the workspace; its chunk-parallel launch
    // writes the factors (2a) as well.  Where it can, the walk that writes the
    // chunk-start states runs in one launch with the reverse walk (2b), which
    // needs only the records.
    f.s_ckpt = ws_S;
    f.factors = ws_F;
    if (bwd_f32_walks_supported(a.K, a.V, C)) {
      e = launch_fwd_f32_record_only(f, ws_R, stream);
      if (e == hipSuccess) e = launch_bwd_f32_walks(a, C, ws_R, ws_S, ws_dS, stream);
      walked = true;
    } else {
      e = launch_fwd_f32_records(f, ws_R, stream);
    }
  } else {
    e = launch_fwd_states(f, true, ws_S, stream);
  }
  if (e != hipSuccess) return e;

  // (2a) chunk factors (bf16 inputs with K or V = 16; float32 ones have them)
  if constexpr (sizeof(TIn) != 4) {
    const size_t LK = a.K + 1;
    const size_t lds = sizeof(float) * (2 * C * LK + 3 * C * C + 3 * C);
    if ((e = set_lds_limit<TIn>((const void*)bwd_prep_kernel<TIn>)) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_prep_kernel<TIn>, dim3(NT * a.H * a.B), dim3(kThreads), lds, stream,
                       static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k), a.alpha, a.beta,
                       ws_F, a.T, a.H, a.K, C);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // (2b) reverse walk (float32: on the matrix cores, from the recompute's records)
  if constexpr (sizeof(TIn) == 4) {
    if (!walked && (e = launch_bwd_f32_dstate(a, C, ws_R, ws_dS, stream)) != hipSuccess) return e;
  } else {
    const int VS = 16;
    const size_t LK = a.K + 1, LV = VS + 1;
    const size_t lds = sizeof(float) * (2 * C * LK + C * LV + 2 * C * C + 2 * C * LV + VS * LK + 3 * C);
    auto run = [&](auto kc) -> hipError_t {
      constexpr int KK = decltype(kc)::value;
      hipError_t r;
      if ((r = set_lds_limit<TIn>((const void*)bwd_dstate_kernel<TIn, KK>)) != hipSuccess) return r;
      hipLaunchKernelGGL((bwd_dstate_kernel<TIn, KK>), dim3(a.V / VS * a.H * a.B), dim3(kThreads), lds,
                         stream, static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                         static_cast<const TIn*>(a.d_o), a.d_sfinal, a.d_s0, ws_F, ws_dS, a.T, a.H,
                         a.V, C, VS);
      return hipGetLastError();
    };
    if ((e = with_k(a.K, run)) != hipSuccess) return e;
  }
  // (3) token gradients (float32: on the matrix cores)
  if constexpr (sizeof(TIn) == 4) {
    if ((e = launch_bwd_f32_local(a, C, ws_S, ws_dS, ws_F, stream)) != hipSuccess) return e;
  } else {
    const size_t LK = a.K + 1, LV = kBwdVS + 1;
    const size_t lds = sizeof(float) * (2 * C * LK + 5 * C * C + 8 * C * LV + 2 * kBwdVS * LK + 7 * C + kThreads);
    auto run = [&](auto kc) -> hipError_t {
      constexpr int KK = decltype(kc)::value;
      hipError_t r;
      if ((r = set_lds_limit<TIn>((const void*)bwd_local_kernel<TIn, KK>)) != hipSuccess) return r;
      hipLaunchKernelGGL((bwd_local_kernel<TIn, KK>), dim3(NT * a.H * a.B), dim3(kThreads), lds, stream,
                         static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                         static_cast<const TIn*>(a.v), static_cast<const TIn*>(a.d_o), a.alpha,
                         a.beta, ws_S, ws_dS, ws_F, static_cast<TIn*>(a.dq), static_cast<TIn*>(a.dk),
                         static_cast<TIn*>(a.dv), a.dalpha, a.dbeta, a.T, a.H, a.V, C);
      return hipGetLastError();
    };
    if ((e = with_k(a.K, run)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// The layout of the path the call takes: the matrix-core path for bf16 inputs
// with K and V in {32, 64, 128}, the float32 path otherwise.
size_t bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, int64_t chunk,
                           bool bf16) {
  if (bf16 && bwd_bf16_supported((int)K, (int)V)) return bwd_bf16_workspace_bytes(B, T, H, K, V);
  const int64_t C = chunk < kBwdC ? chunk : kBwdC;
  const int64_t NT = (T + C - 1) / C;
  size_t bytes = (size_t)(2 * B * H * NT * V * K + B * H * NT * factor_floats((int)C)) * sizeof(float);
  if (!bf16) {  // float32: the records of the matrix-core state recompute
    FwdArgs f;
    f.B = (int)B;
    f.T = (int)T;
    f.H = (int)H;
    f.chunk = (int)C;
    bytes += fwd_f32_record_bytes(f);
  }
  return bytes;
}

hipError_t launch_bwd(const BwdArgs& a, bool bf16, hipStream_t stream) {
  if (bf16 && bwd_bf16_supported(a.K, a.V)) return launch_bwd_bf16(a, stream);
  return bf16 ? launch_bwd_t<__hip_bfloat16>(a, stream) : launch_bwd_t<float>(a, stream);
}

}  // namespace gdn
