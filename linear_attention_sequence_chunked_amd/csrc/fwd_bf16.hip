// Chunkwise gated-delta-rule forward, bfloat16 inputs: MFMA kernel for gfx950.
//
// One workgroup (4 wavefronts) owns one (batch, head, value-slice) stream: rows
// [v0, v0 + VS) of the [V, K] state.  The fp32 state lives in MFMA accumulator
// registers for the whole sequence; the chunks are walked in order.  Per chunk of
// n <= C tokens, padded to a CP-token tile (padding tokens carry alpha = 1,
// beta = 0, q = k = v = 0, which leaves every product and the state unchanged),
// the steps of the extended-WY / UT decomposition are ("Sparse Delta Memory:
// layer and kernels", section "What the layer computes"; "OpenGDN 0.1.0",
// section "Core operator reference"):
//
//   gates   g_r = sum_{i<=r} log2 alpha_i  (wavefront scan), gam = 2^g
//   Gram    A_ri = beta_r 2^(g_r-g_i) k_r.k_i  (i < r),  P_ri = 2^(g_r-g_i) q_r.k_i  (i <= r)
//   solve   Tm = (I + A)^-1: 16x16 diagonal blocks by fp32 substitution, the
//           off-diagonal blocks by two levels of block products on MFMA
//   chain   Y = K S^T, Z = Q S^T           (one bf16 MFMA pass over the state)
//           U = Tm (diag(beta) Vs - diag(beta gam) Y)
//           O = diag(gam) Z + P U           (stored as bf16)
//           S <- gam_n S + (diag(gam_n/gam) U)^T K   (MFMA into the fp32 state)
//
// Every exponent is g_r - g_i with r >= i, or g_n - g_i: never positive.  The
// Gram matrices accumulate exact bf16 products in fp32; the solve's diagonal
// blocks are fp32; all other MFMA operands are bf16 with fp32 accumulation.
// Every output element has one writer and every sum a fixed order, so the result
// is bitwise reproducible.
//
// LDS layouts.  An MFMA operand fragment (16 rows x 32 k) is read either from a
// row-major [row][k] array with one 16-byte read per lane, or from a [k][row]
// array with two gfx950 transpose reads (ds_read_b64_tr_b16).  Accumulator tiles
// are always written transposed ([col][row], 8 bytes per lane).
#include "launch.h"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef bf16x4 __attribute__((address_space(3))) lds_bf16x4;

constexpr int kThreads = 256;
constexpr int kWaves = 4;

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Fragment of rows r0..r0+15, k0..k0+31 from a row-major [row][k] array:
// lane (g = l/16, s = l%16) receives row r0 + s, k = k0 + 8g .. k0 + 8g + 7.
__device__ __forceinline__ bf16x8 frag_rows(const bf16* base, int ld, int r0, int k0, int lane) {
  return *reinterpret_cast<const bf16x8*>(base + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

// Same fragment from a [k][row] array by transpose reads: within each 16-lane
// group the hardware hands lane 4a+c the c-th 16-bit element of the lanes a,
// a+4, a+8, a+12.  Source lane s therefore points at row k0 + 8g + s/4 and
// column r0 + 4(s%4); the second read covers k + 4.
__device__ __forceinline__ bf16x8 frag_cols(const bf16* base, int ld, int r0, int k0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const bf16* p = base + (k0 + 8 * g + (s >> 2)) * ld + r0 + 4 * (s & 3);
  bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * ld));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Accumulator tile (lane holds rows 4g..4g+3 of column s) written transposed:
// dst[c0 + s][r0 + 4g .. r0 + 4g + 3].
__device__ __forceinline__ void store_tile_t(bf16* base, int ld, int c0, int r0, f32x4 d, int lane) {
  const int s = lane & 15, g = lane >> 4;
  *reinterpret_cast<bf16x4*>(base + (c0 + s) * ld + r0 + 4 * g) =
      bf16x4{(bf16)d[0], (bf16)d[1], (bf16)d[2], (bf16)d[3]};
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
  for (int j = 0; j < 8; ++j) z[j] = (bf16)0.0f;
  return z;
}

// 16-deep variants for products over one 16-wide block: the lanes that would hold
// k in [16, 32) read the same (valid) rows as their k in [0, 16) partners and are
// then zeroed, so the 32-deep MFMA adds exact zeros.
__device__ __forceinline__ bf16x8 frag_rows16(const bf16* base, int ld, int r0, int k0, int lane) {
  const bf16x8 f = frag_rows(base, ld, r0, k0 - 16 * ((lane >> 5) & 1), lane);
  return (lane >> 5) ? zero8() : f;
}
__device__ __forceinline__ bf16x8 frag_cols16(const bf16* base, int ld, int r0, int k0, int lane) {
  const bf16x8 f = frag_cols(base, ld, r0, k0 - 16 * ((lane >> 5) & 1), lane);
  return (lane >> 5) ? zero8() : f;
}

template <int KD, int VS, int CP>
struct alignas(16) Smem {
  static constexpr int LDK = KD + 8;   // q, k tiles [CP][LDK]
  static constexpr int LDC = CP + 8;   // CP-wide square tiles [CP][LDC]
  static constexpr int LDV = VS + 8;   // state [KD][LDV]
  bf16 k[CP * LDK];
  bf16 q[CP * LDK];
  bf16 v[CP * VS];
  bf16 st[KD * LDV];                   // state^T in bf16: st[c][v]
  bf16 at[CP * LDC];                   // A^T: at[i][r]
  bf16 pt[CP * LDC];                   // P^T: pt[i][r]
  bf16 tt[CP * LDC];                   // Tm^T: tt[j][i]
  bf16 xt[CP * LDC];                   // block-product scratch (transposed)
  bf16 rt[VS * LDC];                   // R^T: rt[v][j]
  bf16 ut[VS * LDC];                   // U^T
  bf16 upt[VS * LDC];                  // (diag(gam_n/gam) U)^T
  float ad[(CP / 16) * 256];           // fp32 diagonal 16x16 blocks of A, row-major
  float g[CP];                         // cumulative log2 gate
  float gam[CP];                       // 2^g
  float beta[CP];
  float bg[CP];                        // beta * gam
  float dn[CP];                        // gam_n / gam
};

template <int KD, int VS, int CP>
__global__ void __launch_bounds__(kThreads, 1)
fwd_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                const float* __restrict__ alpha, const float* __restrict__ beta,
                const float* __restrict__ s0, bf16* __restrict__ o, float* __restrict__ s_final,
                int T, int H, int K, int V, int C) {
  using SM = Smem<KD, VS, CP>;
  constexpr int LDK = SM::LDK, LDC = SM::LDC, LDV = SM::LDV;
  constexpr int NTB = CP / 16;    // token blocks
  constexpr int NVB = VS / 16;    // value blocks
  constexpr int NCB = KD / 16;    // key-channel blocks
  constexpr int NST = NVB * NCB;  // state tiles
  constexpr int ST_PER_WAVE = (NST + kWaves - 1) / kWaves;
  __shared__ SM sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ls = lane & 15, lg = lane >> 4;
  const int v0 = blockIdx.x * VS;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const size_t tok_stride_k = (size_t)H * K;   // elements between tokens in q, k
  const size_t tok_stride_v = (size_t)H * V;
  const size_t state_base = ((size_t)b * H + h) * (size_t)V * K + (size_t)v0 * K;

  // ---- the upper (never written) blocks of A^T, P^T, Tm^T must read as zeros
  for (int i = tid; i < CP * LDC; i += kThreads) {
    sm.tt[i] = (bf16)0.0f;
    sm.pt[i] = (bf16)0.0f;
    sm.at[i] = (bf16)0.0f;
    sm.xt[i] = (bf16)0.0f;
  }

  // ---- initial state into accumulators (tile t = wave + 4j: vb = t / NCB, cb = t % NCB)
  f32x4 S[ST_PER_WAVE];
#pragma unroll
  for (int j = 0; j < ST_PER_WAVE; ++j) {
    const int t = wave + kWaves * j;
    S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t < NST && s0) {
      const int vb = t / NCB, cb = t % NCB;
      const int c = 16 * cb + ls;
      if (c < K)
        for (int e = 0; e < 4; ++e) S[j][e] = s0[state_base + (size_t)(16 * vb + 4 * lg + e) * K + c];
    }
  }

  // ---- register prefetch of one chunk: q, k rows (8 bf16 per slot), v slice, gates
  constexpr int KCH = KD / 8;                       // 16-byte pieces per q/k row
  constexpr int QK_SLOTS = (CP * KCH + kThreads - 1) / kThreads;
  constexpr int VCH = VS / 8;
  constexpr int V_SLOTS = (CP * VCH + kThreads - 1) / kThreads;
  bf16x8 pq[QK_SLOTS], pk[QK_SLOTS], pv[V_SLOTS];
  float pa = 1.0f, pb = 0.0f;

  auto prefetch = [&](int t0) {
    const int n = min(C, T - t0);
#pragma unroll
    for (int j = 0; j < QK_SLOTS; ++j) {
      const int idx = tid + kThreads * j;
      const int r = idx / KCH, c = (idx % KCH) * 8;
      pq[j] = zero8();
      pk[j] = zero8();
      if (r < n && c < K) {
        const size_t off = ((size_t)b * T + t0 + r) * tok_stride_k + (size_t)h * K + c;
        pq[j] = *reinterpret_cast<const bf16x8*>(q + off);
        pk[j] = *reinterpret_cast<const bf16x8*>(k + off);
      }
    }
#pragma unroll
    for (int j = 0; j < V_SLOTS; ++j) {
      const int idx = tid + kThreads * j;
      const int r = idx / VCH, c = (idx % VCH) * 8;
      pv[j] = zero8();
      if (r < n)
        pv[j] = *reinterpret_cast<const bf16x8*>(
            v + ((size_t)b * T + t0 + r) * tok_stride_v + (size_t)h * V + v0 + c);
    }
    pa = 1.0f;
    pb = 0.0f;
    if (tid < n) {
      const size_t go = ((size_t)b * T + t0 + tid) * H + h;
      pa = alpha[go];
      pb = beta[go];
    }
  };

  prefetch(0);

  for (int t0 = 0; t0 < T; t0 += C) {
    const int n = min(C, T - t0);
    __syncthreads();  // every wave is done with the previous chunk's tiles
    // ---- stage the prefetched chunk in LDS
#pragma unroll
    for (int j = 0; j < QK_SLOTS; ++j) {
      const int idx = tid + kThreads * j;
      const int r = idx / KCH, c = (idx % KCH) * 8;
      if (r < CP) {
        *reinterpret_cast<bf16x8*>(&sm.q[r * LDK + c]) = pq[j];
        *reinterpret_cast<bf16x8*>(&sm.k[r * LDK + c]) = pk[j];
      }
    }
#pragma unroll
    for (int j = 0; j < V_SLOTS; ++j) {
      const int idx = tid + kThreads * j;
      const int r = idx / VCH, c = (idx % VCH) * 8;
      if (r < CP) *reinterpret_cast<bf16x8*>(&sm.v[r * VS + c]) = pv[j];
    }
    const float my_a = pa, my_b = pb;
    // state (bf16, transposed) for this chunk's Y = K S^T, Z = Q S^T
#pragma unroll
    for (int j = 0; j < ST_PER_WAVE; ++j) {
      const int t = wave + kWaves * j;
      if (t < NST) store_tile_t(sm.st, LDV, 16 * (t % NCB), 16 * (t / NCB), S[j], lane);
    }
    __syncthreads();
    if (t0 + C < T) prefetch(t0 + C);  // overlaps with the compute below

    // ---- gates (wave 0): inclusive scan of log2 alpha over the tile
    if (wave == 0) {
      float la = (lane < CP) ? log2f(my_a) : 0.0f;
      float bt = (lane < CP) ? my_b : 0.0f;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        float y = __shfl_up(la, d, 64);
        if (lane >= d) la += y;
      }
      const float glast = __shfl(la, CP - 1, 64);
      if (lane < CP) {
        const float gm = exp2f(la);
        sm.g[lane] = la;
        sm.gam[lane] = gm;
        sm.beta[lane] = bt;
        sm.bg[lane] = bt * gm;
        sm.dn[lane] = exp2f(glast - la);
      }
    }
    // ---- Y = K S^T and Z = Q S^T for token block tb = wave (all value blocks)
    f32x4 Y[NVB], Z[NVB];
    const int tb = wave;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      Y[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
      Z[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (tb < NTB) {
#pragma unroll
      for (int ks = 0; ks < KD / 32; ++ks) {
        const bf16x8 ka = frag_rows(sm.k, LDK, 16 * tb, 32 * ks, lane);
        const bf16x8 qa = frag_rows(sm.q, LDK, 16 * tb, 32 * ks, lane);
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
          const bf16x8 sb = frag_cols(sm.st, LDV, 16 * vb, 32 * ks, lane);
          Y[vb] = mma(ka, sb, Y[vb]);
          Z[vb] = mma(qa, sb, Z[vb]);
        }
      }
    }
    __syncthreads();  // gates visible

    // ---- Gram tiles: A (strictly lower) and P (lower), tile list round-robin over waves
    constexpr int NTRI = NTB * (NTB + 1) / 2;
    for (int t = wave; t < 2 * NTRI; t += kWaves) {
      const bool isP = t >= NTRI;
      int u = isP ? t - NTRI : t;
      int tr = 0;
      while (u > tr) { u -= tr + 1; ++tr; }
      const int tc = u;  // tc <= tr
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KD / 32; ++ks) {
        const bf16x8 a = frag_rows(isP ? sm.q : sm.k, LDK, 16 * tr, 32 * ks, lane);
        const bf16x8 bb = frag_rows(sm.k, LDK, 16 * tc, 32 * ks, lane);
        acc = mma(a, bb, acc);
      }
      const int i = 16 * tc + ls;
      const float gi = sm.g[i];
      f32x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * tr + 4 * lg + e;
        const bool keep = isP ? (i <= r) : (i < r);
        const float dec = keep ? exp2f(sm.g[r] - gi) : 0.0f;
        val[e] = isP ? dec * acc[e] : sm.beta[r] * dec * acc[e];
      }
      if (isP) {
        store_tile_t(sm.pt, LDC, 16 * tc, 16 * tr, val, lane);
      } else {
        store_tile_t(sm.at, LDC, 16 * tc, 16 * tr, val, lane);
        if (tr == tc) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sm.ad[tr * 256 + (4 * lg + e) * 16 + ls] = val[e];
        }
      }
    }
    // ---- R = diag(beta) V - diag(beta gam) Y  ->  R^T (bf16); Z scaled by gam
    if (tb < NTB) {
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f32x4 rr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tb + 4 * lg + e;
          const float vv = (float)sm.v[r * VS + 16 * vb + ls];
          rr[e] = sm.beta[r] * vv - sm.bg[r] * Y[vb][e];
          Z[vb][e] *= sm.gam[r];
        }
        store_tile_t(sm.rt, LDC, 16 * vb, 16 * tb, rr, lane);
      }
    }
    __syncthreads();

    // ---- diagonal blocks of Tm by forward substitution in fp32 (wave 0):
    // lane (block bb = lane/16, column j = lane%16) builds column j of (I + L_bb)^-1.
    if (wave == 0 && lg < NTB) {
      const int bb = lg, j = ls;
      const float* L = &sm.ad[bb * 256];
      float x[16], acc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // x_r = delta_rj - sum_{i<r} L[r][i] x_i ; acc[r] holds the running sum
        x[r] = (r == j) ? 1.0f : ((r < j) ? 0.0f : -acc[r]);
#pragma unroll
        for (int rr = r + 1; rr < 16; ++rr) acc[rr] = fmaf(L[rr * 16 + r], x[r], acc[rr]);
      }
      bf16x8 lo, hi;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        lo[r] = (bf16)x[r];
        hi[r] = (bf16)x[8 + r];
      }
      bf16* dst = &sm.tt[(16 * bb + j) * LDC + 16 * bb];
      *reinterpret_cast<bf16x8*>(dst) = lo;
      *reinterpret_cast<bf16x8*>(dst + 8) = hi;
    }
    __syncthreads();

    // ---- level 1: Tm_ij = -Tm_ii (A_ij Tm_jj) for (i, j) = (1, 0) [and (3, 2)]
    if (wave < NTB / 2) {
      const int bi = 2 * wave + 1, bj = 2 * wave;
      // X = A_ij Tm_jj  (k = the 16 columns of block j)
      const bf16x8 a = frag_cols16(sm.at, LDC, 16 * bi, 16 * bj, lane);
      const bf16x8 bb = frag_rows16(sm.tt, LDC, 16 * bj, 16 * bj, lane);
      f32x4 X = mma(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
      store_tile_t(sm.xt, LDC, 16 * bj, 16 * bi, X, lane);  // xt[col][row]
      __builtin_amdgcn_s_waitcnt(0xc07f);                   // lgkmcnt(0): same-wave LDS order
      // Tm_ij = -Tm_ii X   (k = the 16 rows of block i)
      const bf16x8 t2 = frag_cols16(sm.tt, LDC, 16 * bi, 16 * bi, lane);
      const bf16x8 x2 = frag_rows16(sm.xt, LDC, 16 * bj, 16 * bi, lane);
      f32x4 Tij = mma(t2, x2, f32x4{0.f, 0.f, 0.f, 0.f});
      store_tile_t(sm.tt, LDC, 16 * bj, 16 * bi, -Tij, lane);
    }
    if constexpr (NTB == 4) {
      __syncthreads();
      // ---- level 2a: X2 = A_[23][01] Tm_[01]  (tile (2 + wave/2, wave%2), k = 32)
      {
        const int bi = 2 + wave / 2, bj = wave % 2;
        bf16x8 a = frag_cols(sm.at, LDC, 16 * bi, 0, lane);
        bf16x8 bb = frag_rows(sm.tt, LDC, 16 * bj, 0, lane);
        f32x4 X = mma(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
        store_tile_t(sm.xt, LDC, 16 * bj, 16 * bi, X, lane);
      }
      __syncthreads();
      // ---- level 2b: Tm_[23][01] = -Tm_[23] X2
      {
        const int bi = 2 + wave / 2, bj = wave % 2;
        bf16x8 a = frag_cols(sm.tt, LDC, 16 * bi, 32, lane);
        bf16x8 bb = frag_rows(sm.xt, LDC, 16 * bj, 32, lane);
        f32x4 Tij = mma(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
        store_tile_t(sm.tt, LDC, 16 * bj, 16 * bi, -Tij, lane);
      }
    }
    __syncthreads();

    // ---- U = Tm R for token block tb (value blocks vb); write U^T and (dn U)^T
    if (tb < NTB) {
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f32x4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < CP / 32; ++ks) {
          if (32 * ks > 16 * tb + 15) break;  // Tm is lower triangular
          const bf16x8 a = frag_cols(sm.tt, LDC, 16 * tb, 32 * ks, lane);
          const bf16x8 bb = frag_rows(sm.rt, LDC, 16 * vb, 32 * ks, lane);
          U = mma(a, bb, U);
        }
        store_tile_t(sm.ut, LDC, 16 * vb, 16 * tb, U, lane);
        f32x4 Up;
#pragma unroll
        for (int e = 0; e < 4; ++e) Up[e] = sm.dn[16 * tb + 4 * lg + e] * U[e];
        store_tile_t(sm.upt, LDC, 16 * vb, 16 * tb, Up, lane);
      }
    }
    __syncthreads();

    // ---- O = diag(gam) Z + P U for token block tb, stored as bf16
    if (tb < NTB) {
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f32x4 O = Z[vb];
#pragma unroll
        for (int ks = 0; ks < CP / 32; ++ks) {
          if (32 * ks > 16 * tb + 15) break;  // P is lower triangular
          const bf16x8 a = frag_cols(sm.pt, LDC, 16 * tb, 32 * ks, lane);
          const bf16x8 bb = frag_rows(sm.ut, LDC, 16 * vb, 32 * ks, lane);
          O = mma(a, bb, O);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tb + 4 * lg + e;
          if (r < n)
            o[((size_t)b * T + t0 + r) * tok_stride_v + (size_t)h * V + v0 + 16 * vb + ls] = (bf16)O[e];
        }
      }
    }
    // ---- state: S <- gam_n S + Up^T K
    {
      const float gam_n = sm.gam[CP - 1];
#pragma unroll
      for (int j = 0; j < ST_PER_WAVE; ++j) {
        const int t = wave + kWaves * j;
        if (t < NST) {
          const int vb = t / NCB, cb = t % NCB;
          f32x4 acc = S[j] * gam_n;
#pragma unroll
          for (int ks = 0; ks < CP / 32; ++ks) {
            const bf16x8 a = frag_rows(sm.upt, LDC, 16 * vb, 32 * ks, lane);
            const bf16x8 bb = frag_cols(sm.k, LDK, 16 * cb, 32 * ks, lane);
            acc = mma(a, bb, acc);
          }
          S[j] = acc;
        }
      }
    }
  }

  // ---- final state
  if (s_final) {
#pragma unroll
    for (int j = 0; j < ST_PER_WAVE; ++j) {
      const int t = wave + kWaves * j;
      if (t < NST) {
        const int vb = t / NCB, cb = t % NCB;
        const int c = 16 * cb + ls;
        if (c < K)
          for (int e = 0; e < 4; ++e)
            s_final[state_base + (size_t)(16 * vb + 4 * lg + e) * K + c] = S[j][e];
      }
    }
  }
}

template <int KD, int VS, int CP>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  dim3 grid(a.V / VS, a.H, a.B);
  hipLaunchKernelGGL((fwd_bf16_kernel<KD, VS, CP>), grid, dim3(kThreads), 0, stream,
                     static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                     static_cast<const bf16*>(a.v), a.alpha, a.beta, a.s0,
                     static_cast<bf16*>(a.o), a.s_final, a.T, a.H, a.K, a.V, a.chunk);
  return hipGetLastError();
}

template <int KD, int VS>
hipError_t launch_cp(const FwdArgs& a, hipStream_t stream) {
  return a.chunk <= 32 ? launch<KD, VS, 32>(a, stream) : launch<KD, VS, 64>(a, stream);
}

template <int KD>
hipError_t launch_vs(const FwdArgs& a, int vs, hipStream_t stream) {
  switch (vs) {
    case 16: return launch_cp<KD, 16>(a, stream);
    case 32: return launch_cp<KD, 32>(a, stream);
    default: return launch_cp<KD, 64>(a, stream);
  }
}

// Value-slice width: as wide as possible while the (batch, head, slice) grid
// still covers the 256 compute units; each slice repeats the K-side work
// (gates, Gram, solve), so wider slices mean less repeated work.
int pick_vs(int B, int H, int V) {
  int vs = V < 64 ? V : 64;
  while (vs > 16 && (long)B * H * (V / vs) < 192) vs /= 2;
  return vs;
}

}  // namespace

bool fwd_bf16_supported(int K, int V, int chunk) {
  return (K == 16 || K == 32 || K == 64 || K == 128) && (V == 16 || V == 32 || V == 64 || V == 128) &&
         (chunk == 16 || chunk == 32 || chunk == 64);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (!fwd_bf16_supported(a.K, a.V, a.chunk)) return hipErrorInvalidValue;
  const int vs = pick_vs(a.B, a.H, a.V);
  if (a.K <= 32) return launch_vs<32>(a, vs, stream);
  if (a.K == 64) return launch_vs<64>(a, vs, stream);
  return launch_vs<128>(a, vs, stream);
}

}  // namespace gdn
