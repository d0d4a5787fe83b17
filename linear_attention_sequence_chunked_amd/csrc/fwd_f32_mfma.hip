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

#include "f32_chain.h"
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
// Launch 2: the walk over chunks (f32_chain.h), one workgroup per (sequence,
// head, 16 NG value rows).
template <int KD, int C, int NG, bool WO, bool HV, bool CK>
__global__ void __launch_bounds__(64 * NG * (C / 16), 1)
f32_chain_kernel(const float* __restrict__ q, const float* __restrict__ k,
                 const float* __restrict__ v, const float* __restrict__ s0, float* __restrict__ o,
                 float* __restrict__ s_final, float* __restrict__ s_ckpt,
                 const float* __restrict__ rec, const int* __restrict__ cu, int B, int T, int H,
                 int V, int NT) {
  __shared__ ChainLds<KD, C, NG, WO> lds;
  chain_walk<KD, C, NG, WO, HV, CK>(lds, blockIdx.x, q, k, v, s0, o, s_final, s_ckpt, rec, cu, B,
                                    T, H, V, NT);
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
hipError_t launch_record(const FwdArgs& a, float* rec, hipStream_t stream) {
  const int NT = (a.T + C - 1) / C;
  const long slots = a.cu_seqlens ? (long)(a.T / C) + a.B + 1 : (long)a.B * NT;
  hipLaunchKernelGGL((f32_record_kernel<KD, C>), dim3(slots * a.H), dim3(256), 0, stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k), a.alpha,
                     a.beta, rec, a.cu_seqlens ? nullptr : a.factors, a.cu_seqlens, a.B, a.T, a.H, NT);
  return hipGetLastError();
}

template <int KD, int C>
hipError_t launch_kc(const FwdArgs& a, float* rec, hipStream_t stream) {
  const int NT = (a.T + C - 1) / C;
  hipError_t e = launch_record<KD, C>(a, rec, stream);
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

hipError_t launch_fwd_f32_record_only(const FwdArgs& a, float* rec, hipStream_t stream) {
  if (!fwd_f32_mfma_supported(a.K, a.V, a.chunk) || !rec) return hipErrorInvalidValue;
  auto by_c = [&](auto kc) -> hipError_t {
    constexpr int KD = decltype(kc)::value;
    if (a.chunk == 16) return launch_record<KD, 16>(a, rec, stream);
    if (a.chunk == 32) return launch_record<KD, 32>(a, rec, stream);
    return launch_record<KD, 64>(a, rec, stream);
  };
  if (a.K == 16) return by_c(std::integral_constant<int, 16>());
  if (a.K == 32) return by_c(std::integral_constant<int, 32>());
  if (a.K == 64) return by_c(std::integral_constant<int, 64>());
  return by_c(std::integral_constant<int, 128>());
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
