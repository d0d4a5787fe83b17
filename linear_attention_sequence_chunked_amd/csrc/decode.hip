// Single-token decode step of the gated delta rule:
//
//   S <- alpha S (I - beta k k^T) + beta v k^T,   o = S q
//
// for every (batch, head), with the state S [V, K] updated in place.  This is
// the token step of "Sparse Delta Memory: layer and kernels", section "What the
// layer computes" (decay, read with k, write beta times the error, read with q
// from the updated state), run one token at a time as its decode path does
// (section "Execution"); shapes follow "OpenGDN 0.1.0", section "Core operator
// reference", with T = 1.
//
// Per state row s (one value channel): e = s.k, s <- alpha (s - beta e k) +
// beta v_r k, o_r = s.q -- two row dot products, everything else elementwise.
// The step reads and writes the fp32 state once (2 * V * K * 4 bytes per
// head), so it is bound by HBM bandwidth.  Layout: K / 4 lanes own one row (four
// consecutive channels each, 16-byte accesses; at K = 128 a wavefront holds two
// rows); row dot products reduce over the row's lanes with cross-lane adds in a
// fixed order.
#include "launch.h"

#include <hip/hip_bf16.h>

namespace gdn {
namespace {

constexpr int kThreads = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__hip_bfloat16 x) { return __bfloat162float(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __hip_bfloat16 from_f32<__hip_bfloat16>(float x) {
  return __float2bfloat16(x);
}

// Sum over the LPR lanes that hold one row (butterfly in a fixed order; every
// lane of the row ends with the same total).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, LPR);
  return x;
}

// One workgroup per (batch, head, group of rows_per_block(K) rows); K / 4 lanes
// per row, so every one of the 256 threads owns one 16-byte piece of a row
// (8 rows at K = 128, 64 at K = 16).
constexpr int rows_per_block(int K) { return kThreads / (K / 4); }

template <typename TIn, int K>
__global__ void __launch_bounds__(kThreads)
decode_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
              const float* __restrict__ alpha, const float* __restrict__ beta,
              float* __restrict__ state, TIn* __restrict__ o, int H, int V) {
  constexpr int LPR = K / 4;                      // lanes per row
  constexpr int RPI = kThreads / LPR;             // rows per pass of the block
  constexpr int kRowsPerBlock = rows_per_block(K);
  constexpr int NR = (kRowsPerBlock + RPI - 1) / RPI;  // rows per lane
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;                      // b * H + h
  const int r0 = blockIdx.y * kRowsPerBlock + tid / LPR;
  const int c4 = (tid % LPR) * 4;                 // first channel of this lane
  const float a = alpha[bh], bt = beta[bh];
  float kk[4], qq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kk[j] = to_f32(k[(size_t)bh * K + c4 + j]);
    qq[j] = to_f32(q[(size_t)bh * K + c4 + j]);
  }
  f32x4 s4[NR];
  float vr[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = r0 + i * RPI;
    const bool ok = r < V && r < (int)(blockIdx.y + 1) * kRowsPerBlock;
    // the state streams through once: non-temporal accesses keep it out of the caches
    s4[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(state + ((size_t)bh * V + r) * K + c4))
               : f32x4{0.f, 0.f, 0.f, 0.f};
    vr[i] = ok ? to_f32(v[(size_t)bh * V + r]) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = r0 + i * RPI;
    const bool ok = r < V && r < (int)(blockIdx.y + 1) * kRowsPerBlock;
    float s[4] = {s4[i][0], s4[i][1], s4[i][2], s4[i][3]};
    float e = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) e = fmaf(s[j], kk[j], e);
    e = row_sum<LPR>(e);
    const float w = bt * (vr[i] - a * e);         // beta (v - alpha S k): the corrected write
    float ov = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[j] = fmaf(w, kk[j], a * s[j]);            // alpha S + beta (v - alpha S k) k^T
      ov = fmaf(s[j], qq[j], ov);
    }
    ov = row_sum<LPR>(ov);
    if (ok) {
      __builtin_nontemporal_store(f32x4{s[0], s[1], s[2], s[3]},
                                  reinterpret_cast<f32x4*>(state + ((size_t)bh * V + r) * K + c4));
      if (tid % LPR == 0) o[(size_t)bh * V + r] = from_f32<TIn>(ov);
    }
  }
}

template <typename TIn, int K>
hipError_t launch_k(const DecodeArgs& a, hipStream_t stream) {
  constexpr int RPB = rows_per_block(K);
  dim3 grid(a.B * a.H, (a.V + RPB - 1) / RPB);
  hipLaunchKernelGGL((decode_kernel<TIn, K>), grid, dim3(kThreads), 0, stream,
                     static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                     static_cast<const TIn*>(a.v), a.alpha, a.beta, a.state,
                     static_cast<TIn*>(a.o), a.H, a.V);
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  switch (a.K) {
    case 16: return launch_k<TIn, 16>(a, stream);
    case 32: return launch_k<TIn, 32>(a, stream);
    case 64: return launch_k<TIn, 64>(a, stream);
    case 128: return launch_k<TIn, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  return bf16 ? launch_t<__hip_bfloat16>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace gdn
