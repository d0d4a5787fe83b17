// Chunkwise gated-delta-rule forward, bfloat16 inputs: warp-specialised MFMA
// kernel for gfx950 (MI355X).
//
// What is computed.  For each (batch, head) stream the state S [V, K] follows
// S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t
// ("Sparse Delta Memory: layer and kernels", section "What the layer computes",
// in its dense limit; shapes and streaming as in "OpenGDN 0.1.0", section "Core
// operator reference").  It is evaluated chunk by chunk with the extended-WY /
// UT decomposition.  For a chunk of n <= C tokens (padded to CP rows with
// alpha = 1, beta = 0, q = k = v = 0, which changes nothing) and chunk-start
// state S:
//
//   gates   g_r  = sum_{i<=r} log2 alpha_i,  gam = 2^g           (wave scan)
//   Gram    A_ri = beta_r 2^(g_r-g_i) k_r.k_i  (i < r)            (MFMA)
//           P_ri =        2^(g_r-g_i) q_r.k_i  (i <= r)
//   solve   Tm = (I + A)^-1: 16x16 diagonal blocks by fp32 substitution,
//           off-diagonal blocks by two levels of block products (MFMA)
//   chain   Y = K S^T, Z = Q S^T                                  (MFMA)
//           U = Tm (diag(beta) Vs - diag(beta gam) Y)
//           O = diag(gam) Z + P U          -> o (bf16)
//           S <- gam_n S + (diag(gam_n/gam) U)^T K                 (MFMA into fp32 S)
//
// Every exponent is g_r - g_i with r >= i (or g_n - g_i) and so never positive.
// Gram products are exact bf16 products summed in fp32; the diagonal solve is
// fp32; every other operand is bf16 with fp32 accumulation.  Each output element
// has one writer and each sum a fixed order: results are bitwise reproducible.
//
// Organisation.  One workgroup of 8 wavefronts owns one (stream, value slice of
// VS rows) pair and walks the chunks in order.  The state-independent work of a
// chunk does not wait for the previous chunk, so it is done ahead by other
// waves while the chain waves run the sequential part:
//
//   chain waves (one per 16 value rows): Y, Z, R of chunk x      | U, O, S of chunk x
//   levels wave:                         off-diagonal Tm of x     |
//   diag wave:                           (the other half of it)   | diagonal Tm of x+1
//   Gram waves:                          A, P of chunk x+1        | stage chunk x+2 in LDS,
//                                                                 | load chunk x+3
//
// Two workgroup barriers per chunk separate the phases.  Rings of LDS slots
// carry each chunk's tiles from stage to use: keys 3 deep (read from staging
// until the state update two iterations later), queries, values, P, Tm 2 deep.
//
// LDS layouts.  An MFMA operand (16 rows x 32 k) is read either from a [row][k]
// array (one 16-byte read per lane) or from a [k][row] array with two gfx950
// transpose reads (ds_read_b64_tr_b16).  Accumulator tiles are written
// transposed ([col][row], 8 bytes per lane).  Key and query tiles are row-major
// [token][channel] with rows padded to a stride of 32 bytes modulo 64.
#include "fwd_bf16_kernel.h"

namespace gdn {
namespace {

template <int KD, int VS, int CP>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int nslice = a.V / VS;
  const int nblk = a.B * a.H * nslice;
  if (a.o)
    hipLaunchKernelGGL((fwd_bf16_kernel<KD, VS, CP, true>), dim3(nblk), dim3(kThreads), 0, stream,
                       static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                       static_cast<const bf16*>(a.v), a.alpha, a.beta, a.s0,
                       static_cast<bf16*>(a.o), a.s_final, a.s_ckpt, nullptr, a.cu_seqlens, a.T, a.H, a.K,
                       a.V, a.chunk, nslice);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<KD, VS, CP, false>), dim3(nblk), dim3(kThreads), 0, stream,
                       static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                       static_cast<const bf16*>(a.v), a.alpha, a.beta, a.s0, nullptr, a.s_final,
                       a.s_ckpt, static_cast<bf16*>(a.s_ckpt_bf16), a.cu_seqlens, a.T, a.H, a.K, a.V,
                       a.chunk, nslice);
  return hipGetLastError();
}

template <int KD, int VS>
hipError_t launch_cp(const FwdArgs& a, hipStream_t stream) {
  return a.chunk <= 32 ? launch<KD, VS, 32>(a, stream) : launch<KD, VS, 64>(a, stream);
}

template <int KD>
hipError_t launch_vs(const FwdArgs& a, int vs, hipStream_t stream) {
  return vs == 16 ? launch_cp<KD, 16>(a, stream) : launch_cp<KD, 32>(a, stream);
}

// Value-slice width: 32 rows (two chain waves) while the (batch, head, slice)
// grid still has at least 192 workgroups, else 16 for more parallelism.  Each
// slice repeats the state-independent work, so wider slices do less of it.
int pick_vs(int B, int H, int V) {
  if (V < 32) return 16;
  return (long)B * H * (V / 32) >= 192 ? 32 : 16;
}

// Segment end states N (workgroups [0, nN): values, zero start, V rows) and segment
// transitions A (the rest: no values, identity starts, K rows) of the
// segment-parallel forward, both states only, in one launch.  64 value rows per
// workgroup share each chunk's Gram and solve between four chain waves, so the two
// passes take about as many workgroups as one pass at 32 rows; the layout has no
// query or P rings (SQ = false), which leaves room for the 64-row value ring.
template <int KD>
__global__ void __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
seg_states_kernel(const bf16* __restrict__ k, const bf16* __restrict__ v,
                  const float* __restrict__ alpha, const float* __restrict__ beta,
                  const float* __restrict__ ident, float* __restrict__ n_final,
                  float* __restrict__ a_final, const int* __restrict__ cu, int T, int H, int V,
                  int nN) {
  __shared__ Smem<KD, 64, 64, false> sm;
  const int bid = blockIdx.x;
  // q is never read by the states-only body (no queries are staged)
  if (bid < nN)
    fwd_bf16_body<KD, 64, 64, false, false>(sm, bid, nN, k, k, v, alpha, beta, nullptr, nullptr,
                                            n_final, nullptr, nullptr, cu, T, H, KD, V, 64, V / 64);
  else
    fwd_bf16_body<KD, 64, 64, false, false>(sm, bid - nN, (int)gridDim.x - nN, k, k, nullptr, alpha,
                                            beta, ident, nullptr, a_final, nullptr, nullptr, cu, T, H,
                                            KD, KD, 64, KD / 64);
}

template <int KD>
hipError_t launch_seg_states(const FwdArgs& a, const float* ident, float* a_final, hipStream_t stream) {
  const int nN = a.B * a.H * (a.V / 64), nA = a.B * a.H * (KD / 64);
  hipLaunchKernelGGL((seg_states_kernel<KD>), dim3(nN + nA), dim3(kThreads), 0, stream,
                     static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v), a.alpha, a.beta,
                     ident, a.s_final, a_final, a.cu_seqlens, a.T, a.H, a.V, nN);
  return hipGetLastError();
}

}  // namespace

bool fwd_bf16_seg_states_supported(int K, int V, int chunk) {
  return (K == 64 || K == 128) && (V == 64 || V == 128) && chunk == 64;
}

hipError_t launch_fwd_bf16_seg_states(const FwdArgs& a, const float* ident, float* a_final,
                                      hipStream_t stream) {
  if (!fwd_bf16_seg_states_supported(a.K, a.V, a.chunk) || !a.cu_seqlens || !a.v || a.s0)
    return hipErrorInvalidValue;
  return a.K == 64 ? launch_seg_states<64>(a, ident, a_final, stream)
                   : launch_seg_states<128>(a, ident, a_final, stream);
}

int fwd_bf16_value_slice(int B, int H, int V) { return pick_vs(B, H, V); }

bool fwd_bf16_supported(int K, int V, int chunk) {
  return (K == 16 || K == 32 || K == 64 || K == 128) && (V == 16 || V == 32 || V == 64 || V == 128) &&
         (chunk == 16 || chunk == 32 || chunk == 64);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (!fwd_bf16_supported(a.K, a.V, a.chunk)) return hipErrorInvalidValue;
  const int vs = (a.vs == 16 || a.vs == 32) && a.vs <= a.V ? a.vs : pick_vs(a.B, a.H, a.V);
  if (a.K <= 32) return launch_vs<32>(a, vs, stream);
  if (a.K == 64) return launch_vs<64>(a, vs, stream);
  return launch_vs<128>(a, vs, stream);
}

}  // namespace gdn
