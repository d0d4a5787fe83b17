// Segment-parallel forward for long sequences with few streams.
//
// The token step S <- alpha S (I - beta k k^T) + beta v k^T is affine in the
// state, so a run of tokens maps its start state S to S A + N, with A the
// ordered product of alpha_t (I - beta_t k_t k_t^T) (K x K) and N the end state
// of the same run from a zero start.  Splitting every sequence into P segments:
//
//   1. all segments in parallel: N_s (values v, zero start) and A_s (no values,
//      identity start, K rows) with the chunk kernel in packed-sequence mode;
//   2. per stream, in segment order: start_0 = S0, start_{s+1} = start_s A_s + N_s;
//   3. all segments in parallel again from their true starts, writing o, and the
//      last segment's end state as the final state.
//
// This is the state passing of "Sparse Delta Memory: layer and kernels"
// (section "What the layer computes": the chunk recurrence carries the state
// from chunk to chunk) applied between segments, with the operator contract of
// "OpenGDN 0.1.0", section "Core operator reference".  It costs about two extra
// forward passes (A_s has K rows), so it pays only when the streams alone leave
// most of the GPU idle.
#include "launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

// Segment table over the flattened [B*T] token axis (segment j = b*P + s holds
// tokens b*T + s*L .. min(b*T + (s+1)*L, (b+1)*T)) and identity start states
// for the A pass ([B*P, H, K, K]).
__global__ void __launch_bounds__(kThreads)
seg_init_kernel(int* __restrict__ cu, float* __restrict__ ident, int B, int T, int H, int K, int P,
                int L) {
  const size_t tid = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const int nseg = B * P;
  for (size_t j = tid; j <= (size_t)nseg; j += (size_t)gridDim.x * kThreads) {
    const int b = (int)j / P, s = (int)j - b * P;
    cu[j] = (int)j == nseg ? B * T : b * T + min(s * L, T);
  }
  const size_t total = (size_t)nseg * H * K * K;
  for (size_t i = tid; i < total; i += (size_t)gridDim.x * kThreads) {
    const int c = (int)(i % K), r = (int)((i / K) % K);
    ident[i] = r == c ? 1.0f : 0.0f;
  }
}

// start_0 = S0 (or 0); start_{s+1} = start_s A_s + N_s.  One workgroup of two
// wavefronts per (stream, head, 8 state rows).  The rows of start stay in LDS;
// A_s arrives in one of two LDS buffers by direct global-to-LDS loads issued a
// step ahead, so the next transition streams in while this one is applied.
constexpr int kCombThreads = 128;
constexpr int kCombRows = 8;

__device__ __forceinline__ void fetch_transition(const float* A, float* dst, int K) {
  // each wave instruction moves 64 lanes x 16 bytes = 1 KB to dst + 256 u floats
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int u = w; u < K * K / 256; u += kCombThreads / 64)
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(A + 256 * u + 4 * lane),
        (__attribute__((address_space(3))) void*)(dst + 256 * u), 16, 0, 0);
}

__global__ void __launch_bounds__(kCombThreads)
seg_combine_kernel(const float* __restrict__ s0, const float* __restrict__ Aseg,
                   const float* __restrict__ Nseg, float* __restrict__ start, int H, int K, int V,
                   int P) {
  constexpr int R = kCombRows;
  extern __shared__ float lds[];
  const int LK = K + 1;
  float* cur = lds;                // [R][LK]
  float* nxt = cur + R * LK;       // [R][LK]
  float* Ab = nxt + R * LK;        // [2][K][K]
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * R, h = blockIdx.y, b = blockIdx.z;
  const size_t seg0 = (size_t)b * P * H + h;  // segment s of this stream: seg0 + s * H
  if (P > 1) fetch_transition(Aseg + seg0 * K * K, Ab, K);
  for (int i = tid; i < R * K; i += kCombThreads) {
    const int r = i / K, c = i - r * K;
    cur[r * LK + c] = s0 ? s0[(((size_t)b * H + h) * V + r0 + r) * K + c] : 0.0f;
  }
  // thread: rows r and r + R/2, columns c .. c + 3
  const int r = tid / 32, c = (tid % 32) * 4;
  for (int s = 0; s < P; ++s) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): A_s is in LDS
    __syncthreads();
    const size_t seg = seg0 + (size_t)s * H;
    for (int i = tid; i < R * K; i += kCombThreads) {
      const int rr = i / K, cc = i - rr * K;
      start[(seg * V + r0 + rr) * K + cc] = cur[rr * LK + cc];
    }
    if (s + 1 == P) break;
    if (s + 2 < P) fetch_transition(Aseg + (seg + H) * K * K, Ab + ((s + 1) & 1) * K * K, K);
    const float* As = Ab + (s & 1) * K * K;
    if (c < K) {
      const float* N = Nseg + seg * V * K;
      float a0[4], a1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a0[e] = N[(size_t)(r0 + r) * K + c + e];
        a1[e] = N[(size_t)(r0 + r + R / 2) * K + c + e];
      }
      for (int j = 0; j < K; ++j) {
        const float4 arow = *reinterpret_cast<const float4*>(&As[j * K + c]);
        const float x0 = cur[r * LK + j], x1 = cur[(r + R / 2) * LK + j];
        a0[0] = fmaf(x0, arow.x, a0[0]);
        a0[1] = fmaf(x0, arow.y, a0[1]);
        a0[2] = fmaf(x0, arow.z, a0[2]);
        a0[3] = fmaf(x0, arow.w, a0[3]);
        a1[0] = fmaf(x1, arow.x, a1[0]);
        a1[1] = fmaf(x1, arow.y, a1[1]);
        a1[2] = fmaf(x1, arow.z, a1[2]);
        a1[3] = fmaf(x1, arow.w, a1[3]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        nxt[r * LK + c + e] = a0[e];
        nxt[(r + R / 2) * LK + c + e] = a1[e];
      }
    }
    __syncthreads();
    for (int i = tid; i < R * K; i += kCombThreads) {
      const int rr = i / K, cc = i - rr * K;
      cur[rr * LK + cc] = nxt[rr * LK + cc];
    }
  }
}

// final_state[b] = end state of segment (b, P - 1).
__global__ void __launch_bounds__(kThreads)
seg_final_kernel(const float* __restrict__ ends, float* __restrict__ final_state, int B, int H,
                 int V, int K, int P) {
  const size_t per = (size_t)H * V * K;
  const size_t total = (size_t)B * per;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (size_t)gridDim.x * kThreads) {
    const size_t b = i / per, e = i - b * per;
    final_state[i] = ends[((size_t)b * P + P - 1) * per + e];
  }
}

struct SegLayout {
  int L, nseg;
  size_t cu_off, ident_off, A_off, N_off, start_off, ends_off, bytes;
};

SegLayout seg_layout(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, int64_t chunk,
                     int64_t P) {
  SegLayout g;
  const int64_t per = (T + P - 1) / P;
  g.L = (int)(((per + chunk - 1) / chunk) * chunk);
  g.nseg = (int)(B * P);
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  g.cu_off = off;
  off = align(off + (size_t)(g.nseg + 1) * sizeof(int));
  g.ident_off = off;
  off = align(off + (size_t)g.nseg * H * K * K * sizeof(float));
  g.A_off = off;
  off = align(off + (size_t)g.nseg * H * K * K * sizeof(float));
  g.N_off = off;
  off = align(off + (size_t)g.nseg * H * V * K * sizeof(float));
  g.start_off = off;
  off = align(off + (size_t)g.nseg * H * V * K * sizeof(float));
  g.ends_off = off;
  off = align(off + (size_t)g.nseg * H * V * K * sizeof(float));
  g.bytes = off;
  return g;
}

}  // namespace

size_t fwd_segmented_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                     int64_t chunk, int64_t segments) {
  return seg_layout(B, T, H, K, V, chunk, segments).bytes;
}

hipError_t launch_fwd_segmented(const FwdArgs& a, bool bf16, int P, void* workspace,
                                hipStream_t stream) {
  const SegLayout g = seg_layout(a.B, a.T, a.H, a.K, a.V, a.chunk, P);
  char* ws = static_cast<char*>(workspace);
  int* cu = reinterpret_cast<int*>(ws + g.cu_off);
  float* ident = reinterpret_cast<float*>(ws + g.ident_off);
  float* Aseg = reinterpret_cast<float*>(ws + g.A_off);
  float* Nseg = reinterpret_cast<float*>(ws + g.N_off);
  float* start = reinterpret_cast<float*>(ws + g.start_off);
  float* ends = reinterpret_cast<float*>(ws + g.ends_off);
  auto fwd = [&](const FwdArgs& f) { return bf16 ? launch_fwd_bf16(f, stream) : launch_fwd_f32(f, stream); };
  hipError_t e;

  hipLaunchKernelGGL(seg_init_kernel, dim3(256), dim3(kThreads), 0, stream, cu, ident, a.B, a.T,
                     a.H, a.K, P, g.L);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // 1. per-segment N (values, zero start) and A (no values, identity start, K rows)
  FwdArgs f = a;
  f.B = g.nseg;
  f.T = a.B * a.T;  // the packed token axis
  f.cu_seqlens = cu;
  f.o = nullptr;
  f.s0 = nullptr;
  f.s_final = Nseg;
  f.s_ckpt = nullptr;
  if ((e = fwd(f)) != hipSuccess) return e;
  f.v = nullptr;
  f.V = a.K;
  f.s0 = ident;
  f.s_final = Aseg;
  if ((e = fwd(f)) != hipSuccess) return e;

  // 2. true segment starts, in segment order per stream
  {
    const size_t lds = sizeof(float) * (2 * kCombRows * (a.K + 1) + 2 * (size_t)a.K * a.K);
    if ((e = hipFuncSetAttribute((const void*)seg_combine_kernel,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(seg_combine_kernel, dim3(a.V / kCombRows, a.H, a.B), dim3(kCombThreads), lds,
                       stream, a.s0, Aseg, Nseg, start, a.H, a.K, a.V, P);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // 3. every segment again from its true start, with the output
  f = a;
  f.B = g.nseg;
  f.T = a.B * a.T;
  f.cu_seqlens = cu;
  f.s0 = start;
  f.s_final = a.s_final ? ends : nullptr;
  f.s_ckpt = nullptr;
  if ((e = fwd(f)) != hipSuccess) return e;
  if (a.s_final) {
    hipLaunchKernelGGL(seg_final_kernel, dim3(256), dim3(kThreads), 0, stream, ends, a.s_final,
                       a.B, a.H, a.V, a.K, P);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
