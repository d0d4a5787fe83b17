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

#include <mutex>

// Scratch of the allocation-free segmented forward (gdn_chunk_fwd_segmented_noalloc):
// every GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device (segmented_scratch below).
static __device__ __align__(256) unsigned char scratch[gdn::kSegmentedScratchBytes];

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

// start_0 = S0 (or 0); start_{s+1} = start_s A_s + N_s.  The rows of the state
// are independent chains, so one workgroup takes 16 state rows of one (stream,
// head) with one wavefront per 16 state columns.  The 16 x K row block of start_s
// sits in LDS (one buffer per parity of s, one barrier per step); each wavefront
// forms its 16 x 16 tile of start_s A_s + N_s with float32 matrix-core products
// (16 x 16 x 4 per instruction, two accumulator chains), reading its column tile
// of A_s and N_s from registers that were loaded during the previous step.
//
// Operand layout of the 16 x 16 x 4 float32 product: lane (t = lane % 16,
// g = lane / 16) supplies the left operand's row t and the right operand's column
// t at reduction index g, and receives rows 4g .. 4g + 3 of column t.  Reduction
// index kk = 4m + j of the row block maps to state column k = 16m + 4g + j, so a
// lane reads its four left operands of a group m as one 16-byte LDS read.
typedef float comb_f32x4 __attribute__((ext_vector_type(4)));

template <int K>
struct CombRegs {
  float a[K / 4];  // A_s[16m + 4g + j][col] at index 4m + j
  float n[4];      // N_s[row r0 + 4g + i][col]
};

template <int K>
__device__ __forceinline__ void comb_load(const float* __restrict__ A, const float* __restrict__ N,
                                          int col, int g, CombRegs<K>& r) {
#pragma unroll
  for (int m = 0; m < K / 16; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) r.a[4 * m + j] = A[(size_t)(16 * m + 4 * g + j) * K + col];
#pragma unroll
  for (int i = 0; i < 4; ++i) r.n[i] = N[(size_t)(4 * g + i) * K + col];
}

template <int K>
__global__ void __launch_bounds__(512)
seg_combine_kernel(const float* __restrict__ s0, const float* __restrict__ Aseg,
                   const float* __restrict__ Nseg, float* __restrict__ start, int H, int V, int P) {
  constexpr int NT = K * 4, LX = K + 4;
  __shared__ __attribute__((aligned(16))) float xs[2][16 * LX];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = lane & 15, g = lane >> 4;
  const int col = 16 * w + t;
  // XCD-aware mapping (one-dimensional grid of B * H * V/16): consecutive
  // workgroup ids go to different XCDs, so the row blocks of one (stream, head),
  // which read the same transitions A_s, get ids equal modulo 8 (same XCD, shared
  // L2)
  int item = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) item = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int nrb = V / 16, bh = item / nrb;
  const int r0 = (item - bh * nrb) * 16, h = bh % H, b = bh / H;
  const size_t seg0 = (size_t)b * P * H + h;  // segment s of this stream: seg0 + s * H
  const size_t rowblk = (size_t)r0 * K;       // offset of row r0 in a [V, K] state

  // start_0: every thread holds four of the 16 x K entries (NT = 4K threads)
  float x0[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (s0) {
    const float* src = s0 + (((size_t)b * H + h) * V + r0) * K;
#pragma unroll
    for (int j = 0; j < 4; ++j) x0[j] = src[threadIdx.x + j * NT];
  }
  // A_s, N_s arrive one step ahead in two register sets used in turn (segment
  // indices are clamped to the last transition P - 2, so every load is in
  // bounds; the spare ones go unused)
  auto load = [&](int s, CombRegs<K>& r) {
    const size_t sg = seg0 + (size_t)max(0, min(s, P - 2)) * H;
    comb_load<K>(Aseg + sg * K * K, Nseg + sg * V * K + rowblk, col, g, r);
  };
  CombRegs<K> ra, rb;
  load(0, ra);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = threadIdx.x + j * NT, r = i / K, cc = i - r * K;
    xs[0][r * LX + cc] = x0[j];
    start[seg0 * V * K + rowblk + i] = x0[j];
  }
  // step s applies `use` (segment s) and loads segment s + 1 into `fill`; N is
  // added after the products so that no register of `use` is copied
  auto step = [&](int s, const CombRegs<K>& use, CombRegs<K>& fill) {
    load(s + 1, fill);
    __syncthreads();  // start_s complete in xs[s & 1]
    const float* x = xs[s & 1] + t * LX + 4 * g;
    comb_f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f};
    comb_f32x4 acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < K / 16; ++m) {
      const float4 xv = *reinterpret_cast<const float4*>(x + 16 * m);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv.x, use.a[4 * m + 0], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv.y, use.a[4 * m + 1], acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv.z, use.a[4 * m + 2], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv.w, use.a[4 * m + 3], acc1, 0, 0, 0);
    }
    float* xn = xs[(s + 1) & 1];
    float* out = start + (seg0 + (size_t)(s + 1) * H) * V * K + rowblk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = (acc0[i] + acc1[i]) + use.n[i];
      xn[(4 * g + i) * LX + col] = v;
      out[(size_t)(4 * g + i) * K + col] = v;
    }
  };
  // steps s = 0 .. P - 2: whole pairs, then the odd one (each register set a step
  // loads is read on every path out of its block, so no load is moved later)
  int s = 0;
  for (; s + 2 < P; s += 2) {
    step(s, ra, rb);
    step(s + 1, rb, ra);
  }
  if (s + 1 < P) step(s, ra, rb);
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

// Modelled time of the plain call (P = 1) and of the segmented one.  A forward
// pass over streams of n chunks takes rounds * n * t_chunk: one workgroup per CU
// (the bf16 kernel fills a CU's LDS), rounds = ceil(workgroups / CUs), and
// t_chunk = 2.2 us with 32 value rows per workgroup or 1.86 us with 16 (bf16,
// K = 128, 64-token chunks, measured on MI355X; scaled by chunk / 64 here).  The
// segmented call is three such passes over the segments (the A pass with K state
// rows) plus P - 1 combine steps of about 1.8 us.
int64_t fwd_segments_hint(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, int64_t chunk,
                          int64_t cus) {
  if (B <= 0 || T <= 0 || H <= 0 || K <= 0 || V <= 0 || chunk <= 0 || cus <= 0) return 0;
  if (B * H > (INT64_C(1) << 24)) return 1;  // that many streams fill the GPU by themselves
  // Per-chunk times of the forward kernel (microseconds at 64-token chunks, from
  // kernel traces on MI355X): with outputs 1.97 (32 value rows per workgroup) or
  // 1.71 (16 rows); states only 1.57 or 1.40, and 2.09 for the launch that runs
  // both states-only passes with 64 rows per workgroup (64-token chunks, K and V
  // in {64, 128}).  Each pass also runs two pipeline-fill iterations and costs
  // about 6 us of launch; the combine 1.8 us per segment step plus its launch.
  const double scale = (double)chunk / 64.0;
  constexpr double kLaunch = 6.0;
  auto rounds_of = [&](int64_t wgs) { return (double)((wgs + cus - 1) / cus); };
  auto pass = [&](int64_t streams, int64_t rows, int64_t nchunks, bool outputs) {
    if (streams > (INT64_C(1) << 24)) return 1e30;  // beyond any useful segment count
    const int vs = fwd_bf16_value_slice((int)streams, (int)H, (int)rows);
    const int64_t wgs = streams * H * ((rows + vs - 1) / vs);
    const double per = outputs ? (vs == 32 ? 1.97 : 1.71) : (vs == 32 ? 1.57 : 1.40);
    return rounds_of(wgs) * (double)(nchunks + 2) * per * scale + kLaunch;
  };
  const bool merged = fwd_bf16_seg_states_supported((int)K, (int)V, (int)chunk);
  auto states = [&](int64_t streams, int64_t nchunks) {
    if (!merged) return pass(streams, V, nchunks, false) + pass(streams, K, nchunks, false);
    if (streams > (INT64_C(1) << 24)) return 1e30;
    return rounds_of(streams * H * (V / 64 + K / 64)) * (double)(nchunks + 2) * 2.09 + kLaunch;
  };
  const int64_t nch = (T + chunk - 1) / chunk;
  double best = pass(B, V, nch, true);
  int64_t best_p = 1;
  // at least four chunks per segment, at most 256 segments
  for (int64_t P = 2; P <= 256 && 4 * P <= nch; ++P) {
    const int64_t L = ((T + P - 1) / P + chunk - 1) / chunk;  // chunks per segment
    const double t = states(B * P, L) + pass(B * P, V, L, true) + 1.8 * (double)(P - 1) + kLaunch;
    if (t < best) {
      best = t;
      best_p = P;
    }
  }
  return best_p;
}

size_t fwd_segmented_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                     int64_t chunk, int64_t segments) {
  return seg_layout(B, T, H, K, V, chunk, segments).bytes;
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on device `dev`, looked up on the first call there
// with `dev` current (the caller's current device is restored after).
hipError_t segmented_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_fwd_segmented_noalloc(const FwdArgs& a, bool bf16, int P, hipStream_t stream) {
  if (fwd_segmented_workspace_bytes(a.B, a.T, a.H, a.K, a.V, a.chunk, P) > kSegmentedScratchBytes)
    return hipErrorInvalidValue;
  int dev = -1;
  if (stream) {
    hipDevice_t d;
    const hipError_t e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return e;
    dev = static_cast<int>(d);
  } else {
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
  }
  void* ws = nullptr;
  const hipError_t e = segmented_scratch(dev, &ws);
  if (e != hipSuccess) return e;
  return launch_fwd_segmented(a, bf16, P, ws, stream, /*may_allocate=*/false);
}

hipError_t launch_fwd_segmented(const FwdArgs& a, bool bf16, int P, void* workspace,
                                hipStream_t stream, bool may_allocate) {
  const SegLayout g = seg_layout(a.B, a.T, a.H, a.K, a.V, a.chunk, P);
  char* ws = static_cast<char*>(workspace);
  int* cu = reinterpret_cast<int*>(ws + g.cu_off);
  float* ident = reinterpret_cast<float*>(ws + g.ident_off);
  float* Aseg = reinterpret_cast<float*>(ws + g.A_off);
  float* Nseg = reinterpret_cast<float*>(ws + g.N_off);
  float* start = reinterpret_cast<float*>(ws + g.start_off);
  float* ends = reinterpret_cast<float*>(ws + g.ends_off);
  // float32 passes: the matrix-core forward (factors from the library's stream-ordered
  // pool) when the call may allocate, else the scalar kernel (no scratch)
  auto fwd = [&](const FwdArgs& f) {
    if (bf16) return launch_fwd_bf16(f, stream);
    return may_allocate ? launch_fwd_f32(f, stream) : launch_fwd_f32_scalar(f, stream);
  };
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
  if (bf16 && fwd_bf16_seg_states_supported(a.K, a.V, a.chunk)) {
    // both passes in one launch, 64 value rows per workgroup
    if ((e = launch_fwd_bf16_seg_states(f, ident, Aseg, stream)) != hipSuccess) return e;
  } else {
    if ((e = fwd(f)) != hipSuccess) return e;
    f.v = nullptr;
    f.V = a.K;
    f.s0 = ident;
    f.s_final = Aseg;
    if ((e = fwd(f)) != hipSuccess) return e;
  }

  // 2. true segment starts, in segment order per stream
  {
    const dim3 grid(a.B * a.H * (a.V / 16)), block(4 * a.K);
    switch (a.K) {
      case 16: hipLaunchKernelGGL(seg_combine_kernel<16>, grid, block, 0, stream, a.s0, Aseg, Nseg, start, a.H, a.V, P); break;
      case 32: hipLaunchKernelGGL(seg_combine_kernel<32>, grid, block, 0, stream, a.s0, Aseg, Nseg, start, a.H, a.V, P); break;
      case 64: hipLaunchKernelGGL(seg_combine_kernel<64>, grid, block, 0, stream, a.s0, Aseg, Nseg, start, a.H, a.V, P); break;
      case 128: hipLaunchKernelGGL(seg_combine_kernel<128>, grid, block, 0, stream, a.s0, Aseg, Nseg, start, a.H, a.V, P); break;
      default: return hipErrorInvalidValue;
    }
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
