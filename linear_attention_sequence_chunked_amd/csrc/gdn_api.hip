// C-ABI layer of libgdn: host-side argument checks, then one kernel launch on
// the caller's stream.  Every check runs before any device work, so a failing
// call enqueues nothing and touches no output.  There is exactly one kernel per
// dtype and no fallback: a shape outside the compiled set is an error.
#include <stdint.h>

#include "../../include/gdn.h"
#include "launch.h"

static_assert(GDN_SEGMENTED_NOALLOC_MAX_BYTES == gdn::kSegmentedScratchBytes,
              "header and library disagree on the static scratch size");

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool width_supported(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Shape checks shared by the entry points: INVALID_VALUE for non-positive sizes,
// NOT_SUPPORTED outside the compiled set, SUCCESS otherwise.
gdn_status_t check_shape(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, int64_t chunk,
                         gdn_dtype_t dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || K <= 0 || V <= 0 || chunk <= 0) return GDN_ERROR_INVALID_VALUE;
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return GDN_ERROR_NOT_SUPPORTED;
  if (!width_supported(K) || !width_supported(V)) return GDN_ERROR_NOT_SUPPORTED;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERROR_NOT_SUPPORTED;
  const int64_t maxd = K > V ? K : V;
  if (B > (INT64_C(1) << 31) || T > (INT64_C(1) << 31) || H > (INT64_C(1) << 31) ||
      B * T > (INT64_C(1) << 31) || B * T * H * maxd >= (INT64_C(1) << 31))
    return GDN_ERROR_NOT_SUPPORTED;
  return GDN_SUCCESS;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status_t status) {
  switch (status) {
    case GDN_SUCCESS:
      return "success";
    case GDN_ERROR_INVALID_VALUE:
      return "invalid value: a required pointer is NULL, a size is not positive, a pointer is "
             "not 16-byte aligned, or an output overlaps another buffer";
    case GDN_ERROR_NOT_SUPPORTED:
      return "not supported: K and V must be 16, 32, 64 or 128, chunk 16, 32 or 64, dtype F32 "
             "or BF16, B*T*H*max(K,V) below 2^31 and B*H*V*K at most 2^31";
    case GDN_ERROR_LAUNCH:
      return "kernel launch failed";
    case GDN_ERROR_SCRATCH_LIMIT:
      return "the call needs more scratch than the allocation-free entry point's static buffer "
             "holds (GDN_SEGMENTED_NOALLOC_MAX_BYTES = 64 MiB per device; "
             "gdn_chunk_fwd_segmented_workspace_size gives the need): use gdn_chunk_fwd_segmented "
             "with a workspace, or fewer segments";
  }
  return "unknown status";
}

}  // extern "C"

namespace {

// Shared body of the dense and packed forward entry points.  The token tensors
// hold NTOK = Bt * T token rows (Bt = B dense, 1 packed); states hold B rows.
// may_allocate = false (the allocation-free entry point): float32 inputs take the
// scalar kernel, which needs no scratch, instead of the matrix-core path with its
// pooled factors.
gdn_status_t chunk_fwd_impl(const void* q, const void* k, const void* v, const float* alpha,
                            const float* beta, const int32_t* cu_seqlens, const float* initial_state,
                            void* o, float* final_state, int64_t B, int64_t Bt, int64_t T,
                            int64_t H, int64_t K, int64_t V, int64_t chunk, gdn_dtype_t dtype,
                            void* stream, bool may_allocate = true) {
  if (!q || !k || !v || !alpha || !beta || !o) return GDN_ERROR_INVALID_VALUE;
  const void* ptrs[] = {q, k, v, alpha, beta, initial_state, o, final_state};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERROR_INVALID_VALUE;
  const gdn_status_t st = check_shape(Bt, T, H, K, V, chunk, dtype);
  if (st != GDN_SUCCESS) return st;
  if (B <= 0) return GDN_ERROR_INVALID_VALUE;
  if (B > (INT64_C(1) << 31) / (H * V * K)) return GDN_ERROR_NOT_SUPPORTED;

  const int64_t ntok = Bt * T;
  const int64_t esz = dtype == GDN_DTYPE_F32 ? 4 : 2;
  const Range rq = range_of(q, ntok * H * K * esz), rk = range_of(k, ntok * H * K * esz),
              rv = range_of(v, ntok * H * V * esz), ra = range_of(alpha, ntok * H * 4),
              rb = range_of(beta, ntok * H * 4), ro = range_of(o, ntok * H * V * esz);
  const int64_t state_bytes = B * H * V * K * 4;
  const Range inputs[] = {rq, rk, rv, ra, rb,
                          cu_seqlens ? range_of(cu_seqlens, (B + 1) * 4) : Range{0, 0}};
  for (const Range& r : inputs)
    if (r.hi != r.lo && overlaps(ro, r)) return GDN_ERROR_INVALID_VALUE;
  if (initial_state && overlaps(ro, range_of(initial_state, state_bytes)))
    return GDN_ERROR_INVALID_VALUE;
  if (final_state) {
    const Range rf = range_of(final_state, state_bytes);
    for (const Range& r : inputs)
      if (r.hi != r.lo && overlaps(rf, r)) return GDN_ERROR_INVALID_VALUE;
    if (overlaps(rf, ro)) return GDN_ERROR_INVALID_VALUE;
    if (initial_state && initial_state != final_state &&
        overlaps(rf, range_of(initial_state, state_bytes)))
      return GDN_ERROR_INVALID_VALUE;
  }

  gdn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.s0 = initial_state;
  a.o = o;
  a.s_final = final_state;
  a.B = static_cast<int>(B);
  a.T = static_cast<int>(T);
  a.H = static_cast<int>(H);
  a.K = static_cast<int>(K);
  a.V = static_cast<int>(V);
  a.chunk = static_cast<int>(chunk);
  a.cu_seqlens = cu_seqlens;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = dtype == GDN_DTYPE_BF16 ? gdn::launch_fwd_bf16(a, s)
                   : may_allocate          ? gdn::launch_fwd_f32(a, s)
                                           : gdn::launch_fwd_f32_scalar(a, s);
  return err == hipSuccess ? GDN_SUCCESS : GDN_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

gdn_status_t gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* initial_state, void* o,
                           float* final_state, int64_t B, int64_t T, int64_t H, int64_t K,
                           int64_t V, int64_t chunk, gdn_dtype_t dtype, void* stream) {
  if (B <= 0) return GDN_ERROR_INVALID_VALUE;
  return chunk_fwd_impl(q, k, v, alpha, beta, nullptr, initial_state, o, final_state, B, B, T, H,
                        K, V, chunk, dtype, stream);
}

gdn_status_t gdn_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* alpha,
                                  const float* beta, const int32_t* cu_seqlens, int64_t N,
                                  const float* initial_state, void* o, float* final_state,
                                  int64_t T, int64_t H, int64_t K, int64_t V, int64_t chunk,
                                  gdn_dtype_t dtype, void* stream) {
  if (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0 || N <= 0)
    return GDN_ERROR_INVALID_VALUE;
  return chunk_fwd_impl(q, k, v, alpha, beta, cu_seqlens, initial_state, o, final_state, N, 1, T,
                        H, K, V, chunk, dtype, stream);
}

int64_t gdn_chunk_fwd_segments_hint(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                    int64_t chunk, int64_t num_cus) {
  if (num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return 0;
    num_cus = n;
  }
  return gdn::fwd_segments_hint(B, T, H, K, V, chunk, num_cus);
}

size_t gdn_chunk_fwd_segmented_workspace_size(int64_t B, int64_t T, int64_t H, int64_t K,
                                              int64_t V, int64_t chunk, int64_t segments) {
  if (B <= 0 || T <= 0 || H <= 0 || K <= 0 || V <= 0 || chunk <= 0 || segments <= 0) return 0;
  return gdn::fwd_segmented_workspace_bytes(B, T, H, K, V, chunk, segments);
}

}  // extern "C"

namespace {

// Shared body of the segmented entry points: the caller's workspace, or (noalloc)
// the library's static per-device scratch.
gdn_status_t segmented_impl(const void* q, const void* k, const void* v, const float* alpha,
                            const float* beta, const float* initial_state, void* o,
                            float* final_state, int64_t B, int64_t T, int64_t H, int64_t K,
                            int64_t V, int64_t chunk, int64_t segments, void* workspace,
                            size_t workspace_bytes, bool noalloc, gdn_dtype_t dtype, void* stream) {
  if (segments <= 0) return GDN_ERROR_INVALID_VALUE;
  if (segments == 1)
    return chunk_fwd_impl(q, k, v, alpha, beta, nullptr, initial_state, o, final_state, B, B, T,
                          H, K, V, chunk, dtype, stream, /*may_allocate=*/!noalloc);
  if (!noalloc && (!workspace || !aligned16(workspace))) return GDN_ERROR_INVALID_VALUE;
  // shape checks of the dense call, plus the B * segments packed states
  const gdn_status_t st = check_shape(B, T, H, K, V, chunk, dtype);
  if (st != GDN_SUCCESS) return st;
  if (segments > T || B * segments > (INT64_C(1) << 31) / (H * K * (K > V ? K : V)))
    return GDN_ERROR_NOT_SUPPORTED;
  const size_t need = gdn::fwd_segmented_workspace_bytes(B, T, H, K, V, chunk, segments);
  if (noalloc && need > gdn::kSegmentedScratchBytes) return GDN_ERROR_SCRATCH_LIMIT;
  if (!noalloc && workspace_bytes < need) return GDN_ERROR_INVALID_VALUE;
  const int64_t esz = dtype == GDN_DTYPE_F32 ? 4 : 2;
  const Range others[] = {range_of(q, B * T * H * K * esz), range_of(k, B * T * H * K * esz),
                          range_of(v, B * T * H * V * esz), range_of(alpha, B * T * H * 4),
                          range_of(beta, B * T * H * 4), range_of(o, B * T * H * V * esz),
                          initial_state ? range_of(initial_state, B * H * V * K * 4) : Range{0, 0},
                          final_state ? range_of(final_state, B * H * V * K * 4) : Range{0, 0}};
  if (!noalloc) {
    const Range rw = range_of(workspace, (int64_t)workspace_bytes);
    for (const Range& r : others)
      if (r.hi != r.lo && overlaps(rw, r)) return GDN_ERROR_INVALID_VALUE;
  }
  // the pointer, alignment and overlap checks of the dense call
  if (!q || !k || !v || !alpha || !beta || !o) return GDN_ERROR_INVALID_VALUE;
  const void* ptrs[] = {q, k, v, alpha, beta, initial_state, o, final_state};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERROR_INVALID_VALUE;
  const Range ro = range_of(o, B * T * H * V * esz);
  for (int i = 0; i < 5; ++i)
    if (overlaps(ro, others[i])) return GDN_ERROR_INVALID_VALUE;
  if (initial_state && overlaps(ro, others[6])) return GDN_ERROR_INVALID_VALUE;
  if (final_state) {
    for (int i = 0; i < 6; ++i)
      if (overlaps(others[7], others[i])) return GDN_ERROR_INVALID_VALUE;
    if (initial_state && initial_state != final_state && overlaps(others[7], others[6]))
      return GDN_ERROR_INVALID_VALUE;
  }
  gdn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.s0 = initial_state;
  a.o = o;
  a.s_final = final_state;
  a.B = static_cast<int>(B);
  a.T = static_cast<int>(T);
  a.H = static_cast<int>(H);
  a.K = static_cast<int>(K);
  a.V = static_cast<int>(V);
  a.chunk = static_cast<int>(chunk);
  const bool bf16 = dtype == GDN_DTYPE_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err =
      noalloc ? gdn::launch_fwd_segmented_noalloc(a, bf16, static_cast<int>(segments), s)
              : gdn::launch_fwd_segmented(a, bf16, static_cast<int>(segments), workspace, s);
  return err == hipSuccess ? GDN_SUCCESS : GDN_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

gdn_status_t gdn_chunk_fwd_segmented(const void* q, const void* k, const void* v,
                                     const float* alpha, const float* beta,
                                     const float* initial_state, void* o, float* final_state,
                                     int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                     int64_t chunk, int64_t segments, void* workspace,
                                     size_t workspace_bytes, gdn_dtype_t dtype, void* stream) {
  return segmented_impl(q, k, v, alpha, beta, initial_state, o, final_state, B, T, H, K, V, chunk,
                        segments, workspace, workspace_bytes, false, dtype, stream);
}

gdn_status_t gdn_chunk_fwd_segmented_noalloc(const void* q, const void* k, const void* v,
                                             const float* alpha, const float* beta,
                                             const float* initial_state, void* o,
                                             float* final_state, int64_t B, int64_t T, int64_t H,
                                             int64_t K, int64_t V, int64_t chunk, int64_t segments,
                                             gdn_dtype_t dtype, void* stream) {
  return segmented_impl(q, k, v, alpha, beta, initial_state, o, final_state, B, T, H, K, V, chunk,
                        segments, nullptr, 0, true, dtype, stream);
}

gdn_status_t gdn_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, float* state, void* o, int64_t B, int64_t H,
                             int64_t K, int64_t V, gdn_dtype_t dtype, void* stream) {
  if (!q || !k || !v || !alpha || !beta || !state || !o) return GDN_ERROR_INVALID_VALUE;
  const void* ptrs[] = {q, k, v, alpha, beta, state, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GDN_ERROR_INVALID_VALUE;
  const gdn_status_t st = check_shape(B, 1, H, K, V, 16, dtype);
  if (st != GDN_SUCCESS) return st;
  if (B * H >= (INT64_C(1) << 31) / (K > V ? K : V)) return GDN_ERROR_NOT_SUPPORTED;
  const int64_t esz = dtype == GDN_DTYPE_F32 ? 4 : 2;
  const Range in[] = {range_of(q, B * H * K * esz), range_of(k, B * H * K * esz),
                      range_of(v, B * H * V * esz), range_of(alpha, B * H * 4),
                      range_of(beta, B * H * 4)};
  const Range rs = range_of(state, B * H * V * K * 4), ro = range_of(o, B * H * V * esz);
  for (const Range& r : in)
    if (overlaps(rs, r) || overlaps(ro, r)) return GDN_ERROR_INVALID_VALUE;
  if (overlaps(rs, ro)) return GDN_ERROR_INVALID_VALUE;
  gdn::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.state = state;
  a.o = o;
  a.B = static_cast<int>(B);
  a.H = static_cast<int>(H);
  a.K = static_cast<int>(K);
  a.V = static_cast<int>(V);
  hipError_t err = gdn::launch_decode(a, dtype == GDN_DTYPE_BF16, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GDN_SUCCESS : GDN_ERROR_LAUNCH;
}

size_t gdn_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                    int64_t chunk, gdn_dtype_t dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || K <= 0 || V <= 0 || chunk <= 0) return 0;
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return 0;
  return gdn::bwd_workspace_bytes(B, T, H, K, V, chunk, dtype == GDN_DTYPE_BF16);
}

gdn_status_t gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* initial_state, const void* d_o,
                           const float* d_final_state, void* dq, void* dk, void* dv,
                           float* dalpha, float* dbeta, float* d_initial_state, void* workspace,
                           size_t workspace_bytes, int64_t B, int64_t T, int64_t H, int64_t K,
                           int64_t V, int64_t chunk, gdn_dtype_t dtype, void* stream) {
  if (!q || !k || !v || !alpha || !beta || !d_o || !dq || !dk || !dv || !dalpha || !dbeta ||
      !workspace)
    return GDN_ERROR_INVALID_VALUE;
  const void* ptrs[] = {q, k, v, alpha, beta, initial_state, d_o, d_final_state, dq, dk, dv,
                        dalpha, dbeta, d_initial_state, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERROR_INVALID_VALUE;
  const gdn_status_t st = check_shape(B, T, H, K, V, chunk, dtype);
  if (st != GDN_SUCCESS) return st;
  if (workspace_bytes < gdn::bwd_workspace_bytes(B, T, H, K, V, chunk, dtype == GDN_DTYPE_BF16))
    return GDN_ERROR_INVALID_VALUE;

  const int64_t esz = dtype == GDN_DTYPE_F32 ? 4 : 2;
  const int64_t nk = B * T * H * K, nv = B * T * H * V, ng = B * T * H, ns = B * H * V * K;
  const Range in[] = {range_of(q, nk * esz), range_of(k, nk * esz), range_of(v, nv * esz),
                      range_of(alpha, ng * 4), range_of(beta, ng * 4),
                      initial_state ? range_of(initial_state, ns * 4) : Range{0, 0},
                      range_of(d_o, nv * esz),
                      d_final_state ? range_of(d_final_state, ns * 4) : Range{0, 0}};
  const Range out[] = {range_of(dq, nk * esz), range_of(dk, nk * esz), range_of(dv, nv * esz),
                       range_of(dalpha, ng * 4), range_of(dbeta, ng * 4),
                       d_initial_state ? range_of(d_initial_state, ns * 4) : Range{0, 0},
                       range_of(workspace, (int64_t)workspace_bytes)};
  const int nin = sizeof(in) / sizeof(in[0]), nout = sizeof(out) / sizeof(out[0]);
  for (int i = 0; i < nout; ++i) {
    if (out[i].hi == out[i].lo) continue;
    for (int j = 0; j < nin; ++j)
      if (in[j].hi != in[j].lo && overlaps(out[i], in[j])) return GDN_ERROR_INVALID_VALUE;
    for (int j = i + 1; j < nout; ++j)
      if (out[j].hi != out[j].lo && overlaps(out[i], out[j])) return GDN_ERROR_INVALID_VALUE;
  }

  gdn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.s0 = initial_state;
  a.d_o = d_o;
  a.d_sfinal = d_final_state;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dalpha = dalpha;
  a.dbeta = dbeta;
  a.d_s0 = d_initial_state;
  a.workspace = static_cast<float*>(workspace);
  a.B = static_cast<int>(B);
  a.T = static_cast<int>(T);
  a.H = static_cast<int>(H);
  a.K = static_cast<int>(K);
  a.V = static_cast<int>(V);
  a.chunk = static_cast<int>(chunk);
  hipError_t err = gdn::launch_bwd(a, dtype == GDN_DTYPE_BF16, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GDN_SUCCESS : GDN_ERROR_LAUNCH;
}

}  // extern "C"
