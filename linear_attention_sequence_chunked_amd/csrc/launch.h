// Internal launch interface between the C-ABI layer (gdn_api.hip) and the
// kernel translation units.  Not installed; the public interface is include/gdn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// One forward problem, already validated by the C-ABI layer.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* s0;  // may be null (zeros)
  void* o;
  float* s_final;   // may be null (skip)
  int B, T, H, K, V, chunk;
  float* s_ckpt = nullptr;  // optional chunk-start states [B, H, NT, V, K]
  // bf16 kernel, states only (o null): optional chunk-start states rounded to
  // bf16, [B, H, NT, V, K]
  void* s_ckpt_bf16 = nullptr;
  // fp32 matrix-core kernel, dense batches: optional per-chunk factors for the
  // backward, [B, H, NT] records of 3 C^2 + 3 C floats (M, P, Tm as C x C, the
  // cumulative natural-log gate, gam, beta)
  float* factors = nullptr;
  // optional packed batch: B sequences, sequence b = tokens [cu[b], cu[b+1]) of
  // the [1, T, H, *] tensors; states are [B, H, V, K]
  const int* cu_seqlens = nullptr;
  // bf16 kernel only: value rows per workgroup (16 or 32); 0 picks by grid size
  int vs = 0;
};

// Float32 q/k/v/o on the fp32 matrix cores (fwd_f32_mfma.hip): a chunk-parallel
// launch writes per-(chunk, head) records (gates, Tm, P), then the walk over
// chunks.  launch_fwd_f32 takes the records from a library-owned stream-ordered
// pool; launch_fwd_f32_records takes them from the caller
// (fwd_f32_record_bytes(a) bytes, 16-byte aligned).
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32_records(const FwdArgs& a, float* rec, hipStream_t stream);
// The chunk-parallel record launch alone (the walk left to the caller).
hipError_t launch_fwd_f32_record_only(const FwdArgs& a, float* rec, hipStream_t stream);
size_t fwd_f32_record_bytes(const FwdArgs& a);
bool fwd_f32_mfma_supported(int K, int V, int chunk);
// Float32 q/k/v/o: scalar fp32 kernel (exact fp32 products and sums), no scratch.
hipError_t launch_fwd_f32_scalar(const FwdArgs& a, hipStream_t stream);

// Chunk-start states only (o null): the state at every chunk start to s_ckpt
// [B,H,NT,V,K] -- the scalar fp32 kernel for float32 inputs, the MFMA kernel for
// bfloat16 inputs.
hipError_t launch_fwd_states(const FwdArgs& a, bool bf16, float* s_ckpt, hipStream_t stream);

// One backward problem, already validated by the C-ABI layer.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* s0;        // may be null (zeros)
  const void* d_o;
  const float* d_sfinal;  // may be null (zeros)
  void* dq;
  void* dk;
  void* dv;
  float* dalpha;
  float* dbeta;
  float* d_s0;            // may be null (skip)
  float* workspace;       // bwd_workspace_bytes(...) bytes
  int B, T, H, K, V, chunk;
};
// Workspace of the path a call with these sizes and dtype takes.
size_t bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, int64_t chunk,
                           bool bf16);
hipError_t launch_bwd(const BwdArgs& a, bool bf16, hipStream_t stream);
// Float32 reverse walk on the matrix cores over `chunk`-token chunks (16 or 32),
// reading the records launch_fwd_f32_records wrote for the same chunks; stores
// every chunk's end-state gradient to ws_dS [B, H, NT, V, K] and d_s0.
hipError_t launch_bwd_f32_dstate(const BwdArgs& a, int chunk, const float* rec, float* ws_dS,
                                 hipStream_t stream);
// Both float32 walks in one launch: the reverse walk above and the forward walk
// that writes the chunk-start states to ws_S [B, H, NT, V, K], from the records
// launch_fwd_f32_record_only wrote for the same chunks.  For V a multiple of 32
// and chunk 16 or 32 (bwd_f32_walks_supported).
bool bwd_f32_walks_supported(int K, int V, int chunk);
hipError_t launch_bwd_f32_walks(const BwdArgs& a, int chunk, const float* rec, float* ws_S,
                                float* ws_dS, hipStream_t stream);
// Float32 token gradients on the matrix cores, from the chunk-start states, the
// end-state gradients and the float32 prep's factors (M, P, Tm, gates).
hipError_t launch_bwd_f32_local(const BwdArgs& a, int chunk, const float* ws_S, const float* ws_dS,
                                const float* ws_F, hipStream_t stream);

// Bfloat16 backward on MFMA with 64-token chunks, whatever chunk the caller gave
// (K and V 32, 64 or 128).  Workspace: chunk-start states, chunk-end state
// gradients, per-chunk records.
bool bwd_bf16_supported(int K, int V);
size_t bwd_bf16_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);

// Value rows per workgroup (16 or 32) that the bf16 forward picks for a dense call.
int fwd_bf16_value_slice(int B, int H, int V);

// Segment-parallel forward (P segments per sequence) with a caller workspace.
size_t fwd_segmented_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                     int64_t chunk, int64_t segments);
// Segment count with the lowest modelled time on `cus` compute units (1 = the
// plain call is expected to be fastest).
int64_t fwd_segments_hint(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, int64_t chunk,
                          int64_t cus);
// Float32 inputs run the three passes on the fp32 matrix cores, whose per-chunk
// factors come from the library's stream-ordered pool, unless may_allocate is false
// (then the scalar fp32 kernel, which needs no scratch).
hipError_t launch_fwd_segmented(const FwdArgs& a, bool bf16, int segments, void* workspace,
                                hipStream_t stream, bool may_allocate = true);
// The same with the library's per-device static scratch of kSegmentedScratchBytes
// instead of a caller workspace (no allocation; calls that overlap on one device
// race on it).  hipErrorInvalidValue when the call needs more than that.
constexpr size_t kSegmentedScratchBytes = size_t(64) << 20;
hipError_t launch_fwd_segmented_noalloc(const FwdArgs& a, bool bf16, int segments,
                                        hipStream_t stream);

// One decode step (T = 1), already validated by the C-ABI layer.
struct DecodeArgs {
  const void* q;      // [B, H, K]
  const void* k;      // [B, H, K]
  const void* v;      // [B, H, V]
  const float* alpha; // [B, H]
  const float* beta;  // [B, H]
  float* state;       // [B, H, V, K], updated in place
  void* o;            // [B, H, V]
  int B, H, K, V;
};
hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream);

// The two states-only passes of the segment-parallel forward in one bf16 launch
// with 64 value rows per workgroup: `a` describes the N pass (values a.v, zero
// start, end states to a.s_final, V rows), and the A pass runs beside it over the
// same packed sequences with no values, start states `ident` and K rows, end
// states to `a_final`.  Needs 64-token chunks and K, V in {64, 128}
// (fwd_bf16_seg_states_supported); hipErrorInvalidValue otherwise.
bool fwd_bf16_seg_states_supported(int K, int V, int chunk);
hipError_t launch_fwd_bf16_seg_states(const FwdArgs& a, const float* ident, float* a_final,
                                      hipStream_t stream);

// Bfloat16 q/k/v/o: bf16 MFMA kernel with fp32 accumulation and fp32 state.
// Returns hipErrorInvalidValue for a shape outside its compiled set.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
bool fwd_bf16_supported(int K, int V, int chunk);

}  // namespace gdn
