/*
 * gdn.h -- C ABI of the chunkwise gated-delta-rule forward and backward, and
 * of its single-token decode step, for AMD Instinct MI355X (gfx950).
 *
 * The operation.  For every batch b and head h, with state S of shape [V, K]:
 *
 *     S <- initial_state[b,h]            (zeros when initial_state is NULL)
 *     for t = 0 .. T-1:
 *         S      <- alpha_t S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *         o[b,t,h] = S q_t
 *     final_state[b,h] <- S
 *
 * This is the gated delta rule of "Sparse Delta Memory: layer and kernels"
 * (sparse-delta-memory 2.0.0), section "What the layer computes" -- decay the
 * state, read it with k, write beta times the prediction error, read the output
 * with q from the updated state -- in the dense limit its section "Product-key
 * top-k" describes, with the operator contract (shapes, optional state,
 * streaming continuation) of "OpenGDN 0.1.0", section "Core operator reference".
 * It is computed by the extended-WY / UT chunk decomposition those pages name
 * (cumulative log-gates, decay-weighted K K^T and Q K^T Gram matrices, the solve
 * (I + tril(beta A, -1))^-1, the W/U build, then a sequential inter-chunk state
 * update and readout); chunking changes results only by rounding.
 *
 * Conventions shared by every entry point:
 *  - All pointers are DEVICE pointers (memory from hipMalloc or a torch CUDA
 *    tensor on the current device), except where stated.  The caller owns every
 *    buffer; the library allocates no device memory for these calls, with one
 *    exception: the float32 forward (gdn_chunk_fwd, gdn_chunk_fwd_varlen and
 *    gdn_chunk_fwd_segmented with GDN_DTYPE_F32) takes a stream-ordered scratch of
 *    per-chunk factors from a library-owned memory pool on the stream's device
 *    (see gdn_chunk_fwd); gdn_chunk_fwd_segmented_noalloc never allocates.
 *  - Tensors are dense, contiguous and row-major, each at least 16-byte aligned:
 *        q, k            [B, T, H, K]   element type `dtype`
 *        v, o            [B, T, H, V]   element type `dtype`
 *        alpha, beta     [B, T, H]      float32
 *        initial_state,
 *        final_state     [B, H, V, K]   float32
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *    enqueued on it and the call returns without synchronising the host.
 *  - All argument checks happen on the host BEFORE any device work; on an error
 *    nothing is enqueued and no output is touched.  There is no fallback path:
 *    an unsupported shape or dtype is an error, never a slower kernel.
 *  - Domain (not checked on the device): 0 < alpha <= 1, beta finite.  NaN/Inf
 *    inputs propagate; nothing is clipped.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 8

#if defined(__GNUC__)
#define GDN_API __attribute__((visibility("default")))
#else
#define GDN_API
#endif

typedef enum gdn_status {
    GDN_SUCCESS = 0,
    GDN_ERROR_INVALID_VALUE = 1, /* NULL required pointer, non-positive size, misaligned pointer,
                                    or overlapping input/output buffers */
    GDN_ERROR_NOT_SUPPORTED = 2, /* valid, but outside the compiled kernel set (see below) */
    GDN_ERROR_LAUNCH = 3,        /* the HIP runtime refused the launch */
    GDN_ERROR_SCRATCH_LIMIT = 4  /* gdn_chunk_fwd_segmented_noalloc only: the call needs more
                                    than the static scratch (GDN_SEGMENTED_NOALLOC_MAX_BYTES) */
} gdn_status_t;

typedef enum gdn_dtype {
    GDN_DTYPE_F32 = 0,  /* IEEE float32 q, k, v, o */
    GDN_DTYPE_BF16 = 1  /* bfloat16 q, k, v, o; state arithmetic stays float32 */
} gdn_dtype_t;

/* ABI version of the loaded library (GDN_ABI_VERSION at build time). */
GDN_API int gdn_abi_version(void);

/* Static, NUL-terminated description of a status code (host memory, never freed). */
GDN_API const char *gdn_status_string(gdn_status_t status);

/*
 * gdn_chunk_fwd -- forward of the gated delta rule over T tokens.
 *
 *   q, k           [B,T,H,K] dtype        queries and keys (read only)
 *   v              [B,T,H,V] dtype        values (read only)
 *   alpha, beta    [B,T,H]   float32      decay gate and write strength (read only)
 *   initial_state  [B,H,V,K] float32      state before token 0, or NULL for zeros
 *   o              [B,T,H,V] dtype        output, o[b,t,h] = S_t q_t (written)
 *   final_state    [B,H,V,K] float32      state after token T-1, or NULL to skip
 *   B, T, H        batch, tokens, heads   B >= 1, H >= 1, T >= 1
 *   K, V           key and value widths   each one of 16, 32, 64, 128
 *   chunk          tokens per chunk       16, 32 or 64; T need not be a multiple
 *                                         (the last chunk is shorter)
 *   dtype          element type of q, k, v, o
 *   stream         hipStream_t as void*
 *
 * final_state may be the same pointer as initial_state (the state advances in
 * place); any other overlap between an output and any other buffer is rejected
 * when it is visible from the pointers and sizes.  Passing final_state back as
 * the next call's initial_state continues the stream ("OpenGDN 0.1.0", section
 * "Core operator reference").  The result is bitwise reproducible run to run:
 * every output element has one writer and every sum runs in a fixed order.
 * Sizes: B*T*H*max(K,V) must stay below 2^31 elements and the state B*H*V*K
 * at or below 2^31; larger calls return GDN_ERROR_NOT_SUPPORTED.
 *
 * Float32 inputs run on the fp32 matrix cores in two launches: one over
 * (chunk, head) that builds the state-independent factors of every chunk
 * (cumulative gates, Tm = (I + A)^-1 scaled by beta, the decayed Q K^T), then
 * the walk over chunks.  The factors, (2 chunk^2 + 2 chunk + 4) * 4 bytes per
 * (chunk, head) (33 KB at chunk 64; about B*T*H/chunk of them), live in a
 * stream-ordered allocation from a library-owned pool (hipMallocFromPoolAsync
 * on `stream`, hipFreeAsync on `stream` after the launches; the pool keeps the
 * memory for later calls).  If that allocation fails the call returns
 * GDN_ERROR_LAUNCH.  Bfloat16 inputs allocate nothing.
 */
GDN_API gdn_status_t gdn_chunk_fwd(const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta,
                           const float *initial_state,
                           void *o, float *final_state,
                           int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                           int64_t chunk, gdn_dtype_t dtype, void *stream);

/*
 * gdn_chunk_fwd_varlen -- gdn_chunk_fwd over a packed batch of N independent
 * sequences of different lengths (each starts from its own state; no state
 * passes between sequences).
 *
 *   q, k           [T,H,K] dtype        the N sequences back to back (T tokens in all)
 *   v, o           [T,H,V] dtype
 *   alpha, beta    [T,H]   float32
 *   cu_seqlens     [N+1]   int32        DEVICE array of offsets: sequence n is tokens
 *                                       cu_seqlens[n] .. cu_seqlens[n+1]-1; must be
 *                                       non-decreasing from 0 to T (empty sequences
 *                                       allowed).  Read on the device, not checked:
 *                                       offsets are clamped into [0, T], so a bad
 *                                       table gives wrong results, never an access
 *                                       outside the tensors.  4-byte aligned.
 *   N              number of sequences, N >= 1
 *   initial_state, final_state  [N,H,V,K] float32, NULL allowed as for gdn_chunk_fwd
 *   T, H, K, V, chunk, dtype, stream    as for gdn_chunk_fwd (chunks restart at
 *                                       every sequence start)
 *
 * Equal (bitwise) to N separate gdn_chunk_fwd calls with B = 1.  "OpenGDN 0.1.0",
 * section "Scope", lists packed variable-length batches and reset masks as outside
 * its operator; this entry point adds the first with the same per-sequence
 * contract and covers the second: a reset before token t (the state set to zero,
 * then the token applied) is a sequence boundary at t whose piece starts from a
 * zero initial state, so a batch with resets is one call with a boundary at every
 * row start and every reset (initial states: the row's own for its first piece,
 * zeros for the others; its final state is that of its last piece).
 */
GDN_API gdn_status_t gdn_chunk_fwd_varlen(const void *q, const void *k, const void *v,
                                  const float *alpha, const float *beta,
                                  const int32_t *cu_seqlens, int64_t N,
                                  const float *initial_state,
                                  void *o, float *final_state,
                                  int64_t T, int64_t H, int64_t K, int64_t V,
                                  int64_t chunk, gdn_dtype_t dtype, void *stream);

/*
 * gdn_chunk_fwd_segments_hint -- a `segments` value for gdn_chunk_fwd_segmented:
 * the count with the lowest modelled time for these sizes, 1 when the plain call
 * (gdn_chunk_fwd) is expected to be fastest.  The model: each of the three passes
 * walks every segment's chunks with one workgroup per compute unit at a time
 * (about 2.2 us per chunk with 32 value rows per workgroup, 1.86 us with 16, for
 * bf16 with 64-token chunks on MI355X), and the combine adds about 1.8 us per
 * segment.  Segments keep at least four chunks each; at most 256.
 *
 *   num_cus   compute units to plan for; 0 = those of the current device
 *             (the only case that makes a runtime call)
 *
 * Returns 0 when a size is not positive or the device cannot be queried.  Host
 * only: nothing is enqueued.  The value is advice; any 1 <= segments <= T is
 * accepted by gdn_chunk_fwd_segmented.
 */
GDN_API int64_t gdn_chunk_fwd_segments_hint(int64_t B, int64_t T, int64_t H, int64_t K,
                                            int64_t V, int64_t chunk, int64_t num_cus);

/*
 * gdn_chunk_fwd_segmented_workspace_size -- bytes of device workspace that
 * gdn_chunk_fwd_segmented needs (0 when a size is not positive).  It holds, per
 * (batch, segment, head), a K x K transition, three [V, K] states and a K x K
 * identity, all float32, plus the segment table.
 */
GDN_API size_t gdn_chunk_fwd_segmented_workspace_size(int64_t B, int64_t T, int64_t H,
                                                      int64_t K, int64_t V, int64_t chunk,
                                                      int64_t segments);

/*
 * gdn_chunk_fwd_segmented -- the result of gdn_chunk_fwd (same arguments and
 * outputs, up to float rounding) computed with every sequence split into
 * `segments` pieces of equal chunk-aligned length that run in parallel:
 *
 *   1. every segment from a zero state gives its end state N_s, and from an
 *      identity [K, K] state with zero values gives its transition A_s
 *      (the token step is affine in the state: S_end = S_start A_s + N_s);
 *   2. per stream, start_{s+1} = start_s A_s + N_s from start_0 = initial_state;
 *   3. every segment again from its true start writes o (and the last one the
 *      final state).
 *
 * For bfloat16 inputs with 64-token chunks and K, V in {64, 128} the two
 * state passes of step 1 run in one launch.  Float32 inputs run every pass on the
 * fp32 matrix cores, with the per-chunk factors of gdn_chunk_fwd (from the
 * library's pool, see gdn_chunk_fwd).
 *
 * State passing between chunks is the chunk recurrence of "Sparse Delta Memory:
 * layer and kernels", section "What the layer computes", applied between
 * segments.  It costs about 2.5 times the work of gdn_chunk_fwd and shortens the
 * sequential part `segments` times, so it pays only when B * H alone leaves most
 * of the GPU idle (long sequences, few streams).
 *
 *   segments       1 <= segments <= T (1 is exactly gdn_chunk_fwd, no workspace used)
 *   workspace      device scratch of at least
 *                  gdn_chunk_fwd_segmented_workspace_size(...) bytes, 16-byte
 *                  aligned, owned by the caller, contents undefined afterwards;
 *                  it may not overlap any other buffer
 *   the rest       as for gdn_chunk_fwd
 */
GDN_API gdn_status_t gdn_chunk_fwd_segmented(const void *q, const void *k, const void *v,
                                     const float *alpha, const float *beta,
                                     const float *initial_state,
                                     void *o, float *final_state,
                                     int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                     int64_t chunk, int64_t segments,
                                     void *workspace, size_t workspace_bytes,
                                     gdn_dtype_t dtype, void *stream);

/* Size of the static per-device scratch of gdn_chunk_fwd_segmented_noalloc. */
#define GDN_SEGMENTED_NOALLOC_MAX_BYTES ((size_t)64 << 20)

/*
 * gdn_chunk_fwd_segmented_noalloc -- gdn_chunk_fwd_segmented without a
 * workspace argument and without any allocation, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * The scratch lives in a static device array of GDN_SEGMENTED_NOALLOC_MAX_BYTES
 * (64 MiB) that every GPU the library runs on holds until the process ends (its
 * address is looked up once per device, on the first call there).  A call whose
 * gdn_chunk_fwd_segmented_workspace_size(...) exceeds it returns
 * GDN_ERROR_SCRATCH_LIMIT before any device work (B1 T32768 H16 with 4 segments
 * needs 21 MB; so does H2 with 32).  The call itself allocates nothing (no
 * hipMalloc, no allocating library routine); nothing in the scratch needs to
 * start at zero, and every pass overwrites what the next one reads.
 *
 * All calls on one GPU share that GPU's array: calls that overlap in time on one
 * device (different streams, or several host threads without ordering) RACE on
 * it and give wrong results.  Calls in one stream's order are safe.
 *
 *   arguments      as for gdn_chunk_fwd_segmented, without workspace and
 *                  workspace_bytes; results identical (bitwise) to it for
 *                  bfloat16 inputs.  Float32 inputs run on the scalar fp32
 *                  kernel here (the other entry points' fp32 matrix-core path
 *                  draws its per-chunk factors from a pool), so they agree with
 *                  gdn_chunk_fwd_segmented to rounding (within 1e-5 relative L2).
 */
GDN_API gdn_status_t gdn_chunk_fwd_segmented_noalloc(const void *q, const void *k, const void *v,
                                             const float *alpha, const float *beta,
                                             const float *initial_state,
                                             void *o, float *final_state,
                                             int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                                             int64_t chunk, int64_t segments,
                                             gdn_dtype_t dtype, void *stream);

/*
 * gdn_decode_step -- one token of the recurrence for every (batch, head), the
 * state advanced in place (the decode path of "Sparse Delta Memory: layer and
 * kernels", sections "What the layer computes" and "Execution"):
 *
 *     S <- alpha S (I - beta k k^T) + beta v k^T;   o = S q
 *
 *   q, k       [B,H,K] dtype     this token's query and key (read only)
 *   v          [B,H,V] dtype     this token's value (read only)
 *   alpha, beta [B,H]  float32   gates (read only)
 *   state      [B,H,V,K] float32 read and overwritten with the new state
 *   o          [B,H,V] dtype     output (written)
 *   K, V       16, 32, 64 or 128 each
 *
 * Equal, up to float32 rounding, to gdn_chunk_fwd with T = 1 and
 * final_state == initial_state == state.  Arithmetic is float32 in a fixed order
 * (bitwise reproducible).  No buffer may overlap another.  Errors as for
 * gdn_chunk_fwd.
 */
GDN_API gdn_status_t gdn_decode_step(const void *q, const void *k, const void *v,
                             const float *alpha, const float *beta, float *state,
                             void *o, int64_t B, int64_t H, int64_t K, int64_t V,
                             gdn_dtype_t dtype, void *stream);

/*
 * gdn_chunk_bwd_workspace_size -- bytes of device workspace gdn_chunk_bwd needs
 * for these sizes and this dtype (the layout of the path the call takes).
 *  - bfloat16 with K and V in {32, 64, 128}: the MFMA path with 64-token chunks,
 *    whatever `chunk` is; per (batch, head, chunk) two [V, K] states rounded to
 *    bfloat16 (the chunk-start state and the state gradient, kept in the precision
 *    the path's matrix products read them in) and a 16896-byte record (two bf16
 *    64 x 64 matrices, two float32 64-vectors):
 *        B * H * ceil(T / 64) * (2 * V * K * 2 + 16896) bytes.
 *  - otherwise (float32, or bfloat16 with K or V = 16): the float32 path, per
 *    (batch, head, backward chunk of C = min(chunk, 32) tokens) two float32
 *    [V, K] states and the chunk's float32 factors (three C x C matrices and
 *    three C-vectors):
 *        B * H * ceil(T / C) * (2 * V * K + 3 * C * C + 3 * C) * 4 bytes,
 *    and for float32 inputs also the per-chunk records of the matrix-core state
 *    recompute, R(C) = (C/16) (C/16 + 1) * 256 + 2 C + 4 floats each (1604 at
 *    C = 32, 548 at C = 16):
 *        + B * H * ceil(T / C) * R(C) * 4 bytes.
 * Returns 0 when a size is not positive or the dtype is not F32 or BF16.
 */
GDN_API size_t gdn_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t K,
                                            int64_t V, int64_t chunk, gdn_dtype_t dtype);

/*
 * gdn_chunk_bwd -- reverse mode of gdn_chunk_fwd for the loss
 *     L = sum(o * d_o) + sum(final_state * d_final_state).
 *
 *   q, k, v, alpha, beta, initial_state   as for gdn_chunk_fwd (read only)
 *   d_o            [B,T,H,V] dtype        gradient of o (read only)
 *   d_final_state  [B,H,V,K] float32      gradient of final_state, or NULL for zeros
 *   dq, dk         [B,T,H,K] dtype        dL/dq, dL/dk (written)
 *   dv             [B,T,H,V] dtype        dL/dv (written)
 *   dalpha, dbeta  [B,T,H]   float32      dL/dalpha, dL/dbeta with respect to the
 *                                         gates themselves (written)
 *   d_initial_state [B,H,V,K] float32     dL/dinitial_state, or NULL to skip
 *   workspace      device scratch of workspace_bytes >=
 *                  gdn_chunk_bwd_workspace_size(B, T, H, K, V, chunk, dtype);
 *                  owned by the caller, contents undefined after the call
 *   B .. dtype, stream                    as for gdn_chunk_fwd
 *
 * The chunk-start states are recomputed from the inputs (nothing is kept from a
 * forward call), the chunks are walked in reverse to carry the state gradient,
 * and every chunk then forms its token gradients from its two boundary states:
 * "OpenGDN 0.1.0", section "Core operator reference" (backward from recomputed
 * fp32 chunk-boundary states) and "Sparse Delta Memory: layer and kernels",
 * sections "What the layer computes" and "Execution" (the backward walks the
 * chunks in reverse).  Float32 inputs: all arithmetic float32.  Bfloat16 inputs
 * with K, V in {32, 64, 128}: 64-token chunks whatever `chunk` is (the chunk size
 * changes results only by rounding), matrix products on bf16 MFMA with bf16
 * operands and float32 accumulation, everything else float32 (K or V = 16: the
 * float32 path).  Every sum has a fixed order,
 * so results are bitwise reproducible; dq, dk, dv are rounded to dtype once.
 * All work is enqueued on `stream` alone (three launches on both matrix-core
 * paths, bf16 and float32 with V a multiple of 32: the two independent
 * sequential walks share the second one).  No output may
 * overlap any other buffer (inputs, other outputs, workspace).  Errors as for
 * gdn_chunk_fwd; a workspace smaller than required is GDN_ERROR_INVALID_VALUE.
 */
GDN_API gdn_status_t gdn_chunk_bwd(const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta,
                           const float *initial_state,
                           const void *d_o, const float *d_final_state,
                           void *dq, void *dk, void *dv,
                           float *dalpha, float *dbeta, float *d_initial_state,
                           void *workspace, size_t workspace_bytes,
                           int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                           int64_t chunk, gdn_dtype_t dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
