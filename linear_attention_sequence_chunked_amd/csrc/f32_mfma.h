// Shared pieces of the float32 matrix-core kernels (forward and backward walks):
// the 16-deep fp32 product in one fixed lane layout and the per-(chunk, head)
// record the chunk-parallel launch writes.
//
// Operand layout of v_mfma_f32_16x16x4_f32: lane (g = lane / 16, s = lane % 16)
// supplies A[s][g] and B[g][s]; the accumulator gives lane (g, s) rows
// 4g .. 4g + 3 of column s.  mma16 runs four of them with lane (g, s) holding a
// float4 A[s][4g .. 4g + 3] and B[4g .. 4g + 3][s], product j taking element j of
// both, which contracts over 16 k in all; an accumulator tile is then, as it
// stands, the right operand of a 16-deep product.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {
namespace f32mfma {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x4 a, f32x4 b, f32x4 c) {
  c = mma4(a[0], b[0], c);
  c = mma4(a[1], b[1], c);
  c = mma4(a[2], b[2], c);
  return mma4(a[3], b[3], c);
}
__device__ __forceinline__ f32x4 zero4f() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }

// Record of one (chunk, head): the lower 16 x 16 blocks of Tm diag(beta), then
// those of P, each block 256 floats row-major and block (I, J <= I) at index
// I (I + 1) / 2 + J, so that a wave's float4 operand load of a block is one
// contiguous kilobyte; then gam_t = 2^g_t [C], dn_t = 2^(g_n - g_t) [C] and 2^g_n
// (padded to 4 floats).  With beta folded into Tm the walk forms
// U = (Tm diag(beta)) (V - diag(gam) X).  record_floats is the one definition of
// the record size, used by the kernels and by the host's allocation alike.
constexpr int record_blocks(int C) { return (C / 16) * (C / 16 + 1) / 2; }
constexpr int record_floats(int C) { return 2 * record_blocks(C) * 256 + 2 * C + 4; }
template <int C>
struct Rec {
  static constexpr int kTm = 0, kP = record_blocks(C) * 256, kGam = 2 * record_blocks(C) * 256,
                       kDn = kGam + C, kGn = kGam + 2 * C;
  static constexpr int kFloats = record_floats(C);
  static_assert(kGn + 4 == kFloats, "record layout");
  // offset of element (r, c) of lower block (I, J)
  static __device__ __forceinline__ int at(int I, int J, int r, int c) {
    return (I * (I + 1) / 2 + J) * 256 + r * 16 + c;
  }
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// Packed batch: sequence b is tokens [cl(cu[b]), cl(max(cu[b+1], cu[b]))) with
// offsets clamped into [0, T].  Its chunk c has record slot cl(cu[b]) / C + b + c:
// distinct for distinct (b, c) and below T / C + B + 1.
__device__ __forceinline__ void packed_seq(const int* cu, int b, int T, int& s, int& e) {
  s = clampi(cu[b], 0, T);
  e = clampi(max(cu[b + 1], s), s, T);
}


}  // namespace f32mfma
}  // namespace gdn
