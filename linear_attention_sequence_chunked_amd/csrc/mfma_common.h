// Building blocks for bf16 MFMA kernels on gfx950 (MI355X): operand fragments
// of v_mfma_f32_16x16x32_bf16 from LDS (row reads and ds_read_b64_tr_b16
// transpose reads), accumulator tiles back to LDS or straight into operand
// layout (permlane swaps), an LDS-only workgroup barrier and a wavefront scan.
//
// MFMA 16x16x32 bf16 layout: operand fragments hold 16 rows x 32 k; lane
// (g = lane / 16, s = lane % 16) has row s, k = 8g .. 8g + 7.  The 16 x 16 fp32
// accumulator gives lane (g, s) rows 4g .. 4g + 3 of column s.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {
namespace mfma {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef bf16x4 __attribute__((address_space(3))) lds_bf16x4;
typedef bf16x8 __attribute__((address_space(3))) lds_bf16x8;
typedef bf16 __attribute__((address_space(3))) lbf16;
typedef float __attribute__((address_space(3))) lf32;
typedef f32x4 __attribute__((address_space(3))) lf32x4;

// LDS pointer with a per-lane part, made opaque to the optimiser: every access
// of a tile is then this register plus a constant in the instruction's offset
// field, instead of one precomputed address register (and one add per chunk)
// per access.
template <typename T>
__device__ __forceinline__ T* pin(T* p) {
  asm volatile("" : "+v"(p));
  return p;
}
template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds(T* p) {
  return (__attribute__((address_space(3))) T*)p;
}
__device__ __forceinline__ bf16x8 ld8(const lbf16* p) { return *reinterpret_cast<const lds_bf16x8*>(p); }
__device__ __forceinline__ bf16x4 tr4(const lbf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}
// MFMA operand from a [k][row] array through a base that already holds the
// lane part (row k0 + 8g + s/4, column 4(s%4)): two transpose reads.
__device__ __forceinline__ bf16x8 frag_cols_at(const lbf16* cb, int ld, int r0, int k0) {
  const bf16x4 lo = tr4(cb + k0 * ld + r0), hi = tr4(cb + (k0 + 4) * ld + r0);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ int cols_lane(int ld, int lane) {
  return (8 * (lane >> 4) + ((lane & 15) >> 2)) * ld + 4 * (lane & 3);
}
__device__ __forceinline__ int rows_lane(int ld, int lane) { return (lane & 15) * ld + 8 * (lane >> 4); }


__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = (bf16)0.0f;
  return z;
}

__device__ __forceinline__ bf16x4 tr_read(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

// Operand fragment of rows r0..r0+15, k0..k0+31 from a row-major [row][k] array
// (leading dimension ld): lane (g = lane/16, s = lane%16) receives row r0 + s,
// k = k0 + 8g .. k0 + 8g + 7.
__device__ __forceinline__ bf16x8 frag_rows(const bf16* base, int ld, int r0, int k0, int lane) {
  return *reinterpret_cast<const bf16x8*>(base + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

// The same fragment from a [k][row] array by transpose reads.  Within each
// 16-lane group the hardware gives lane 4a+c the c-th 16-bit element read by
// lanes a, a+4, a+8, a+12; so source lane s points at row k0 + 8g + s/4,
// column r0 + 4(s%4), and a second read covers k + 4.
__device__ __forceinline__ bf16x8 frag_cols(const bf16* base, int ld, int r0, int k0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const bf16* p = base + (k0 + 8 * g + (s >> 2)) * ld + r0 + 4 * (s & 3);
  const bf16x4 lo = tr_read(p), hi = tr_read(p + 4 * ld);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// 16-deep products: lanes that would hold k in [16, 32) read their partner's
// (valid) rows and are zeroed, so the 32-deep MFMA adds exact zeros.
__device__ __forceinline__ bf16x8 frag_rows16(const bf16* base, int ld, int r0, int k0, int lane) {
  const bf16x8 f = frag_rows(base, ld, r0, k0 - 16 * ((lane >> 5) & 1), lane);
  return (lane >> 5) ? zero8() : f;
}
__device__ __forceinline__ bf16x8 frag_cols16(const bf16* base, int ld, int r0, int k0, int lane) {
  const bf16x8 f = frag_cols(base, ld, r0, k0 - 16 * ((lane >> 5) & 1), lane);
  return (lane >> 5) ? zero8() : f;
}

// Key and query tiles: row-major [token][channel] with 8 elements of padding
// per row (row stride KD + 8).  A 16-byte fragment read by 16 lanes of
// consecutive rows then covers all 64 banks, and every fragment of a tile is a
// constant offset from one per-lane base address (no per-read address math).
// swz gives the element offset of (row, col) in such a tile.
template <int KD>
__device__ __forceinline__ int swz(int row, int col) {
  return row * (KD + 8) + col;
}
// Accumulator tile (lane holds rows 4g..4g+3 of column s) stored transposed:
// dst[(c0 + s) * ld + r0 + 4g + e] = d[e], as bf16.
__device__ __forceinline__ void store_tile_t(bf16* base, int ld, int c0, int r0, f32x4 d, int lane) {
  const int s = lane & 15, g = lane >> 4;
  *reinterpret_cast<bf16x4*>(base + (c0 + s) * ld + r0 + 4 * g) =
      bf16x4{(bf16)d[0], (bf16)d[1], (bf16)d[2], (bf16)d[3]};
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every
// outstanding global load and store (a workgroup-scope fence on all memory),
// which would stall the prefetch of the next chunks at every barrier; no data
// passes between the waves of a workgroup through global memory here.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Two accumulator tiles a (rows 0..15) and b (rows 16..31) of the same 16
// columns -> the MFMA operand whose k index is their row (k = 8g + j for lane
// group g), without LDS.  Each lane packs its 4 rows (4g..4g+3) of a tile into
// two bf16-pair dwords; viewing a wave as four 16-lane rows [x0 x1 x2 x3],
// permlane32_swap(a, b) gives ([a0 a1 b0 b1], [a2 a3 b2 b3]) and permlane16_swap
// of that pair gives ([a0 a2 b0 b2], [a1 a3 b1 b3]): group g then holds rows
// 8g..8g+3 and 8g+4..8g+7, the operand layout.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int pack2(float x, float y) {
  typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(int, bf16x2{(bf16)x, (bf16)y});
}
__device__ __forceinline__ bf16x8 acc_pair_to_frag(f32x4 a, f32x4 b) {
  const i32x2 s_lo = __builtin_amdgcn_permlane32_swap(pack2(a[0], a[1]), pack2(b[0], b[1]), false, false);
  const i32x2 s_hi = __builtin_amdgcn_permlane32_swap(pack2(a[2], a[3]), pack2(b[2], b[3]), false, false);
  const i32x2 t_lo = __builtin_amdgcn_permlane16_swap(s_lo[0], s_lo[1], false, false);
  const i32x2 t_hi = __builtin_amdgcn_permlane16_swap(s_hi[0], s_hi[1], false, false);
  return __builtin_bit_cast(bf16x8, i32x4{t_lo[0], t_hi[0], t_lo[1], t_hi[1]});
}

// The same two tiles as an operand without moving data between lanes: lane
// group g keeps rows 4g..4g+3 of a, then of b, as its eight k values, so the
// operand's k order is {4g..4g+3, 16+4g..16+4g+3} ("tau order").  The other
// operand of that product must take its k in the same order: frag_cols_tau_at
// below, or, for the key channels of the state, the channel order the state
// rows are kept in.
__device__ __forceinline__ bf16x8 acc_pair_pack(f32x4 a, f32x4 b) {
  return __builtin_bit_cast(bf16x8, i32x4{pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(b[0], b[1]), pack2(b[2], b[3])});
}
// Lane part of a tau-order operand read from a [k][row] array: row 4g + s/4,
// column cstep * (s % 4) (cstep 4 for consecutive rows of the operand).
__device__ __forceinline__ int cols_lane_tau(int ld, int lane, int cstep) {
  return (4 * (lane >> 4) + ((lane & 15) >> 2)) * ld + cstep * (lane & 3);
}
// Operand from a [k][row] array with k in tau order: transpose reads of rows
// k0 + 4g + s/4 and k0 + 16 + 4g + s/4 (base from cols_lane_tau).
__device__ __forceinline__ bf16x8 frag_cols_tau_at(const lbf16* cb, int ld, int r0, int k0) {
  const bf16x4 lo = tr4(cb + k0 * ld + r0), hi = tr4(cb + (k0 + 16) * ld + r0);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ float bits_f(int x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ int f_bits(float x) { return __builtin_bit_cast(int, x); }

// Inclusive prefix sum over the 64 lanes of a wavefront, in a fixed order:
// shifts 1, 2, 4, 8 inside each 16-lane row (DPP), then the row totals.
__device__ __forceinline__ float wave_scan(float x, int lane) {
  x += bits_f(__builtin_amdgcn_update_dpp(0, f_bits(x), 0x111, 0xf, 0xf, false));
  x += bits_f(__builtin_amdgcn_update_dpp(0, f_bits(x), 0x112, 0xf, 0xf, false));
  x += bits_f(__builtin_amdgcn_update_dpp(0, f_bits(x), 0x114, 0xf, 0xf, false));
  x += bits_f(__builtin_amdgcn_update_dpp(0, f_bits(x), 0x118, 0xf, 0xf, false));
  const float t0 = bits_f(__builtin_amdgcn_readlane(f_bits(x), 15));
  const float t1 = bits_f(__builtin_amdgcn_readlane(f_bits(x), 31));
  const float t2 = bits_f(__builtin_amdgcn_readlane(f_bits(x), 47));
  const int row = lane >> 4;
  const float add = row == 0 ? 0.0f : (row == 1 ? t0 : (row == 2 ? t0 + t1 : (t0 + t1) + t2));
  return x + add;
}

}  // namespace mfma
}  // namespace gdn
