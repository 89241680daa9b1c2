// mfma_util.hpp -- small device helpers for CDNA4 (gfx950) matrix cores.
//
// Lane layouts of v_mfma_f32_32x32x16_bf16 (wave of 64 lanes, g = lane / 32):
//   A (32 x 16): lane holds A[lane % 32][8 g + j], j = 0..7
//   B (16 x 32): lane holds B[8 g + j][lane % 32], j = 0..7
//   D (32 x 32): lane holds D[8 (r / 4) + 4 g + (r % 4)][lane % 32], r = 0..15
//
// Feeding an accumulator back as the B operand.  Because the contraction
// order does not matter, a K-step may use any 16 rows as long as A and B agree
// on the permutation.  For the rows held by accumulator registers
// r0 .. r0+7 (r0 = 0 or 8) of a 32-row tile, lane group g holds rows
//   16 (r0 / 8) + 4 g + {0,1,2,3}   and   16 (r0 / 8) + 8 + 4 g + {0,1,2,3}.
// So with  kperm(h, g, j) = 16 h + 4 g + (j % 4) + 8 (j / 4)  (h = r0 / 8),
// B-operand element j of the lane is simply accumulator register 8 h + j,
// and the A operand must take its column kperm(h, g, j).
//
// Split precision ("bf16x3").  An fp32 value x is split as hi = bf16(x),
// lo = bf16(x - hi) (x - hi is exact in fp32).  A product of two fp32
// operands is formed as hi*hi + hi*lo + lo*hi: every partial product is
// exact in fp32 and the dropped terms are ~2^-16 relative.  When one operand
// is exactly representable in bf16 (bf16 inputs), its lo part is zero and
// two MFMAs suffice ("bf16x2").
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pic {

// Gates are handled in base 2 (log2 / exp2): sums of log2(alpha) are exact
// for power-of-two gates, and lambda is converted to natural log once, at
// the end of a build.
constexpr float kLn2 = 0.693147180559945309f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// row of accumulator register r for lane group g (32x32 tile)
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// permuted K index for B-from-accumulator steps (see header comment)
__device__ __forceinline__ int kperm(int h, int g, int j) {
  return 16 * h + 4 * g + (j & 3) + 8 * (j >> 2);
}

__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }
__device__ __forceinline__ float from_bf16(__bf16 x) { return static_cast<float>(x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// split a pair: hi = bf16(x) (round to nearest even, one packed convert),
// unpacked back to fp32 by shift / mask, lo = bf16(x - hi) (x - hi exact)
__device__ __forceinline__ void split2(float x0, float x1, unsigned& hp, unsigned& lp) {
  const bf16x2 h = __builtin_convertvector((f32x2){x0, x1}, bf16x2);
  hp = __builtin_bit_cast(unsigned, h);
  const float h0 = __uint_as_float(hp << 16), h1 = __uint_as_float(hp & 0xffff0000u);
  lp = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x0 - h0, x1 - h1}, bf16x2));
}

// split 8 fp32 values into hi/lo bf16 parts
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
  unsigned h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) split2(x[2 * j], x[2 * j + 1], h[j], l[j]);
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  hi = __builtin_bit_cast(bf16x8, (u32x4){h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, (u32x4){l[0], l[1], l[2], l[3]});
}

// B operand (hi/lo) from accumulator registers 8h .. 8h+7 of a tile
__device__ __forceinline__ void split_acc_half(const f32x16& acc, int h, bf16x8& hi, bf16x8& lo) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = acc[8 * h + j];
  split8(x, hi, lo);
}

__device__ __forceinline__ unsigned short bf16_bits(__bf16 x) {
  return __builtin_bit_cast(unsigned short, x);
}
__device__ __forceinline__ __bf16 bits_bf16(unsigned short x) {
  return __builtin_bit_cast(__bf16, x);
}

// load 4 consecutive bf16 values (8 bytes) from LDS
__device__ __forceinline__ bf16x4 lds_load4(const __bf16* p) {
  return *reinterpret_cast<const bf16x4*>(p);
}

// gather an A-operand fragment for a permuted K-step from a row-major bf16
// matrix in LDS: columns c0 + {0..3} and c0 + 8 + {0..3}
__device__ __forceinline__ bf16x8 lds_perm8(const __bf16* row, int c0) {
  bf16x4 a = lds_load4(row + c0);
  bf16x4 b = lds_load4(row + c0 + 8);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// v from another lane by a DPP pattern; lanes without a source (or in rows
// outside ROW_MASK) get 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum of s over aligned groups of N lanes (N = 1, 2, 4 or 8), every lane of
// the group receiving the sum; lane exchanges on DPP (no LDS round trip).
template <int N>
__device__ __forceinline__ float group_sum(float s) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "group of 1, 2, 4 or 8 lanes");
  if (N >= 2) s += dpp_f<0xB1>(s);   // partner lane ^ 1: quad_perm(1, 0, 3, 2)
  if (N >= 4) s += dpp_f<0x4E>(s);   // partner lane ^ 2: quad_perm(2, 3, 0, 1)
  if (N >= 8) s += dpp_f<0x141>(s);  // lane 7 - i of each half-row: the other quad
  return s;
}

// Inclusive prefix sum over the 64 lanes of a wave on DPP: shifts by
// 1, 2, 4, 8 inside each row of 16 lanes, then row broadcasts of lanes 15
// and 31 into the later rows.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x += dpp_f<0x111>(x);         // row_shr:1
  x += dpp_f<0x112>(x);         // row_shr:2
  x += dpp_f<0x114>(x);         // row_shr:4
  x += dpp_f<0x118>(x);         // row_shr:8
  x += dpp_f<0x142, 0xA>(x);    // row_bcast:15 into rows 1 and 3
  x += dpp_f<0x143, 0xC>(x);    // row_bcast:31 into rows 2 and 3
  return x;
}

// Inclusive prefix sum inside each half wave (lanes 0-31 and 32-63): the
// steps of wave_inclusive_scan without the broadcast across halves.
__device__ __forceinline__ float half_wave_scan(float x) {
  x += dpp_f<0x111>(x);        // row_shr:1
  x += dpp_f<0x112>(x);        // row_shr:2
  x += dpp_f<0x114>(x);        // row_shr:4
  x += dpp_f<0x118>(x);        // row_shr:8
  x += dpp_f<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
  return x;
}

// 8 consecutive bf16 (16 bytes) from LDS
__device__ __forceinline__ bf16x8 lds_load8(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

}  // namespace pic
