// stage_util.hpp -- LDS layouts shared by the dense build kernels: the token
// order inside K-dimensions, the XOR swizzle of transposed rows, and the
// packing of two tokens' 16-bit elements into one 32-bit word.
#pragma once

#include <hip/hip_runtime.h>

namespace pic {

// Storage position of token t inside a token-indexed K dimension: bits 2 and
// 3 swapped, so that positions 8g .. 8g+7 of every 16 hold tokens
// 4g + {0..3} and 4g + 8 + {0..3} -- the row order of an MFMA accumulator
// half used as a B operand (kperm in mfma_util.hpp).  tpos is an involution.
__device__ __forceinline__ int tpos(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

// (16-bit element j of token a, element j of token b) as one 32-bit word
__device__ __forceinline__ unsigned ws_pair(const uint4& a, const uint4& b, int j) {
  const unsigned wa = (j < 2) ? a.x : (j < 4) ? a.y : (j < 6) ? a.z : a.w;
  const unsigned wb = (j < 2) ? b.x : (j < 4) ? b.y : (j < 6) ? b.z : b.w;
  return __builtin_amdgcn_perm(wb, wa, (j & 1) ? 0x07060302u : 0x05040100u);
}

__device__ __forceinline__ uint4 ws_pick(bool ok, uint4 x) {
  return make_uint4(ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u, ok ? x.w : 0u);
}

// Element offset of 16-byte chunk `chunk` of row `row` in a transposed
// (channel-major) K^T / V^T buffer with row stride LD: the chunks of a row
// are XOR-swizzled by the row's 8-row group, so that the transposed writes of
// staging spread over the LDS banks; readers apply the same swizzle.
template <int LD>
__device__ __forceinline__ int kt_at(int row, int chunk) {
  return row * LD + 8 * (chunk ^ ((row >> 3) & 7));
}

// The same offset for rows 32 t + cl read by lane (g, cl) at chunk
// 4 s + 2 hh + g: the swizzle only flips bits of the chunk index, so it is a
// per-lane base for each half hh plus a constant for (t, s).
template <int LD>
__device__ __forceinline__ int kt_lane_base(int cl, int g, int hh) {
  return cl * LD + 8 * (g ^ ((cl >> 3) & 1)) + 16 * (hh ^ ((cl >> 4) & 1));
}
template <int LD>
__device__ __forceinline__ int kt_tile(int t, int s) {
  return 32 * t * LD + 32 * (s ^ (t & 1));
}

// a copy of v the compiler cannot see through: keeps per-lane address
// arithmetic inside a loop instead of holding it in registers across it
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

}  // namespace pic
