// k_conv_warmup.hip -- convolution warm-up for variants with a short causal
// depthwise convolution of width W in front of the linear layer.
// [xix.ai HYPIC article (French), paragraph on linear layers: variants with a
//  short convolution need the convolution state warmed up.]
//
// The conv output of token t, y_t = sum_{j<W} w_j x_(t-j) per channel, reads
// the W-1 raw inputs before t, so a segment's first W-1 outputs depend on the
// segment before it and cannot be cached position-independently.  On reuse
// they are recomputed here, from the segment's head and the previous
// segment's raw tail, into the seam layout [B][n * n_warm][H][dc] that the
// seam compose takes; the cached pair covers the tokens after them.
//
// One thread per four output channels; the taps are gathered from the head or
// the history (absent history reads as zero) and accumulated in fp32; the
// result is stored in the input's type (bf16 rounded to nearest even).
#include <algorithm>

#include "pic_internal.hpp"

namespace pic {
namespace {

template <bool BF16>
__device__ __forceinline__ float4 load4(const void* x, int64_t off) {
  if constexpr (BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const __bf16*>(x) + off);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
  }
}

__device__ __forceinline__ unsigned bf16_bits(float f) {
  const unsigned u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;  // nearest even (finite inputs)
}

template <bool BF16>
__global__ __launch_bounds__(256) void conv_warmup_kernel(ConvArgs a) {
  const int g4 = a.dc / 4;
  const int64_t total = int64_t(a.batch) * a.n * a.n_warm * a.heads * g4;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int c = 4 * int(i % g4);
    int64_t r = i / g4;
    const int h = int(r % a.heads);
    r /= a.heads;
    const int64_t row = r % (int64_t(a.n) * a.n_warm);  // entry * n_warm + t
    const int b = int(r / (int64_t(a.n) * a.n_warm));
    const int e = int(row / a.n_warm), t = int(row % a.n_warm);
    const int64_t head = table_at(a.d_head_start, e), hend = table_at(a.d_hist_end, e);
    const int hlen = table_at(a.d_hist_len, e);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const float* w = a.weight + (int64_t(h) * a.dc + c) * a.width;
    for (int j = 0; j < a.width; ++j) {
      const int tau = t - j;
      int64_t src;
      if (tau >= 0)
        src = head + tau;
      else if (-tau <= hlen)
        src = hend + tau;
      else
        continue;
      const float4 xv = load4<BF16>(a.x, ((int64_t(b) * a.n_tokens + src) * a.heads + h) * a.dc + c);
      acc[0] = fmaf(w[j], xv.x, acc[0]);
      acc[1] = fmaf(w[a.width + j], xv.y, acc[1]);
      acc[2] = fmaf(w[2 * a.width + j], xv.z, acc[2]);
      acc[3] = fmaf(w[3 * a.width + j], xv.w, acc[3]);
    }
    const int64_t o = ((int64_t(b) * a.n * a.n_warm + row) * a.heads + h) * a.dc + c;
    if constexpr (BF16) {
      const uint2 u = make_uint2(bf16_bits(acc[0]) | (bf16_bits(acc[1]) << 16),
                                 bf16_bits(acc[2]) | (bf16_bits(acc[3]) << 16));
      *reinterpret_cast<uint2*>(static_cast<__bf16*>(a.y) + o) = u;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.y) + o) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

}  // namespace

hipError_t launch_conv_warmup(const ConvArgs& a, hipStream_t s) {
  const int64_t total = int64_t(a.batch) * a.n * a.n_warm * a.heads * (a.dc / 4);
  if (total <= 0) return hipSuccess;
  if (a.dc % 4) return hipErrorInvalidConfiguration;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  if (a.bf16)
    hipLaunchKernelGGL(conv_warmup_kernel<true>, dim3(unsigned(blocks)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(conv_warmup_kernel<false>, dim3(unsigned(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pic
