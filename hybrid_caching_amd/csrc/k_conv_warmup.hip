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
// Width 4 (the usual short convolution) with W - 1 + n_warm <= 16: one thread
// per (batch row, entry, four channels of a head) loads the entry's whole tap
// window -- its W - 1 history inputs and n_warm head inputs -- into registers
// at once, a single memory round trip after the entry's three table reads,
// and forms the n_warm outputs from them.  Other widths: a thread owns four
// channels of one head, keeps their taps in registers and walks 32 output
// tokens (weights are read once per 32 tokens, not per token), gathering each
// output's taps from the head or the history.  Absent history reads as zero;
// accumulation in fp32; the result is stored in the input's type (bf16
// rounded to nearest even).
#include "pic_internal.hpp"

namespace pic {
namespace {

constexpr int kMaxConv = 16;  // widest convolution (the header's limit)

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

constexpr int kRows = 32;  // output tokens per block

template <bool BF16>
__global__ __launch_bounds__(256) void conv_warmup_kernel(ConvArgs a, int item_blocks) {
  // a thread owns four channels of one head and its taps (in registers) and
  // walks kRows output tokens (layer, entry, t)
  const int g4 = a.dc / 4, items = a.heads * g4;
  const int it = (blockIdx.x % item_blocks) * 256 + threadIdx.x;
  if (it >= items) return;
  const int h = it / g4, c = 4 * (it - h * g4);
  float w[kMaxConv][4];
#pragma unroll
  for (int j = 0; j < kMaxConv; ++j)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w[j][u] = (j < a.width) ? a.weight[(int64_t(h) * a.dc + c + u) * a.width + j] : 0.f;
  const int64_t per_b = int64_t(a.n) * a.n_warm, rows = int64_t(a.batch) * per_b;
  const int64_t r0 = int64_t(blockIdx.x / item_blocks) * kRows;
  const int64_t r1 = r0 + kRows < rows ? r0 + kRows : rows;
  for (int64_t rr = r0; rr < r1; ++rr) {
    const int b = int(rr / per_b);
    const int64_t row = rr - int64_t(b) * per_b;  // entry * n_warm + t
    const int e = int(row / a.n_warm), t = int(row - int64_t(e) * a.n_warm);
    const int64_t head = table_at(a.d_head_start, e), hend = table_at(a.d_hist_end, e);
    const int hlen = table_at(a.d_hist_len, e);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxConv; ++j) {
      const int tau = t - j;
      // taps past the width, and history taps past the history, read nothing
      if (j < a.width && (tau >= 0 || -tau <= hlen)) {
        const int64_t src = (tau >= 0) ? head + tau : hend + tau;
        const float4 xv =
            load4<BF16>(a.x, ((int64_t(b) * a.n_tokens + src) * a.heads + h) * a.dc + c);
        acc[0] = fmaf(w[j][0], xv.x, acc[0]);
        acc[1] = fmaf(w[j][1], xv.y, acc[1]);
        acc[2] = fmaf(w[j][2], xv.z, acc[2]);
        acc[3] = fmaf(w[j][3], xv.w, acc[3]);
      }
    }
    const int64_t o = (rr * a.heads + h) * a.dc + c;
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

constexpr int kSpan = 16;  // window positions held in registers (width 4), at most

template <bool BF16>
__device__ __forceinline__ void store4(void* y, int64_t o, const float (&acc)[4]) {
  if constexpr (BF16) {
    const uint2 u = make_uint2(bf16_bits(acc[0]) | (bf16_bits(acc[1]) << 16),
                               bf16_bits(acc[2]) | (bf16_bits(acc[3]) << 16));
    *reinterpret_cast<uint2*>(static_cast<__bf16*>(y) + o) = u;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(y) + o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
}

// width 4: window position i holds input tau = i - 3 of the entry (tau < 0:
// history token hist_end + tau, present when -tau <= hist_len; tau >= 0: head
// token head_start + tau), and output t = sum_{m < 4} w_(3-m) z[t + m];
// KZ positions (6 for the usual n_warm = 3, else kSpan)
template <bool BF16, int KZ>
__global__ __launch_bounds__(256) void conv_warmup_w4_kernel(ConvArgs a, int item_blocks) {
  constexpr int KW = 4;
  const int g4 = a.dc / 4, items = a.heads * g4;
  const int it = (blockIdx.x % item_blocks) * 256 + threadIdx.x;
  if (it >= items) return;
  const int64_t be = blockIdx.x / item_blocks;  // (batch row, entry)
  const int b = int(be / a.n), e = int(be - int64_t(b) * a.n);
  const int h = it / g4, c = 4 * (it - h * g4);
  const int nw = a.n_warm;
  const int64_t head = table_at(a.d_head_start, e), hend = table_at(a.d_hist_end, e);
  const int hlen = table_at(a.d_hist_len, e);
  const int64_t ts = int64_t(a.heads) * a.dc;  // elements from one token to the next
  const int64_t xb = int64_t(b) * a.n_tokens * ts + int64_t(h) * a.dc + c;
  // every position is loaded (absent ones from the first head token, a valid
  // address) and the absent ones then zeroed, so that no load is conditional
  float4 z[KZ];
#pragma unroll
  for (int i = 0; i < KZ; ++i) {
    const int tau = i - (KW - 1);
    const bool ok = tau < nw && (tau >= 0 || -tau <= hlen);
    const int64_t src = !ok ? head : (tau >= 0 ? head + tau : hend + tau);
    const float4 v = load4<BF16>(a.x, xb + src * ts);
    z[i] = ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // taps of channels c .. c+3: 16 consecutive floats ([heads][dc][4])
  const float4* wp = reinterpret_cast<const float4*>(a.weight + (int64_t(h) * a.dc + c) * KW);
  float wr[KW][4];  // wr[m][u]: tap j = 3 - m of channel c + u
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float4 w4 = wp[u];
    wr[3][u] = w4.x;
    wr[2][u] = w4.y;
    wr[1][u] = w4.z;
    wr[0][u] = w4.w;
  }
  const int64_t row0 = int64_t(b) * a.n * nw + int64_t(e) * nw;  // output row of t = 0
#pragma unroll
  for (int t = 0; t + KW <= KZ; ++t) {
    if (t < nw) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KW; ++m) {
        acc[0] = fmaf(wr[m][0], z[t + m].x, acc[0]);
        acc[1] = fmaf(wr[m][1], z[t + m].y, acc[1]);
        acc[2] = fmaf(wr[m][2], z[t + m].z, acc[2]);
        acc[3] = fmaf(wr[m][3], z[t + m].w, acc[3]);
      }
      store4<BF16>(a.y, ((row0 + t) * a.heads + h) * a.dc + c, acc);
    }
  }
}

}  // namespace

hipError_t launch_conv_warmup(const ConvArgs& a, hipStream_t s) {
  const int64_t rows = int64_t(a.batch) * a.n * a.n_warm;  // output tokens
  if (rows <= 0 || a.heads <= 0 || a.dc <= 0) return hipSuccess;
  const int item_blocks = (a.heads * (a.dc / 4) + 255) / 256;
  const int64_t blocks = (rows + kRows - 1) / kRows * item_blocks;
  if (a.dc % 4 || a.width > kMaxConv || blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int64_t w4_blocks = int64_t(a.batch) * a.n * item_blocks;
  if (a.width == 4 && a.n_warm >= 1 && a.n_warm + 3 <= kSpan && w4_blocks <= 0x7fffffffLL) {
    const dim3 grid{unsigned(w4_blocks), 1, 1};
    if (a.n_warm == 3) {
      if (a.bf16)
        hipLaunchKernelGGL((conv_warmup_w4_kernel<true, 6>), grid, dim3(256), 0, s, a, item_blocks);
      else
        hipLaunchKernelGGL((conv_warmup_w4_kernel<false, 6>), grid, dim3(256), 0, s, a, item_blocks);
    } else if (a.bf16) {
      hipLaunchKernelGGL((conv_warmup_w4_kernel<true, kSpan>), grid, dim3(256), 0, s, a, item_blocks);
    } else {
      hipLaunchKernelGGL((conv_warmup_w4_kernel<false, kSpan>), grid, dim3(256), 0, s, a, item_blocks);
    }
    return hipGetLastError();
  }
  if (a.bf16)
    hipLaunchKernelGGL(conv_warmup_kernel<true>, dim3(unsigned(blocks)), dim3(256), 0, s, a, item_blocks);
  else
    hipLaunchKernelGGL(conv_warmup_kernel<false>, dim3(unsigned(blocks)), dim3(256), 0, s, a, item_blocks);
  return hipGetLastError();
}

}  // namespace pic
