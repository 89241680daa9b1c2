// k_compose_seam.hip -- reuse with seam windows.  Along a chain of cached
// pairs, each entry first advances the running state through its seam tokens
// one token at a time, writing o_t = S_t^T q_t after each, and then applies the
// entry's pair:  S <- e^lambda That S + S0  (dense: split-bf16 matrix-core
// products, as in the dense compose; scalar / diagonal: one scale per head or
// per key row).
// [xix.ai HYPIC article (French), paragraph on full-attention layers: the
//  first w tokens (8 by default) of every inner segment are kept out of the
//  cache and recomputed on reuse under the full prefix; the linear layers run
//  the running state through them and pass each token's output to the
//  attention layer above.  Paragraph on linear layers: applying a cached pair
//  left-multiplies the state by T_C and adds S(C|0).]
//
// One workgroup of four waves per (request, layer, head).  Wave w owns columns
// [32w, 32w+32) of the state in 32x32 accumulator layout: lane (g, c) holds
// column 32w + c, rows 32t + 8i + 4g + {0..3} of tile t.  A seam token is a
// rank-one update in fp32 on the vector units:
//   dense     u = S^T k,  S <- a S + k (b (v - a u))^T
//   scalar    S <- a S + k v^T
//   diagonal  S <- Diag(a) S + k v^T
// A lane holds half of each of its column's rows, so the column sums S^T k
// and S^T q take a partial sum over its 64 rows and one exchange with lane
// l ^ 32.  Seam tokens are staged in LDS a few at a time (fp32, zero padded
// to 128 channels), each lane reading its 64 key entries once per token.
#include "mfma_util.hpp"
#include "pic_internal.hpp"

namespace pic {
namespace {

constexpr int SP = 128;        // padded head size (state rows and columns)
constexpr int SNT = SP / 32;   // 32-row tiles of a column strip
constexpr int STW = 4;         // seam tokens staged per round
constexpr int SLDR = SP + 8;   // row stride of the staged operator (bf16)

template <bool BF16>
__device__ __forceinline__ float ld_in(const void* p, int64_t i) {
  if (BF16) return static_cast<float>(static_cast<const __bf16*>(p)[i]);
  return static_cast<const float*>(p)[i];
}

template <int FORM, bool BF16>
__global__ __launch_bounds__(256) void compose_seam_kernel(SeamArgs sa) {
  __shared__ __attribute__((aligned(16))) __bf16 th_hi[FORM == kDense ? SP * SLDR : 8];
  __shared__ __attribute__((aligned(16))) __bf16 th_lo[FORM == kDense ? SP * SLDR : 8];
  __shared__ __attribute__((aligned(16))) float sk[STW][SP];
  __shared__ __attribute__((aligned(16))) float sq[STW][SP];
  __shared__ __attribute__((aligned(16))) float sv[STW][SP];
  __shared__ __attribute__((aligned(16))) float sg[STW][FORM == kDiag ? SP : 4];  // gates
  __shared__ float sb[STW];                                                       // beta

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int dk = sa.c.dk, dv = sa.c.dv, H = sa.c.heads;
  const int64_t BH = int64_t(sa.c.batch) * H;
  const int64_t unit = blockIdx.x;
  const int64_t r = unit / BH, bh = unit % BH;
  const int b = int(bh / H), h = int(bh % H);
  const int n = wave * 32 + (lane & 31);  // state column of this lane
  const bool ncol = n < dv;
  const int64_t sdd = int64_t(dk) * dv;
  const int64_t NS = sa.n_seam;

  f32x16 S[SNT];
#pragma unroll
  for (int t = 0; t < SNT; ++t)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = t * 32 + acc_row(q, g);
      S[t][q] = (sa.c.S_in && ncol && row < dk) ? sa.c.S_in[unit * sdd + int64_t(row) * dv + n] : 0.f;
    }

  // operator of one chain step (dense), this thread's float4 items, zero padded
  float4 pre[16];
  auto load_op = [&](int64_t pu) {
    const float* Tp = sa.c.pool_T_hat + pu * int64_t(dk) * dk;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int e = threadIdx.x + it * 256;
      const int row = (e * 4) / SP, col = (e * 4) % SP;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row < dk && col < dk) x = *reinterpret_cast<const float4*>(Tp + row * dk + col);
      pre[it] = x;
    }
  };

  // stage seam tokens t0 .. t0+m-1 (m <= STW) into LDS
  auto stage = [&](int64_t t0, int m) {
#pragma unroll
    for (int i = 0; i < STW * SP / 256; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int tt = e / SP, ch = e % SP;
      if (tt < m) {
        const int64_t tok = (int64_t(b) * NS + t0 + tt) * H + h;
        sk[tt][ch] = ch < dk ? ld_in<BF16>(sa.k, tok * dk + ch) : 0.f;
        sq[tt][ch] = ch < dk ? ld_in<BF16>(sa.q, tok * dk + ch) : 0.f;
        sv[tt][ch] = ch < dv ? ld_in<BF16>(sa.v, tok * dv + ch) : 0.f;
        if (FORM == kDiag) sg[tt][ch] = ch < dk ? sa.alpha[tok * dk + ch] : 1.f;
        if (FORM != kDiag && ch == 0) {
          sg[tt][0] = sa.alpha[tok];
          sb[tt] = (FORM == kDense && sa.beta) ? sa.beta[tok] : 1.f;
        }
      }
    }
  };

  // one seam token (staged slot tt, seam token index t): update, then readout
  auto token = [&](int tt, int64_t t) {
    float kr[SNT][16];
#pragma unroll
    for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(&sk[tt][32 * t4 + 8 * i + 4 * g]);
        kr[t4][4 * i] = x.x; kr[t4][4 * i + 1] = x.y; kr[t4][4 * i + 2] = x.z; kr[t4][4 * i + 3] = x.w;
      }
    const float vn = sv[tt][n];
    if (FORM == kDense) {
      float u = 0.f;
#pragma unroll
      for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
        for (int q = 0; q < 16; ++q) u = fmaf(kr[t4][q], S[t4][q], u);
      u += __shfl_xor(u, 32);
      const float a = sg[tt][0];
      const float cc = sb[tt] * (vn - a * u);
#pragma unroll
      for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
        for (int q = 0; q < 16; ++q) S[t4][q] = fmaf(kr[t4][q], cc, a * S[t4][q]);
    } else if (FORM == kScalar) {
      const float a = sg[tt][0];
#pragma unroll
      for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
        for (int q = 0; q < 16; ++q) S[t4][q] = fmaf(kr[t4][q], vn, a * S[t4][q]);
    } else {
#pragma unroll
      for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 ga = *reinterpret_cast<const float4*>(&sg[tt][32 * t4 + 8 * i + 4 * g]);
          const float gv[4] = {ga.x, ga.y, ga.z, ga.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            S[t4][4 * i + e] = fmaf(kr[t4][4 * i + e], vn, gv[e] * S[t4][4 * i + e]);
        }
    }
    float o = 0.f;
#pragma unroll
    for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(&sq[tt][32 * t4 + 8 * i + 4 * g]);
        o = fmaf(x.x, S[t4][4 * i], o);
        o = fmaf(x.y, S[t4][4 * i + 1], o);
        o = fmaf(x.z, S[t4][4 * i + 2], o);
        o = fmaf(x.w, S[t4][4 * i + 3], o);
      }
    o += __shfl_xor(o, 32);
    if (g == 0 && ncol) sa.O[((int64_t(b) * NS + t) * H + h) * dv + n] = o;
  };

  const int64_t c0 = chain_offset(sa.c, r), c1 = chain_offset(sa.c, r + 1);
  if (FORM == kDense && c0 < c1) load_op(int64_t(chain_entry(sa.c, c0)) * BH + bh);
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t pu = int64_t(chain_entry(sa.c, c)) * BH + bh;
    // the entry's seam window
    const int64_t t_lo = seam_offset(sa, c), t_hi = seam_offset(sa, c + 1);
    for (int64_t t0 = t_lo; t0 < t_hi; t0 += STW) {
      const int m = int(t_hi - t0 < STW ? t_hi - t0 : STW);
      __syncthreads();  // the previous round's tokens are no longer read
      stage(t0, m);
      __syncthreads();
      for (int tt = 0; tt < m; ++tt) token(tt, t0 + tt);
    }
    // then the entry's pair
    const float* S0p = sa.c.pool_S0 + pu * sdd;
    if (FORM == kDense) {
      __syncthreads();  // every wave is done reading the previous operator
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int e = threadIdx.x + it * 256;
        const int row = (e * 4) / SP, col = (e * 4) % SP;
        unsigned h0, l0, h1, l1;
        split2(pre[it].x, pre[it].y, h0, l0);
        split2(pre[it].z, pre[it].w, h1, l1);
        // columns permuted within each 16 (bits 2 and 3 swapped) so that the
        // 8 columns of a permuted K-step are contiguous
        const int pcol = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
        *reinterpret_cast<uint2*>(th_hi + row * SLDR + pcol) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(th_lo + row * SLDR + pcol) = make_uint2(l0, l1);
      }
      if (c + 1 < c1) load_op(int64_t(chain_entry(sa.c, c + 1)) * BH + bh);
      f32x16 s0[SNT];
#pragma unroll
      for (int t = 0; t < SNT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = t * 32 + acc_row(q, g);
          s0[t][q] = (ncol && row < dk) ? S0p[int64_t(row) * dv + n] : 0.f;
        }
      const float scale = expf(sa.c.pool_log_scale[pu]);
      __syncthreads();
      f32x16 acc[SNT];
#pragma unroll
      for (int t = 0; t < SNT; ++t) acc[t] = zero16();
#pragma unroll
      for (int ks = 0; ks < 2 * SNT; ++ks) {
        const int t = ks >> 1, hh = ks & 1;
        bf16x8 bhi, blo;
        split_acc_half(S[t], hh, bhi, blo);
        const int kc = 32 * t + 16 * hh + 8 * g;
#pragma unroll
        for (int mt = 0; mt < SNT; ++mt) {
          const int arow = mt * 32 + (lane & 31);
          const bf16x8 ahi = lds_load8(th_hi + arow * SLDR + kc);
          const bf16x8 alo = lds_load8(th_lo + arow * SLDR + kc);
          acc[mt] = mfma32(alo, bhi, acc[mt]);
          acc[mt] = mfma32(ahi, blo, acc[mt]);
          acc[mt] = mfma32(ahi, bhi, acc[mt]);
        }
      }
#pragma unroll
      for (int t = 0; t < SNT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) S[t][q] = fmaf(scale, acc[t][q], s0[t][q]);
    } else {
      const float sc = (FORM == kScalar) ? expf(sa.c.pool_log_scale[pu]) : 1.f;
#pragma unroll
      for (int t = 0; t < SNT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = t * 32 + acc_row(q, g);
          const bool in = ncol && row < dk;
          const float rs = (FORM == kDiag) ? (row < dk ? expf(sa.c.pool_log_scale[pu * dk + row]) : 1.f) : sc;
          S[t][q] = fmaf(rs, S[t][q], in ? S0p[int64_t(row) * dv + n] : 0.f);
        }
    }
  }

  if (ncol) {
#pragma unroll
    for (int t = 0; t < SNT; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = t * 32 + acc_row(q, g);
        if (row < dk) sa.c.S_out[unit * sdd + int64_t(row) * dv + n] = S[t][q];
      }
  }
}

template <int FORM>
void launch_seam_t(const SeamArgs& a, dim3 grid, hipStream_t s) {
  if (a.qkv_bf16)
    hipLaunchKernelGGL((compose_seam_kernel<FORM, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((compose_seam_kernel<FORM, false>), grid, dim3(256), 0, s, a);
}

}  // namespace

hipError_t launch_compose_seams(const SeamArgs& a, hipStream_t s) {
  const int64_t units = int64_t(a.c.n_req) * a.c.batch * a.c.heads;
  if (units <= 0) return hipSuccess;
  if (units > 0x7fffffffLL || a.c.dk > SP || a.c.dv > SP) return hipErrorInvalidConfiguration;
  const dim3 grid{unsigned(units), 1, 1};
  switch (a.c.form) {
    case kScalar: launch_seam_t<kScalar>(a, grid, s); break;
    case kDiag: launch_seam_t<kDiag>(a, grid, s); break;
    case kDense: launch_seam_t<kDense>(a, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pic
