// k_rerotate.hip -- moving cached pairs to another position under rotary
// position embeddings on the keys.
// [xix.ai HYPIC article (French), paragraph on linear layers: variants with
//  rotary embeddings need the cached state re-rotated.]
//
// A segment built with its keys rotated at positions t and placed p positions
// later has every key rotated by R_p on top; R_p is orthogonal, so each token
// transition becomes R_p T_t R_p^T and the pair becomes
//     S0' = R_p S0,   That' = R_p That R_p^T,   lambda' = lambda
// (exact for the scalar and dense forms, and for per-channel gates that are
// equal within every rotated channel pair).  R_p turns channel pair i, (2i,
// 2i+1) or (i, i + rot/2), by p * base^(-2i/rot); channels from rot on stay.
//
// One workgroup per (entry, layer, head).  The pair's angles are formed in
// fp64 (an fp32 product p * theta loses the angle at long offsets) and kept in
// LDS as fp32 cos / sin.  Each thread step writes one float4 of the output:
// S0 rows combine the row and its partner; That rows are combined the same
// way, then columns (the partner column lies in the same float4 for the
// interleaved pairing and in the float4 rot/8 groups away for the half one).
// Memory bound: every pool float is read once from HBM (partner reads hit the
// cache) and every output float written once.
#include "pic_internal.hpp"

namespace pic {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ float4 comb(float c, float s, float4 m, float4 p) {
  return make_float4(fmaf(s, p.x, c * m.x), fmaf(s, p.y, c * m.y), fmaf(s, p.z, c * m.z),
                     fmaf(s, p.w, c * m.w));
}

__global__ __launch_bounds__(kThreads) void rerotate_kernel(RotateArgs a) {
  __shared__ float cs_c[64], cs_s[64];
  const int BH = a.batch * a.heads;
  const int j = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int64_t src = int64_t(table_at(a.d_idx, j)) * BH + bh;
  const int64_t dst = int64_t(j) * BH + bh;
  const int rot = a.rot_dim, h2 = rot / 2, dk = a.dk, dv = a.dv;
  const bool half = a.half;
  if (int(threadIdx.x) < h2) {
    const double theta = pow(a.base, -2.0 * double(threadIdx.x) / double(rot));
    double sn, cn;
    sincos(double(table_at(a.d_shift, j)) * theta, &sn, &cn);
    cs_c[threadIdx.x] = float(cn);
    cs_s[threadIdx.x] = float(sn);
  }
  const int per = (a.form == kDiag) ? dk : 1;
  for (int t = threadIdx.x; t < per; t += kThreads)
    a.log_scale_out[dst * per + t] = a.pool_log_scale[src * per + t];
  __syncthreads();

  // row x of R M = c M[x] + s M[px]  (s carries the sign of x's place in its pair)
  auto rowrot = [&](int x, float& c, float& s, int& px) {
    if (x >= rot) {
      c = 1.f;
      s = 0.f;
      px = x;
      return;
    }
    int i;
    if (half) {
      const bool first = x < h2;
      i = first ? x : x - h2;
      px = first ? x + h2 : x - h2;
      s = first ? -cs_s[i] : cs_s[i];
    } else {
      i = x >> 1;
      px = x ^ 1;
      s = (x & 1) ? cs_s[i] : -cs_s[i];
    }
    c = cs_c[i];
  };

  {
    const float* M = a.pool_S0 + src * int64_t(dk) * dv;
    float* O = a.S0_out + dst * int64_t(dk) * dv;
    const int g4 = dv / 4;
    for (int e = threadIdx.x; e < dk * g4; e += kThreads) {
      const int x = e / g4, g = e % g4;
      float c, s;
      int px;
      rowrot(x, c, s, px);
      const float4 r = comb(c, s, ld4(M + int64_t(x) * dv + 4 * g), ld4(M + int64_t(px) * dv + 4 * g));
      *reinterpret_cast<float4*>(O + int64_t(x) * dv + 4 * g) = r;
    }
  }
  if (a.pool_T_hat) {
    const float* M = a.pool_T_hat + src * int64_t(dk) * dk;
    float* O = a.T_hat_out + dst * int64_t(dk) * dk;
    const int g4 = dk / 4;
    for (int e = threadIdx.x; e < dk * g4; e += kThreads) {
      const int x = e / g4, g = e % g4;
      float c, s;
      int px;
      rowrot(x, c, s, px);
      const float* mx = M + int64_t(x) * dk;
      const float* mp = M + int64_t(px) * dk;
      const float4 own = comb(c, s, ld4(mx + 4 * g), ld4(mp + 4 * g));
      float4 out = own;
      if (4 * g < rot) {
        const float ov[4] = {own.x, own.y, own.z, own.w};
        float pv[4];
        if (half) {
          const int pg = (4 * g < h2) ? g + h2 / 4 : g - h2 / 4;
          const float4 part = comb(c, s, ld4(mx + 4 * pg), ld4(mp + 4 * pg));
          pv[0] = part.x; pv[1] = part.y; pv[2] = part.z; pv[3] = part.w;
        } else {
          pv[0] = ov[1]; pv[1] = ov[0]; pv[2] = ov[3]; pv[3] = ov[2];
        }
        float r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int y = 4 * g + u;
          int i;
          float sc;
          if (half) {
            i = y < h2 ? y : y - h2;
            sc = y < h2 ? -cs_s[i] : cs_s[i];
          } else {
            i = y >> 1;
            sc = (y & 1) ? cs_s[i] : -cs_s[i];
          }
          r[u] = fmaf(sc, pv[u], cs_c[i] * ov[u]);
        }
        out = make_float4(r[0], r[1], r[2], r[3]);
      }
      *reinterpret_cast<float4*>(O + int64_t(x) * dk + 4 * g) = out;
    }
  }
}

}  // namespace

hipError_t launch_rerotate(const RotateArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n) * a.batch * a.heads;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL || a.rot_dim > 128 || a.rot_dim % 8 || a.dk % 4 || a.dv % 4)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(rerotate_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pic
