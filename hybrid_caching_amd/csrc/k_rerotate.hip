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
// LDS as fp32 cos / sin.  A thread item holds everything one rotation step
// mixes: a rotated row pair (or one unrotated row) of float4 groups, and for
// That also the partner column group (in the same float4 for the interleaved
// pairing, rot/8 groups away for the half one).  Memory bound: every pool
// float is read once and every output float written once.
#include "pic_internal.hpp"

namespace pic {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

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

  // Work items pair what the rotation mixes, so each thread reads every value
  // it combines and no value is read twice: a row unit is a rotated row pair
  // (a, b) (u < rot/2) or one unrotated row; for That a column unit is the
  // float4 group pair (g, g + rot/8) (half pairing, g < rot/8) or one group
  // (interleaved pairs sit inside a float4; groups past rot/4 are unrotated).
  const int n_ru = h2 + (dk - rot);
  auto row_unit = [&](int u, int& ra, int& rb, float& c, float& s) {
    if (u < h2) {
      ra = half ? u : 2 * u;
      rb = half ? u + h2 : 2 * u + 1;
      c = cs_c[u];
      s = cs_s[u];
    } else {
      ra = rb = rot + (u - h2);
      c = 1.f;
      s = 0.f;
    }
  };
  // (x_a, x_b) -> (c x_a - s x_b, s x_a + c x_b), per float4 lane
  auto turn = [](float c, float s, float4& xa, float4& xb) {
    const float4 a0 = xa, b0 = xb;
    xa = make_float4(fmaf(-s, b0.x, c * a0.x), fmaf(-s, b0.y, c * a0.y), fmaf(-s, b0.z, c * a0.z),
                     fmaf(-s, b0.w, c * a0.w));
    xb = make_float4(fmaf(s, a0.x, c * b0.x), fmaf(s, a0.y, c * b0.y), fmaf(s, a0.z, c * b0.z),
                     fmaf(s, a0.w, c * b0.w));
  };

  {
    const float* M = a.pool_S0 + src * int64_t(dk) * dv;
    float* O = a.S0_out + dst * int64_t(dk) * dv;
    const int g4 = dv / 4;
    for (int e = threadIdx.x; e < n_ru * g4; e += kThreads) {
      const int u = e / g4, g = e % g4;
      int ra, rb;
      float c, s;
      row_unit(u, ra, rb, c, s);
      float4 xa = ld4(M + int64_t(ra) * dv + 4 * g);
      if (ra == rb) {
        *reinterpret_cast<float4*>(O + int64_t(ra) * dv + 4 * g) = xa;
        continue;
      }
      float4 xb = ld4(M + int64_t(rb) * dv + 4 * g);
      turn(c, s, xa, xb);
      *reinterpret_cast<float4*>(O + int64_t(ra) * dv + 4 * g) = xa;
      *reinterpret_cast<float4*>(O + int64_t(rb) * dv + 4 * g) = xb;
    }
  }
  if (a.pool_T_hat) {
    const float* M = a.pool_T_hat + src * int64_t(dk) * dk;
    float* O = a.T_hat_out + dst * int64_t(dk) * dk;
    const int r8 = rot / 8, r4 = rot / 4;
    const int n_cu = half ? r8 + (dk / 4 - r4) : dk / 4;
    for (int e = threadIdx.x; e < n_ru * n_cu; e += kThreads) {
      const int u = e / n_cu, v = e % n_cu;
      int ra, rb;
      float c, s;
      row_unit(u, ra, rb, c, s);
      const bool rpair = ra != rb;
      // column groups of this item: ga and (half pairing, rotated) gb
      int ga, gb;
      if (half) {
        ga = v < r8 ? v : r4 + (v - r8);
        gb = v < r8 ? v + r8 : ga;
      } else {
        ga = gb = v;
      }
      const bool cpair = ga != gb;
      float4 aa = ld4(M + int64_t(ra) * dk + 4 * ga), ba = aa, ab = aa, bb = aa;
      if (rpair) ba = ld4(M + int64_t(rb) * dk + 4 * ga);
      if (cpair) {
        ab = ld4(M + int64_t(ra) * dk + 4 * gb);
        if (rpair) bb = ld4(M + int64_t(rb) * dk + 4 * gb);
      }
      // rows
      if (rpair) {
        turn(c, s, aa, ba);
        if (cpair) turn(c, s, ab, bb);
      }
      // columns
      if (cpair) {
        // column 4 ga + l pairs with 4 gb + l, angle index 4 ga + l
        const float4 cc = make_float4(cs_c[4 * ga], cs_c[4 * ga + 1], cs_c[4 * ga + 2], cs_c[4 * ga + 3]);
        const float4 ss = make_float4(cs_s[4 * ga], cs_s[4 * ga + 1], cs_s[4 * ga + 2], cs_s[4 * ga + 3]);
        auto cturn = [&](float4& xa, float4& xb) {
          const float4 a0 = xa, b0 = xb;
          xa = make_float4(fmaf(-ss.x, b0.x, cc.x * a0.x), fmaf(-ss.y, b0.y, cc.y * a0.y),
                           fmaf(-ss.z, b0.z, cc.z * a0.z), fmaf(-ss.w, b0.w, cc.w * a0.w));
          xb = make_float4(fmaf(ss.x, a0.x, cc.x * b0.x), fmaf(ss.y, a0.y, cc.y * b0.y),
                           fmaf(ss.z, a0.z, cc.z * b0.z), fmaf(ss.w, a0.w, cc.w * b0.w));
        };
        cturn(aa, ab);
        if (rpair) cturn(ba, bb);
      } else if (!half && 4 * ga < rot) {
        // interleaved: columns (4ga, 4ga+1) and (4ga+2, 4ga+3), angles 2ga, 2ga+1
        const float c0 = cs_c[2 * ga], s0 = cs_s[2 * ga], c1 = cs_c[2 * ga + 1], s1 = cs_s[2 * ga + 1];
        auto iturn = [&](float4& x) {
          const float4 y = x;
          x = make_float4(fmaf(-s0, y.y, c0 * y.x), fmaf(s0, y.x, c0 * y.y),
                          fmaf(-s1, y.w, c1 * y.z), fmaf(s1, y.z, c1 * y.w));
        };
        iturn(aa);
        if (rpair) iturn(ba);
      }
      *reinterpret_cast<float4*>(O + int64_t(ra) * dk + 4 * ga) = aa;
      if (rpair) *reinterpret_cast<float4*>(O + int64_t(rb) * dk + 4 * ga) = ba;
      if (cpair) {
        *reinterpret_cast<float4*>(O + int64_t(ra) * dk + 4 * gb) = ab;
        if (rpair) *reinterpret_cast<float4*>(O + int64_t(rb) * dk + 4 * gb) = bb;
      }
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
