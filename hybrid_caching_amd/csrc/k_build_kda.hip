// k_build_kda.hip -- build of the pair (lambda_C, That_C, S(C|0)) for the
// dense delta form with per-channel gates (KDA form):
//     T_t = (I - b_t k_t k_t^T) Diag(a_t),   a_t in (0, 1]^dk,
//     S_t = T_t S_{t-1} + b_t k_t v_t^T.
// The gate does not factor out of the product, so the pair is split as
//     lambda_C = sum_t ln m_t   (m_t: the token's largest gate)
//     That_C   = prod_t (I - b_t k_t k_t^T) Diag(a_t / m_t)
// (the dense GDN split when every channel has the same gate; ||That|| <= 1),
// which the dense compose applies unchanged.
// [xix.ai HYPIC article (French), paragraph on linear layers: KDA is among
//  the families whose token transitions are composed; T_C is the product of
//  a segment's token transitions.]
//
// Token by token in fp32 on the vector units.  S and That take the same step
// with a different gate g and target y:
//     X <- Diag(g) X;   r = X^T k;   X <- X + k (b (y - r))^T
// S: g = a_t, y = v_t.   That: g = a_t / m_t, y = 0.
// One workgroup of eight waves per (segment, layer, head): waves 0-3 hold S,
// waves 4-7 hold That, 32 columns per wave.  Lane (p, q) of a wave (q = lane
// % 4, p = lane / 4) holds rows 32q .. 32q+31 of columns 2p, 2p+1 of its
// wave's 32: each k and gate value read from LDS serves two columns, and the
// column sums r reduce over the four lanes of a quad with DPP.  Per state
// element and token: one multiply and two fmas.
// Tokens are staged in LDS sixteen at a time (fp32, zero padded to 128
// channels): k and both gates in four groups of 32 rows, each group padded to
// 36 floats so that the four row groups of a wave read distinct banks.
#include "pic_internal.hpp"

namespace pic {
namespace {

constexpr int KP = 128;   // padded head size
constexpr int KTW = 16;   // tokens staged per round (512 threads, 32 per token)
constexpr int RG = 36;    // LDS stride of a 32-row group (32 + 4 pad)
constexpr int KTH = 512;  // threads per workgroup

__device__ __forceinline__ float quad_sum(float x) {
  // quad_perm [1,0,3,2] then [2,3,0,1]: every lane of a quad gets the sum
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                             0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                             0x4E, 0xF, 0xF, false));
  return x;
}

template <bool BF16>
__global__ __launch_bounds__(KTH) void build_kda_kernel(BuildArgs a) {
  __shared__ __attribute__((aligned(16))) float sk[KTW][4 * RG];   // k
  __shared__ __attribute__((aligned(16))) float sg[2][KTW][4 * RG];  // a, a / m
  __shared__ __attribute__((aligned(16))) float sv[KTW][KP];        // v
  __shared__ float sb[KTW], sl[KTW];                                 // b, ln m

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int role = wave >> 2;  // 0: S, 1: That
  const int q = lane & 3, p = lane >> 2;
  const int dk = a.dk, dv = a.dv, H = a.heads;
  const int BH = a.batch * H;
  const int seg = seg_in_order(a, int(build_unit(a, blockIdx.x) / BH));
  const int bh = int(build_unit(a, blockIdx.x) % BH);
  const int b = bh / H, h = bh % H;
  const int64_t t_begin = seg_offset(a, seg), t_end = seg_offset(a, seg + 1);
  const int64_t N = a.n_tokens;
  const int64_t unit = (int64_t(seg) * a.batch + b) * H + h;
  const int ncols = role ? dk : dv;
  const int n0 = 32 * (wave & 3) + 2 * p;  // the lane's first column
  const int r0 = 32 * q;                   // the lane's first row
  // waves whose 32 columns are all padding skip the arithmetic (wave-uniform)
  const bool active = 32 * (wave & 3) < ncols;

  float X[32][2];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    X[i][0] = (role && r0 + i == n0 && n0 < dk) ? 1.f : 0.f;
    X[i][1] = (role && r0 + i == n0 + 1 && n0 + 1 < dk) ? 1.f : 0.f;
  }
  float lam = 0.f;

  // staging: thread e holds channels 4 (e % 32) .. +3 of token e / 32
  const int rt = threadIdx.x >> 5, rc = 4 * (threadIdx.x & 31);
  const int rs = (rc >> 5) * RG + (rc & 31);  // the channels' place in a grouped row
  auto ld4 = [&](const void* base, int64_t off) -> float4 {
    if constexpr (BF16) {
      const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const __bf16*>(base) + off);
      return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                         __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
    } else {
      return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    }
  };

  for (int64_t t0 = t_begin; t0 < t_end; t0 += KTW) {
    const int m = int(t_end - t0 < KTW ? t_end - t0 : KTW);
    __syncthreads();  // the previous round's tokens are no longer read
    {
      // tokens past the segment's end read its last token (never used)
      const int64_t tl = t0 + rt < t_end ? t0 + rt : t_end - 1;
      const int64_t tok = (int64_t(b) * N + tl) * H + h;
      const bool ck = rc < dk, cv = rc < dv;
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      float4 kk = z, vv = z, aa = z;
      if (ck) {
        kk = ld4(a.k, tok * dk + rc);
        aa = *reinterpret_cast<const float4*>(a.alpha + tok * dk + rc);
      }
      if (cv) vv = ld4(a.v, tok * dv + rc);
      // the token's largest gate: over this thread's four channels, then over
      // the 32 threads of the token (half a wave); padded channels hold 0
      float mx = fmaxf(fmaxf(aa.x, aa.y), fmaxf(aa.z, aa.w));
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
      const float4 am = make_float4(aa.x / mx, aa.y / mx, aa.z / mx, aa.w / mx);
      *reinterpret_cast<float4*>(&sk[rt][rs]) = kk;
      *reinterpret_cast<float4*>(&sg[0][rt][rs]) = aa;
      *reinterpret_cast<float4*>(&sg[1][rt][rs]) = am;
      *reinterpret_cast<float4*>(&sv[rt][rc]) = vv;
      if ((threadIdx.x & 31) == 0) {
        sl[rt] = logf(mx);
        sb[rt] = a.beta ? a.beta[tok] : 1.f;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0)
      for (int tt = 0; tt < m; ++tt) lam += sl[tt];
    if (!active) continue;
#pragma unroll 1
    for (int tt = 0; tt < m; ++tt) {
      const float* kq = &sk[tt][q * RG];
      const float* gq = &sg[role][tt][q * RG];
      float kr[32];
      float ra[2] = {0.f, 0.f}, rb[2] = {0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 k4 = *reinterpret_cast<const float4*>(kq + 4 * j);
        const float4 g4 = *reinterpret_cast<const float4*>(gq + 4 * j);
        const float kv[4] = {k4.x, k4.y, k4.z, k4.w}, gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * j + e;
          kr[i] = kv[e];
          X[i][0] *= gv[e];
          X[i][1] *= gv[e];
          // two partial sums per column
          ra[i & 1] = fmaf(kv[e], X[i][0], ra[i & 1]);
          rb[i & 1] = fmaf(kv[e], X[i][1], rb[i & 1]);
        }
      }
      const float r_0 = quad_sum(ra[0] + ra[1]), r_1 = quad_sum(rb[0] + rb[1]);
      const float be = sb[tt];
      float y0 = 0.f, y1 = 0.f;
      if (!role) {
        const float2 v2 = *reinterpret_cast<const float2*>(&sv[tt][n0]);
        y0 = v2.x;
        y1 = v2.y;
      }
      const float c0 = be * (y0 - r_0), c1 = be * (y1 - r_1);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        X[i][0] = fmaf(kr[i], c0, X[i][0]);
        X[i][1] = fmaf(kr[i], c1, X[i][1]);
      }
    }
  }

  if (n0 < ncols) {
    // ncols and n0 are even: both columns are in range
    const int ld = role ? dk : dv;
    float* out = (role ? a.T_hat : a.S0) + unit * int64_t(dk) * ld;
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (r0 + i < dk)
        *reinterpret_cast<float2*>(out + int64_t(r0 + i) * ld + n0) = make_float2(X[i][0], X[i][1]);
  }
  if (threadIdx.x == 0) a.log_scale[unit] = lam;
}

}  // namespace

hipError_t launch_build_kda(const BuildArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_seg) * a.batch * a.heads;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL || a.dk > KP || a.dv > KP || a.dk % 16 || a.dv % 16)
    return hipErrorInvalidConfiguration;
  if (a.qkv_bf16)
    hipLaunchKernelGGL(build_kda_kernel<true>, dim3(unsigned(blocks)), dim3(KTH), 0, s, a);
  else
    hipLaunchKernelGGL(build_kda_kernel<false>, dim3(unsigned(blocks)), dim3(KTH), 0, s, a);
  return hipGetLastError();
}

}  // namespace pic
