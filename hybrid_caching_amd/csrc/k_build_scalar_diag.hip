// k_build_scalar_diag.hip -- build the cached pair (lambda_C, S(C|0)) of the
// scalar-decay (RetNet / Mamba2-like) and diagonal-gate (GLA-like) forms for
// every (segment, layer, head).
//
// Per token: S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T (scalar: alpha_t I), so
//   T_C = Diag(e^{lambda_C}),  lambda_C = sum_t ln alpha_t (per channel; one
//   value for the scalar form), and
//   S(C|0) = sum_t e^{lambda_C - B_t} (.) k_t v_t^T   (row scaling, B_t = the
//   inclusive prefix of ln alpha).
// [xix.ai HYPIC article (French), paragraph on linear layers: T_C is the
//  product of the token transitions, S(C|0) the final state from zero; decay
//  (RetNet, Mamba2) and gating (GLA) families.  remio.ai (Japanese), section on
//  state composition: scalar and diagonal transition forms.]
//
// Chunked form, chunk of C = 64 tokens, in log space (base 2): with b_t the
// in-chunk inclusive prefix of log2 alpha (per channel for the diagonal form),
//   S <- 2^{b_C} (.) S + Kw^T V,   Kw_t = 2^{b_C - b_t} (.) k_t  (all factors <= 1).
// The contraction Kw^T V (dk x 64 times 64 x dv per chunk) runs on MFMA:
// Kw is fp32 and is split into hi/lo bf16; V is exact in bf16 for bf16 inputs.
// One workgroup per (segment, layer, head); wave w owns columns [32w, 32w+32)
// of S in accumulators; K is transposed into LDS while it is scaled.
#include "mfma_util.hpp"
#include "pic_internal.hpp"

namespace pic {
namespace {

constexpr int kChunkSD = 64;

template <int DP, bool INBF16, bool DIAG>
struct SdLds {
  static constexpr int C = kChunkSD;
  static constexpr int NP = INBF16 ? 1 : 2;
  static constexpr int KT_LD = C + 8;  // bf16 row stride of Kw^T and V^T
  static constexpr int KT = 0;                                 // Kw^T hi, lo [2][DP][KT_LD]
  static constexpr int VT = KT + 2 * DP * KT_LD * 2;           // V^T [NP][DP][KT_LD]
  static constexpr int BM = VT + NP * DP * KT_LD * 2;          // diag: prefix [C][DP] fp32
  static constexpr int BM_BYTES = DIAG ? C * DP * 4 : C * 4;   // scalar: r_t [C]
  static constexpr int TS = BM + BM_BYTES;                     // diag: part totals [2][DP]
  static constexpr int TS_BYTES = DIAG ? 2 * DP * 4 : 16;      // scalar: gamma
  static constexpr int TOTAL = TS + TS_BYTES;
};

template <bool INBF16>
__device__ __forceinline__ void load8_sd(const void* base, int64_t elem, bool valid, float* out) {
  if (!valid) {
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = 0.f;
    return;
  }
  if (INBF16) {
    const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const __bf16*>(base) + elem);
    const unsigned w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[2 * j] = __uint_as_float(w[j] << 16);
      out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    const float4 x = p[0], y = p[1];
    out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    out[4] = y.x; out[5] = y.y; out[6] = y.z; out[7] = y.w;
  }
}

__device__ __forceinline__ void st_pair_sd(__bf16* p, __bf16 a, __bf16 b) {
  const unsigned v = unsigned(bf16_bits(a)) | (unsigned(bf16_bits(b)) << 16);
  *reinterpret_cast<unsigned*>(p) = v;
}

template <int DP, bool INBF16, bool DIAG>
__global__ __launch_bounds__(2 * DP) void build_sd_kernel(BuildArgs a) {
  using L = SdLds<DP, INBF16, DIAG>;
  constexpr int C = kChunkSD, NT = DP / 32, NTH = 2 * DP, KT = L::KT_LD;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  __bf16* Kth = reinterpret_cast<__bf16*>(smem + L::KT);  // [DP][KT]
  __bf16* Ktl = Kth + DP * KT;
  __bf16* Vt = reinterpret_cast<__bf16*>(smem + L::VT);   // [NP][DP][KT]
  float* Bm = reinterpret_cast<float*>(smem + L::BM);
  float* Ts = reinterpret_cast<float*>(smem + L::TS);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, cl = lane & 31;
  const int H = a.heads, dk = a.dk, dv = a.dv;
  const int BH = a.batch * H;
  const int seg = seg_in_order(a, int(build_unit(a, blockIdx.x) / BH));
  const int bh = int(build_unit(a, blockIdx.x) % BH), b = bh / H, h = bh % H;
  const int64_t t_begin = seg_offset(a, seg), t_end = seg_offset(a, seg + 1);
  const int64_t N = a.n_tokens;
  const int ncol = wave * 32 + cl;
  // diag: thread (part, channel) scans half of the chunk for one channel
  const int ch = tid % DP, part = tid / DP;

  f32x16 S[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) S[t] = zero16();
  float lam = 0.f;

  for (int64_t c0 = t_begin; c0 < t_end; c0 += C) {
    const int len = (t_end - c0 < C) ? int(t_end - c0) : C;
    __syncthreads();  // previous chunk done with LDS

    // ---------------- gate prefixes
    if (DIAG) {
      float run = 0.f;
      const int tb = part * (C / 2);
#pragma unroll 4
      for (int t = tb; t < tb + C / 2; ++t) {
        float x = 0.f;
        if (t < len && ch < dk) x = log2f(a.alpha[((int64_t(b) * N + c0 + t) * H + h) * dk + ch]);
        run += x;
        Bm[t * DP + ch] = run;
      }
      Ts[part * DP + ch] = run;
    } else if (wave == 0) {
      float x = (lane < len) ? log2f(a.alpha[(int64_t(b) * N + c0 + lane) * H + h]) : 0.f;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      const float bend = __shfl(x, 63, 64);
      Bm[lane] = exp2f(bend - x);
      if (lane == 0) Ts[0] = bend;
      lam += bend;
    }
    __syncthreads();
    if (DIAG && part == 0) lam += Ts[ch] + Ts[DP + ch];

    // ---------------- stage Kw^T (scaled, split) and V^T
    for (int item = tid; item < (C / 2) * (DP / 8); item += NTH) {
      const int tp = item / (DP / 8), i0 = (item % (DP / 8)) * 8, t0 = 2 * tp;
      float ka[8], kb[8], va[8], vb[8];
      const int64_t row0 = (int64_t(b) * N + c0 + t0) * H + h;
      load8_sd<INBF16>(a.k, row0 * dk + i0, t0 < len && i0 < dk, ka);
      load8_sd<INBF16>(a.k, (row0 + H) * dk + i0, t0 + 1 < len && i0 < dk, kb);
      load8_sd<INBF16>(a.v, row0 * dv + i0, t0 < len && i0 < dv, va);
      load8_sd<INBF16>(a.v, (row0 + H) * dv + i0, t0 + 1 < len && i0 < dv, vb);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float wa, wb;
        if (DIAG) {
          const int i = i0 + j;
          const float tot = Ts[i] + Ts[DP + i];
          const float ba = Bm[t0 * DP + i] + (t0 >= C / 2 ? Ts[i] : 0.f);
          const float bb = Bm[(t0 + 1) * DP + i] + (t0 + 1 >= C / 2 ? Ts[i] : 0.f);
          wa = exp2f(tot - ba);
          wb = exp2f(tot - bb);
        } else {
          wa = Bm[t0];
          wb = Bm[t0 + 1];
        }
        const float xa = wa * ka[j], xb = wb * kb[j];
        const __bf16 ah = to_bf16(xa), bh = to_bf16(xb);
        st_pair_sd(Kth + (i0 + j) * KT + t0, ah, bh);
        st_pair_sd(Ktl + (i0 + j) * KT + t0, to_bf16(xa - from_bf16(ah)), to_bf16(xb - from_bf16(bh)));
        const __bf16 vah = to_bf16(va[j]), vbh = to_bf16(vb[j]);
        st_pair_sd(Vt + (i0 + j) * KT + t0, vah, vbh);
        if (!INBF16)
          st_pair_sd(Vt + DP * KT + (i0 + j) * KT + t0, to_bf16(va[j] - from_bf16(vah)),
                     to_bf16(vb[j] - from_bf16(vbh)));
      }
    }
    __syncthreads();

    // ---------------- S <- e^{b_C} (.) S + Kw^T V  (this wave's column strip)
    if (DIAG) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = t * 32 + acc_row(q, g);
          S[t][q] *= exp2f(Ts[row] + Ts[DP + row]);
        }
    } else {
      const float gam = exp2f(Ts[0]);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) S[t][q] *= gam;
    }
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      const int kc = ks * 16 + 8 * g;
      const bf16x8 vh = lds_load8(Vt + ncol * KT + kc);
      bf16x8 vl;
      if (!INBF16) vl = lds_load8(Vt + DP * KT + ncol * KT + kc);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int row = t * 32 + cl;
        const bf16x8 kh = lds_load8(Kth + row * KT + kc);
        const bf16x8 kl = lds_load8(Ktl + row * KT + kc);
        S[t] = mfma32(kl, vh, S[t]);
        if (!INBF16) S[t] = mfma32(kh, vl, S[t]);
        S[t] = mfma32(kh, vh, S[t]);
      }
    }
  }

  const int64_t unit = (int64_t(seg) * a.batch + b) * H + h;
  if (ncol < dv) {
    float* out = a.S0 + unit * int64_t(dk) * dv;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = t * 32 + acc_row(q, g);
        if (row < dk) out[int64_t(row) * dv + ncol] = S[t][q];
      }
  }
  if (DIAG) {
    if (part == 0 && ch < dk) a.log_scale[unit * dk + ch] = lam * kLn2;
  } else if (tid == 0) {
    a.log_scale[unit] = lam * kLn2;
  }
}

template <int DP, bool INBF16, bool DIAG>
hipError_t launch_sd_t(const BuildArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_seg) * a.batch * a.heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((build_sd_kernel<DP, INBF16, DIAG>), dim3(unsigned(blocks)), dim3(2 * DP),
                     0, s, a);
  return hipGetLastError();
}

template <bool INBF16, bool DIAG>
hipError_t launch_sd_dp(const BuildArgs& a, hipStream_t s) {
  const int d = a.dk > a.dv ? a.dk : a.dv;
  if (d <= 32) return launch_sd_t<32, INBF16, DIAG>(a, s);
  if (d <= 64) return launch_sd_t<64, INBF16, DIAG>(a, s);
  return launch_sd_t<128, INBF16, DIAG>(a, s);
}

}  // namespace

hipError_t launch_build_scalar_diag(const BuildArgs& a, hipStream_t s) {
  const bool diag = a.form == kDiag;
  // bf16 inputs take the streaming kernel (k_build_sd_pipe.hip)
  if (a.qkv_bf16) return launch_build_sd_pipe(a, s);
  return diag ? launch_sd_dp<false, true>(a, s) : launch_sd_dp<false, false>(a, s);
}

}  // namespace pic
