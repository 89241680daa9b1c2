// k_build_dense.hip -- build the cached pair (lambda_C, That_C, S(C|0)) of the
// dense gated-delta (GDN) form for every (segment, layer, head).
//
// Per token: S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
// T_C = prod_t alpha_t (I - beta_t k_t k_t^T) = e^{lambda_C} That_C.
// [xix.ai HYPIC article (French), paragraph on linear layers: T_C is the
//  product of the segment's token transition matrices and S(C|0) its final
//  state from zero; dense delta-rule transitions (DeltaNet, GDN, KDA) are the
//  heaviest family.  remio.ai (Japanese), section on state composition: the
//  pair is built once, at the segment's first prefill.]
//
// Chunked form (chunk of C = 64 tokens, gates handled in log space so nothing
// overflows; base 2 in the code): with b_t the inclusive prefix of log2(alpha)
// inside the chunk, gamma = 2^{b_C}, r_t = 2^{b_C - b_t} (<= 1), K, V the chunk's rows,
//   L   = diag(beta) * strictly-lower(K K^T)
//   X   = (I + L)^{-1}                      (unit lower triangular)
//   U   = X diag(beta) K                    so  prod_t (I - beta_t k_t k_t^T) = I - K^T U
//   W   = X diag(beta * r) V
// and the chunk advances the running pair by
//   That <- That - K^T (U That)
//   S    <- gamma S + K^T (W - gamma U S)
//   lambda <- lambda + b_C   (times ln 2 on output).
// (Derivation: dividing S_t by the in-chunk gate product turns the chunk into
// an ungated delta rule with values v_t / g_t; the product of the rank-one
// factors has the compact form I - K^T U with U from the triangular system.)
//
// Mapping to gfx950.  One workgroup per (segment, layer, head) walks the
// segment chunk by chunk.  2*DP/32 waves: waves [0, DP/32) hold 32-column
// strips of S, waves [DP/32, 2*DP/32) hold strips of That, in MFMA
// accumulators for the whole segment.  The chunk's K, K^T, V^T, the
// triangular solve and U live in LDS.  Products with an fp32 operand use the
// split-bf16 scheme (hi*hi + hi*lo + lo*hi); K and V are exact in bf16 when
// the inputs are bf16, so their lo parts are skipped.  Dims below DP are
// zero-padded (exact: padded keys/values add nothing and padded operator
// columns stay the identity).
#include "mfma_util.hpp"
#include "pic_internal.hpp"

namespace pic {
namespace {

constexpr int kChunk = 64;

template <int DP, bool INBF16>
struct DenseLds {
  static constexpr int C = kChunk;
  static constexpr int NP = INBF16 ? 1 : 2;  // parts stored for K / V (hi[, lo])
  static constexpr int KR_LD = DP + 8;       // bf16 row stride of K (row-major) and U
  static constexpr int KT_LD = C + 8;        // bf16 row stride of K^T and V^T
  static constexpr int X_LD = C + 4;         // fp32 row stride of L and X
  // region 1: K row-major [NP][C][KR_LD] while staging / K K^T, then U hi/lo
  static constexpr int R1 = 0;
  static constexpr int R1_BYTES = 2 * C * KR_LD * 2;
  static constexpr int KT = R1 + R1_BYTES;
  static constexpr int VT = KT + NP * DP * KT_LD * 2;
  static constexpr int LM = VT + NP * DP * KT_LD * 2;
  static constexpr int XM = LM + C * X_LD * 4;
  static constexpr int YM = XM + C * X_LD * 4;
  static constexpr int GB = YM + 3 * 256 * 4;
  static constexpr int GR = GB + C * 4;
  static constexpr int GG = GR + C * 4;
  static constexpr int TOTAL = GG + 16;
  static_assert(NP * C * KR_LD * 2 <= R1_BYTES, "K staging must fit region 1");
};

// 8 consecutive inputs (bf16 or fp32) as floats; zeros when !valid
template <bool INBF16>
__device__ __forceinline__ void load8(const void* base, int64_t elem, bool valid, float* out) {
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

// store two tokens' values of one channel as a packed pair (t, t+1)
__device__ __forceinline__ void st_pair(__bf16* p, __bf16 a, __bf16 b) {
  const unsigned v = unsigned(bf16_bits(a)) | (unsigned(bf16_bits(b)) << 16);
  *reinterpret_cast<unsigned*>(p) = v;
}

template <int DP, bool INBF16>
__global__ __launch_bounds__(2 * DP * 2) void build_dense_kernel(BuildArgs a) {
  using L = DenseLds<DP, INBF16>;
  constexpr int C = kChunk, NT = DP / 32, NW = 2 * NT, NTH = NW * 64;
  constexpr int KR = L::KR_LD, KT = L::KT_LD, XL = L::X_LD;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  __bf16* Kr = reinterpret_cast<__bf16*>(smem + L::R1);  // [NP][C][KR]
  __bf16* Uh = reinterpret_cast<__bf16*>(smem + L::R1);  // [C][KR]
  __bf16* Ul = Uh + C * KR;
  __bf16* Kt = reinterpret_cast<__bf16*>(smem + L::KT);  // [NP][DP][KT]
  __bf16* Vt = reinterpret_cast<__bf16*>(smem + L::VT);  // [NP][DP][KT]
  float* Lm = reinterpret_cast<float*>(smem + L::LM);    // [C][XL]
  float* Xm = reinterpret_cast<float*>(smem + L::XM);    // [C][XL]
  float* Ym = reinterpret_cast<float*>(smem + L::YM);    // [3][16][16]
  float* gb = reinterpret_cast<float*>(smem + L::GB);    // beta per token
  float* gr = reinterpret_cast<float*>(smem + L::GR);    // e^{b_C - b_t}
  float* gg = reinterpret_cast<float*>(smem + L::GG);    // gamma

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, cl = lane & 31;
  const int H = a.heads, dk = a.dk, dv = a.dv;
  const int BH = a.batch * H;
  const int seg = seg_in_order(a, int(build_unit(a, blockIdx.x) / BH));
  const int bh = int(build_unit(a, blockIdx.x) % BH), b = bh / H, h = bh % H;
  const int64_t t_begin = seg_offset(a, seg), t_end = seg_offset(a, seg + 1);
  const int64_t N = a.n_tokens;
  const bool s_wave = wave < NT;  // S strip; otherwise That strip
  const int strip = s_wave ? wave : wave - NT;
  const int ncol = strip * 32 + cl;

  f32x16 X[NT];  // this wave's strip of S or That
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int q = 0; q < 16; ++q)
      X[t][q] = (!s_wave && t * 32 + acc_row(q, g) == ncol) ? 1.f : 0.f;
  float lam = 0.f;

  for (int64_t c0 = t_begin; c0 < t_end; c0 += C) {
    const int len = (t_end - c0 < C) ? int(t_end - c0) : C;
    __syncthreads();  // the previous chunk is done with K^T and U

    // ---------------- stage K (row-major and transposed), V^T, gates
    for (int item = tid; item < (C / 2) * (DP / 8); item += NTH) {
      const int tp = item / (DP / 8), i0 = (item % (DP / 8)) * 8, t0 = 2 * tp;
      float ka[8], kb[8], va[8], vb[8];
      const int64_t row0 = (int64_t(b) * N + c0 + t0) * H + h;
      load8<INBF16>(a.k, row0 * dk + i0, t0 < len && i0 < dk, ka);
      load8<INBF16>(a.k, (row0 + H) * dk + i0, t0 + 1 < len && i0 < dk, kb);
      load8<INBF16>(a.v, row0 * dv + i0, t0 < len && i0 < dv, va);
      load8<INBF16>(a.v, (row0 + H) * dv + i0, t0 + 1 < len && i0 < dv, vb);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const __bf16 kah = to_bf16(ka[j]), kbh = to_bf16(kb[j]);
        const __bf16 vah = to_bf16(va[j]), vbh = to_bf16(vb[j]);
        Kr[t0 * KR + i0 + j] = kah;
        Kr[(t0 + 1) * KR + i0 + j] = kbh;
        st_pair(Kt + (i0 + j) * KT + t0, kah, kbh);
        st_pair(Vt + (i0 + j) * KT + t0, vah, vbh);
        if (!INBF16) {
          const __bf16 kal = to_bf16(ka[j] - from_bf16(kah)), kbl = to_bf16(kb[j] - from_bf16(kbh));
          const __bf16 val = to_bf16(va[j] - from_bf16(vah)), vbl = to_bf16(vb[j] - from_bf16(vbh));
          Kr[C * KR + t0 * KR + i0 + j] = kal;
          Kr[C * KR + (t0 + 1) * KR + i0 + j] = kbl;
          st_pair(Kt + DP * KT + (i0 + j) * KT + t0, kal, kbl);
          st_pair(Vt + DP * KT + (i0 + j) * KT + t0, val, vbl);
        }
      }
    }
    if (wave == 0) {
      const bool valid = lane < len;
      const int64_t gi = (int64_t(b) * N + c0 + lane) * H + h;
      float x = valid ? log2f(a.alpha[gi]) : 0.f;
      const float bt = valid ? (a.beta ? a.beta[gi] : 1.f) : 0.f;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      const float bend = __shfl(x, 63, 64);
      gb[lane] = bt;
      gr[lane] = exp2f(bend - x);
      if (lane == 0) gg[0] = exp2f(bend);
      lam += bend;
    }
    __syncthreads();

    // ---------------- L = diag(beta) strictly-lower(K K^T), fp32
    for (int tile = wave; tile < 4; tile += NW) {
      const int mt = tile >> 1, nt = tile & 1;
      if (nt > mt) {  // upper tile: zeros
        for (int e = lane; e < 32 * 32; e += 64)
          Lm[(mt * 32 + e / 32) * XL + nt * 32 + e % 32] = 0.f;
        continue;
      }
      f32x16 acc = zero16();
#pragma unroll
      for (int ks = 0; ks < DP / 16; ++ks) {
        const int kc = ks * 16 + 8 * g;
        const bf16x8 ah = lds_load8(Kr + (mt * 32 + cl) * KR + kc);
        const bf16x8 bh = lds_load8(Kr + (nt * 32 + cl) * KR + kc);
        if (!INBF16) {
          const bf16x8 al = lds_load8(Kr + C * KR + (mt * 32 + cl) * KR + kc);
          const bf16x8 bl = lds_load8(Kr + C * KR + (nt * 32 + cl) * KR + kc);
          acc = mfma32(al, bh, acc);
          acc = mfma32(ah, bl, acc);
        }
        acc = mfma32(ah, bh, acc);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = mt * 32 + acc_row(q, g), j = nt * 32 + cl;
        Lm[i * XL + j] = (j < i) ? gb[i] * acc[q] : 0.f;
      }
    }
    __syncthreads();

    // ---------------- X = (I + L)^{-1}: 16x16 diagonal blocks by substitution,
    // then block rows by  X_ij = -X_ii * sum_{m=j}^{i-1} L_im X_mj
    if (tid < 64) {
      const int bi = tid >> 4, cc = tid & 15, o = 16 * bi;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) s = fmaf(Lm[(o + r) * XL + o + m], x[m], s);
        x[r] = (r < cc) ? 0.f : ((r == cc) ? 1.f : -s);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Xm[(o + r) * XL + o + cc] = x[r];
    } else {
      // zero the strictly upper blocks (bi < bj)
      for (int e = tid - 64; e < 6 * 256; e += NTH - 64) {
        const int blk = e >> 8, r = (e >> 4) & 15, cc = e & 15;
        const int bi = (blk < 3) ? 0 : ((blk < 5) ? 1 : 2);
        const int bj = (blk < 3) ? blk + 1 : ((blk < 5) ? blk - 1 : 3);
        Xm[(16 * bi + r) * XL + 16 * bj + cc] = 0.f;
      }
    }
#pragma unroll 1
    for (int bi = 1; bi < 4; ++bi) {
      __syncthreads();
      for (int e = tid; e < bi * 256; e += NTH) {
        const int bj = e >> 8, r = (e >> 4) & 15, cc = e & 15;
        float s = 0.f;
        for (int m = bj; m < bi; ++m) {
#pragma unroll
          for (int q = 0; q < 16; ++q)
            s = fmaf(Lm[(16 * bi + r) * XL + 16 * m + q], Xm[(16 * m + q) * XL + 16 * bj + cc], s);
        }
        Ym[e] = s;
      }
      __syncthreads();
      for (int e = tid; e < bi * 256; e += NTH) {
        const int bj = e >> 8, r = (e >> 4) & 15, cc = e & 15;
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q)
          s = fmaf(Xm[(16 * bi + r) * XL + 16 * bi + q], Ym[bj * 256 + q * 16 + cc], s);
        Xm[(16 * bi + r) * XL + 16 * bj + cc] = -s;
      }
    }
    __syncthreads();
    const float gam = gg[0];

    // ---------------- U = X diag(beta) K (one 32x32 tile per wave) ;
    // S waves also form their strip of W = X diag(beta r) V
    {
      const int mt = wave / NT, nt = wave % NT;
      f32x16 acc = zero16();
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) {
        const int kc = ks * 16 + 8 * g;
        float av[8];
        const float* xr = Xm + (mt * 32 + cl) * XL + kc;
#pragma unroll
        for (int j = 0; j < 8; ++j) av[j] = xr[j] * gb[kc + j];
        bf16x8 ah, al;
        split8(av, ah, al);
        const bf16x8 kh = lds_load8(Kt + (nt * 32 + cl) * KT + kc);
        if (!INBF16) {
          const bf16x8 kl = lds_load8(Kt + DP * KT + (nt * 32 + cl) * KT + kc);
          acc = mfma32(ah, kl, acc);
        }
        acc = mfma32(al, kh, acc);
        acc = mfma32(ah, kh, acc);
      }
      // region 1 (K row-major) is dead since the K K^T step: overwrite with U
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = mt * 32 + acc_row(q, g), j = nt * 32 + cl;
        const __bf16 hi = to_bf16(acc[q]);
        Uh[i * KR + j] = hi;
        Ul[i * KR + j] = to_bf16(acc[q] - from_bf16(hi));
      }
    }
    f32x16 Wm[2];
    if (s_wave) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
          const int kc = ks * 16 + 8 * g;
          float av[8];
          const float* xr = Xm + (mt * 32 + cl) * XL + kc;
#pragma unroll
          for (int j = 0; j < 8; ++j) av[j] = xr[j] * (gb[kc + j] * gr[kc + j]);
          bf16x8 ah, al;
          split8(av, ah, al);
          const bf16x8 vh = lds_load8(Vt + (strip * 32 + cl) * KT + kc);
          if (!INBF16) {
            const bf16x8 vl = lds_load8(Vt + DP * KT + (strip * 32 + cl) * KT + kc);
            acc = mfma32(ah, vl, acc);
          }
          acc = mfma32(al, vh, acc);
          acc = mfma32(ah, vh, acc);
        }
        Wm[mt] = acc;
      }
    }
    __syncthreads();  // U complete

    // ---------------- chain update of this wave's strip
    // P = U * X_strip  (2 row tiles of 32 tokens), B operand from accumulators
    f32x16 P[2];
    P[0] = zero16();
    P[1] = zero16();
#pragma unroll
    for (int ks = 0; ks < 2 * NT; ++ks) {
      const int t = ks >> 1, hh = ks & 1;
      bf16x8 bhi, blo;
      split_acc_half(X[t], hh, bhi, blo);
      const int kc = 32 * t + 16 * hh + 4 * g;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int row = mt * 32 + cl;
        const bf16x8 ah = lds_perm8(Uh + row * KR, kc);
        const bf16x8 al = lds_perm8(Ul + row * KR, kc);
        P[mt] = mfma32(al, bhi, P[mt]);
        P[mt] = mfma32(ah, blo, P[mt]);
        P[mt] = mfma32(ah, bhi, P[mt]);
      }
    }
    // S strip:     M = W - gamma P ;  S = gamma S + K^T M
    // That strip:  M = -P          ;  That = That + K^T M
    if (s_wave) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q = 0; q < 16; ++q) P[mt][q] = fmaf(-gam, P[mt][q], Wm[mt][q]);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) X[t][q] *= gam;
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q = 0; q < 16; ++q) P[mt][q] = -P[mt][q];
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int mt = ks >> 1, hh = ks & 1;
      bf16x8 bhi, blo;
      split_acc_half(P[mt], hh, bhi, blo);
      const int kc = 32 * mt + 16 * hh + 4 * g;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const __bf16* kr = Kt + (t * 32 + cl) * KT;
        const bf16x8 kh = lds_perm8(kr, kc);
        if (!INBF16) {
          const bf16x8 kl = lds_perm8(kr + DP * KT, kc);
          X[t] = mfma32(kl, bhi, X[t]);
        }
        X[t] = mfma32(kh, blo, X[t]);
        X[t] = mfma32(kh, bhi, X[t]);
      }
    }
  }

  // ---------------- write the pair
  const int64_t unit = (int64_t(seg) * a.batch + b) * H + h;
  if (s_wave) {
    if (ncol < dv) {
      float* out = a.S0 + unit * int64_t(dk) * dv;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = t * 32 + acc_row(q, g);
          if (row < dk) out[int64_t(row) * dv + ncol] = X[t][q];
        }
    }
  } else if (ncol < dk) {
    float* out = a.T_hat + unit * int64_t(dk) * dk;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = t * 32 + acc_row(q, g);
        if (row < dk) out[int64_t(row) * dk + ncol] = X[t][q];
      }
  }
  if (tid == 0) a.log_scale[unit] = lam * kLn2;
}

template <int DP, bool INBF16>
hipError_t launch_dense_t(const BuildArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_seg) * a.batch * a.heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((build_dense_kernel<DP, INBF16>), dim3(unsigned(blocks)), dim3(4 * DP), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_dense(const BuildArgs& a, hipStream_t s) {
  const int d = a.dk > a.dv ? a.dk : a.dv;
  const int dp = d <= 32 ? 32 : (d <= 64 ? 64 : 128);
  // bf16 inputs take the producer/consumer kernel (k_build_dense_ws.hip)
  if (a.qkv_bf16) return launch_build_dense_ws(a, s);
  switch (dp) {
    case 32: return launch_dense_t<32, false>(a, s);
    case 64: return launch_dense_t<64, false>(a, s);
    default: return launch_dense_t<128, false>(a, s);
  }
}

}  // namespace pic
