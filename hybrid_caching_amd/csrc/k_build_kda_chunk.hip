// k_build_kda_chunk.hip -- chunked build of the KDA pairs on the matrix cores
// (bf16 k/v, fp16 operands, dk = dv = 128; PIC_PREC_FP16).
// [xix.ai HYPIC article (French), paragraph on linear layers: KDA among the
//  families whose states compose; T_C is the product of the segment's token
//  transitions and S(C|0) its final state from zero.]
//
// Per token T_t = (I - b_t k_t k_t^T) Diag(a_t) (a_t one gate per key
// channel).  Within a chunk of C = 32 tokens let g_t be the per-channel gate
// product from the chunk's start through token t and gamma = g_C.  Then
// X_t = Diag(g_t)^{-1} S_t follows a delta rule whose read key is
// k^_t = g_t (.) k_t and whose write key is k~_t = k_t / g_t:
//   X_t = X_{t-1} + b_t k~_t (v_t - X_{t-1}^T k^_t)^T.
// Its chunked (UT) form, with L = strictly-lower(K^ K~^T) and
// A = (I + diag(b) L)^{-1} diag(b):
//   E  = A (V - K^ S)
//   S' = Diag(gamma) S + K-^T E,        K-_t = (gamma / g_t) (.) k_t
//   T_chunk = Diag(gamma) - K-^T A K^
// Every factor of K^ and K- is a gate product (at most 1).  L_ts multiplies
// k_t (.) g_t / g_m by k_s (.) g_m / g_s with g_m the product through the
// chunk's middle, so each factor spans at most 16 tokens of decay (their
// product, g_t / g_s, is at most 1).  Inputs whose 16-token gate products
// leave fp16's range make those factors overflow; the stored values are then
// not finite and the overflow flag reports it.
//
// That.  The chunks' T_chunk are multiplied into XT, kept at a power-of-two
// scale per wave (re-normalised after every chunk, so that XT enters the next
// chunk's products as fp16 with its largest entry in [1/2, 1); a scaling of
// the columns commutes with the left products).  The per-token split of the KDA pair is
// applied once at the end: lambda_C = sum_t ln m_t (m_t the token's largest
// gate) and That_C = T_C / prod_t m_t, i.e. XT times one power of two.
//
// One workgroup of eight waves per (segment, layer, head): waves 0-3 hold
// columns [32w, 32w+32) of S, waves 4-7 columns [32(w-4), ..) of XT, in
// accumulators for the whole segment.  Per chunk: (1) every wave turns the
// gates of its eighth of the chunk's tokens (4 tokens, two channels per
// lane) into log2 prefix sums; (2) after a barrier, the prefix sums across
// eighths give g_t, gamma and g_m, and the waves write K^, K-, the two
// halves of L's factors and V (fp16, token-major) and issue the next chunk's
// loads; (3) wave 0 forms L on the matrix cores and inverts I + diag(b) L
// in fp32 by 16 x 16 blocks (one lane per column), while the others form
// Y = K^ S (S waves) or Y = K^ XT (XT waves); (4) the S waves form E = A (V - Y) and S <- gamma (.) S + K-^T E,
// the XT waves F = A Y and XT <- gamma (.) XT - K-^T F.  Three barriers per
// chunk.
#include <type_traits>

#include "mfma_util.hpp"
#include "pic_internal.hpp"

namespace pic {
namespace {

typedef _Float16 kf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 kf16x2 __attribute__((ext_vector_type(2)));
typedef short ki16x4 __attribute__((ext_vector_type(4)));
typedef short ki16x8 __attribute__((ext_vector_type(8)));
typedef unsigned ku32x4 __attribute__((ext_vector_type(4)));
typedef unsigned ku32x2 __attribute__((ext_vector_type(2)));

constexpr int KD = 128;          // head size (dk = dv)
constexpr int KC = 32;           // tokens per chunk
constexpr int KNT = KD / 32;     // row tiles of a column strip
constexpr int KRL = 152;         // row stride (halves) of the token-major fp16 tiles
constexpr int KLL = 36;          // row stride (floats) of L
constexpr int KAL = 40;          // row stride (halves) of A

constexpr int K_TILE = KC * KRL * 2;
constexpr int O_KH = 0;                       // K^   [C][KRL] fp16
constexpr int O_KB = O_KH + K_TILE;           // K-   [C][KRL]
constexpr int O_VH = O_KB + K_TILE;           // V    [C][KRL]
constexpr int O_KA = O_VH + K_TILE;           // k (.) g_t / g_m
constexpr int O_KCF = O_KA + K_TILE;          // k (.) g_m / g_t
constexpr int O_L = O_KCF + K_TILE;           // N^T [C][KLL] fp32, then X11^T [16][KLL]
constexpr int O_A = O_L + (KC + 16) * KLL * 4;  // A [C][KAL] fp16
constexpr int O_DG = O_A + KC * KAL * 2;      // gamma [KD] fp32
constexpr int O_QT = O_DG + KD * 4;           // per-wave totals of log2 gates [8][KD]
constexpr int O_BT = O_QT + 8 * KD * 4;       // beta of the chunk's tokens [C]
constexpr int O_MU = O_BT + KC * 4;           // per-wave sums of log2 m_t [8]
constexpr int K_LDS = O_MU + 32;
static_assert(K_LDS <= 80 * 1024, "two workgroups per CU");
static_assert(O_L % 16 == 0 && O_A % 16 == 0 && O_DG % 16 == 0 && O_QT % 16 == 0 &&
              O_BT % 16 == 0 && (KRL * 2) % 16 == 0, "alignment");

__device__ __forceinline__ f32x16 kmfma(const kf16x8& a, const kf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ unsigned kpk(float x0, float x1) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x0, x1}, kf16x2));
}
// accumulator registers 8h .. 8h+7 as an fp16 operand
__device__ __forceinline__ kf16x8 kacc8(const f32x16& a, int h) {
  ku32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = kpk(a[8 * h + 2 * j], a[8 * h + 2 * j + 1]);
  return __builtin_bit_cast(kf16x8, w);
}
// two bf16 values in a word -> floats
__device__ __forceinline__ float kbf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float kbf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
// the operand pieces of a permuted K-step from a row of fp16: positions
// p .. p+3 and p+8 .. p+11
__device__ __forceinline__ kf16x8 krow_perm(const _Float16* p) {
  const ku32x2 lo = *reinterpret_cast<const ku32x2*>(p);
  const ku32x2 hi = *reinterpret_cast<const ku32x2*>(p + 8);
  const ku32x4 w = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(kf16x8, w);
}
// transposed read: in each group of 16 lanes, lane i receives 16-bit element
// (i & 3) of the 8 bytes addressed by lane 4j + (i >> 2), j = 0..3
__device__ __forceinline__ ki16x4 ktr4(const _Float16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) ki16x4*)(p));
}
__device__ __forceinline__ float kf(short s) { return float(__builtin_bit_cast(_Float16, s)); }

__device__ __forceinline__ float klog2_gate(float x) {
  return __builtin_amdgcn_logf(__int_as_float(max(__float_as_int(x), 0x00800000)));
}
__device__ __forceinline__ float kexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// maximum over the 64 lanes (uniform result)
__device__ __forceinline__ float kwave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  const int xi = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

template <class T>
__device__ __forceinline__ T kgload(const T* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}

__global__ __launch_bounds__(512) void build_kda_chunk_kernel(BuildArgs a) {
  __shared__ __attribute__((aligned(16))) char sm[K_LDS];
  _Float16* Kh = reinterpret_cast<_Float16*>(sm + O_KH);
  _Float16* Kb = reinterpret_cast<_Float16*>(sm + O_KB);
  _Float16* Vh = reinterpret_cast<_Float16*>(sm + O_VH);
  _Float16* Ka = reinterpret_cast<_Float16*>(sm + O_KA);
  _Float16* Kc = reinterpret_cast<_Float16*>(sm + O_KCF);
  float* Lm = reinterpret_cast<float*>(sm + O_L);
  _Float16* Am = reinterpret_cast<_Float16*>(sm + O_A);
  float* Dg = reinterpret_cast<float*>(sm + O_DG);
  float* Qt = reinterpret_cast<float*>(sm + O_QT);
  float* Bt = reinterpret_cast<float*>(sm + O_BT);
  float* Mu = reinterpret_cast<float*>(sm + O_MU);

  const int H = a.heads, BH = a.batch * H;
  const int seg = seg_in_order(a, blockIdx.x / BH);
  const int bh = blockIdx.x % BH, b = bh / H, h = bh % H;
  const int64_t t_begin = seg_offset(a, seg), ntok = seg_offset(a, seg + 1) - t_begin;
  const int n = int((ntok + KC - 1) / KC);
  const int64_t unit = (int64_t(seg) * a.batch + b) * H + h;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 5, cl = lane & 31, G = lane >> 4;
  const bool tw = wave >= 4;        // an XT wave
  const int cw = wave & 3;          // its column block
  // token rows of this (segment, layer, head): row r of the segment is at
  // element (base + r H) D of k, v and alpha, and at base + r H of beta
  const int64_t base = (int64_t(b) * a.n_tokens + t_begin) * H + h;
  const __bf16* kb = static_cast<const __bf16*>(a.k) + base * KD;
  const __bf16* vb = static_cast<const __bf16*>(a.v) + base * KD;
  const float* ab = a.alpha + base * KD;
  const float* bb = a.beta ? a.beta + base : nullptr;
  auto chunk_len = [&](int ci) {
    const int64_t rest = ntok - int64_t(ci) * KC;
    return rest < KC ? int(rest) : KC;
  };

  // ---- state: columns [32 cw, 32 cw + 32) of S (waves 0-3) or XT (4-7)
  f32x16 X[KNT];
#pragma unroll
  for (int t = 0; t < KNT; ++t)
#pragma unroll
    for (int q = 0; q < 16; ++q)
      X[t][q] = (tw && t * 32 + acc_row(q, g) == cw * 32 + cl) ? 1.f : 0.f;
  int E = 0;          // XT waves: XT = T * 2^-E (T the unnormalised product)
  float musum = 0.f;  // sum of log2 m_t over this wave's tokens (uniform)

  // ---- raw inputs of a chunk in registers: this wave's eighth of the
  // tokens (4w .. 4w+3), channels 2 lane and 2 lane + 1
  constexpr int TW = KC / 8;
  const int tq = TW * wave;
  unsigned rk[TW], rv[TW];
  f32x2 ra[TW];
  float rb = 0.f;  // wave 0, lanes 0-31: beta of token lane
  auto load_raw = [&](int ci) __attribute__((always_inline)) {
    const int len = chunk_len(ci);
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      const int64_t r = int64_t(ci) * KC + min(tq + tt, len - 1);
      rk[tt] = kgload(reinterpret_cast<const unsigned*>(kb + r * H * KD) + lane);
      rv[tt] = kgload(reinterpret_cast<const unsigned*>(vb + r * H * KD) + lane);
      ra[tt] = kgload(reinterpret_cast<const f32x2*>(ab + r * H * KD) + lane);
    }
    if (wave == 0 && lane < KC) {
      const int64_t r = int64_t(ci) * KC + min(lane, len - 1);
      rb = bb ? kgload(bb + r * H) : 1.f;
    }
  };
  if (n > 0) load_raw(0);

#pragma unroll 1
  for (int ci = 0; ci < n; ++ci) {
    const int len = chunk_len(ci);
    // ---- (1) log2 gates of the wave's tokens; tokens past the end have gates 1
    float c0[TW], c1[TW];
    {
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int tt = 0; tt < TW; ++tt) {
        const bool ok = tq + tt < len;
        const float x0 = ok ? ra[tt][0] : 1.f, x1 = ok ? ra[tt][1] : 1.f;
        p0 += klog2_gate(x0);
        p1 += klog2_gate(x1);
        c0[tt] = p0;
        c1[tt] = p1;
        musum += klog2_gate(kwave_max(fmaxf(x0, x1)));
      }
      *reinterpret_cast<f32x2*>(Qt + wave * KD + 2 * lane) = (f32x2){p0, p1};
      if (wave == 0 && lane < KC) Bt[lane] = lane < len ? rb : 0.f;
    }
    __syncthreads();  // barrier 1: the waves' totals; the previous chunk's tiles are free

    // ---- (2) g_t, gamma, g_m; the chunk's operand tiles
    {
      float pre0 = 0.f, pre1 = 0.f, tot0 = 0.f, tot1 = 0.f, mid0 = 0.f, mid1 = 0.f;
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) {
        const f32x2 v = *reinterpret_cast<const f32x2*>(Qt + qq * KD + 2 * lane);
        if (qq < wave) {
          pre0 += v[0];
          pre1 += v[1];
        }
        if (qq < 4) {
          mid0 += v[0];
          mid1 += v[1];
        }
        tot0 += v[0];
        tot1 += v[1];
      }
      if (wave == 0) *reinterpret_cast<f32x2*>(Dg + 2 * lane) = (f32x2){kexp2(tot0), kexp2(tot1)};
#pragma unroll
      for (int tt = 0; tt < TW; ++tt) {
        const int t = tq + tt;
        const float l0 = pre0 + c0[tt], l1 = pre1 + c1[tt];
        const float k0 = kbf_lo(rk[tt]), k1 = kbf_hi(rk[tt]);
        const int at = t * KRL + 2 * lane;
        *reinterpret_cast<unsigned*>(Kh + at) = kpk(k0 * kexp2(l0), k1 * kexp2(l1));
        *reinterpret_cast<unsigned*>(Kb + at) = kpk(k0 * kexp2(tot0 - l0), k1 * kexp2(tot1 - l1));
        *reinterpret_cast<unsigned*>(Ka + at) = kpk(k0 * kexp2(l0 - mid0), k1 * kexp2(l1 - mid1));
        *reinterpret_cast<unsigned*>(Kc + at) = kpk(k0 * kexp2(mid0 - l0), k1 * kexp2(mid1 - l1));
        *reinterpret_cast<unsigned*>(Vh + at) = kpk(kbf_lo(rv[tt]), kbf_hi(rv[tt]));
      }
    }
    // the next chunk's inputs stream in while this one is applied
    if (ci + 1 < n) load_raw(ci + 1);
    __syncthreads();  // barrier 2: the chunk's tiles

    // ---- (3) wave 0: L and the triangular solve; the others: Y = K^ X
    f32x16 Y = zero16();
    auto form_y = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < 2 * KNT; ++ks) {
        const kf16x8 kh = krow_perm(Kh + cl * KRL + 16 * ks + 4 * g);
        Y = kmfma(kh, kacc8(X[ks >> 1], ks & 1), Y);
      }
    };
    if (wave == 0) {
      // L (rows t, columns s) = Ka Kc^T
      f32x16 Lacc = zero16();
#pragma unroll
      for (int ks = 0; ks < 2 * KNT; ++ks) {
        const kf16x8 x = *reinterpret_cast<const kf16x8*>(Ka + cl * KRL + 16 * ks + 8 * g);
        const kf16x8 y = *reinterpret_cast<const kf16x8*>(Kc + cl * KRL + 16 * ks + 8 * g);
        Lacc = kmfma(x, y, Lacc);
      }
      // Nt = (diag(beta) strictly-lower(L))^T: Nt[s][t] = beta_t L_ts for s < t
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int t = acc_row(q, g);
        Lm[cl * KLL + t] = cl < t ? Bt[t] * Lacc[q] : 0.f;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // X = (I + N)^{-1} by 16x16 blocks, each lane one column: lanes 0-15 the
      // columns of X00 = (I + N00)^{-1}, lanes 16-31 those of X11 (forward
      // substitution as rank-one updates: once x[s] is final, every later
      // x[t] -= N[t][s] x[s]); then lanes 0-15 form X10 = -X11 (N10 X00).
      const int j = cl & 15, o = cl & 16;
      float x[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) x[t] = (t == j) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < 15; ++s) {
        const float* nrow = Lm + (o + s) * KLL + o;
#pragma unroll
        for (int t4 = s / 4; t4 < 4; ++t4) {
          const float4 nv = *reinterpret_cast<const float4*>(nrow + 4 * t4);
          const float n4[4] = {nv.x, nv.y, nv.z, nv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * t4 + e > s) x[4 * t4 + e] -= n4[e] * x[s];
        }
      }
      // X11 columns, transposed (row u = column u of X11), for lanes 0-15
      float* X11t = Lm + KC * KLL;  // rows 32 .. 47 of the L buffer
      if (g == 0 && o == 16) {
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
          *reinterpret_cast<float4*>(X11t + j * KLL + 4 * t4) =
              make_float4(x[4 * t4], x[4 * t4 + 1], x[4 * t4 + 2], x[4 * t4 + 3]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      float x10[16];
      if (o == 0) {
        // m = N10 X00[:, j]: m[t] = sum_s N[16 + t][s] x[s]
        float m[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) m[t] = 0.f;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const float* nrow = Lm + s * KLL + 16;
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4) {
            const float4 nv = *reinterpret_cast<const float4*>(nrow + 4 * t4);
            m[4 * t4 + 0] += nv.x * x[s];
            m[4 * t4 + 1] += nv.y * x[s];
            m[4 * t4 + 2] += nv.z * x[s];
            m[4 * t4 + 3] += nv.w * x[s];
          }
        }
        // x10 = -X11 m: x10[t] = -sum_u X11[t][u] m[u]
#pragma unroll
        for (int t = 0; t < 16; ++t) x10[t] = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float* xr = X11t + u * KLL;
#pragma unroll
          for (int t4 = u / 4; t4 < 4; ++t4) {
            const float4 xv = *reinterpret_cast<const float4*>(xr + 4 * t4);
            x10[4 * t4 + 0] -= xv.x * m[u];
            x10[4 * t4 + 1] -= xv.y * m[u];
            x10[4 * t4 + 2] -= xv.z * m[u];
            x10[4 * t4 + 3] -= xv.w * m[u];
          }
        }
      }
      // A = X diag(beta): column cl scaled by beta_cl
      const float bj = Bt[cl];
      if (g == 0) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          Am[t * KAL + cl] = static_cast<_Float16>(o == 0 ? x[t] * bj : 0.f);
          Am[(16 + t) * KAL + cl] = static_cast<_Float16>((o == 0 ? x10[t] : x[t]) * bj);
        }
      }
      form_y();
    } else {
      form_y();
    }
    __syncthreads();  // barrier 3: A

    // ---- (4) S waves: E = A (V - Y), S <- gamma (.) S + K-^T E;
    //          XT waves: F = A Y, XT <- gamma (.) XT - K-^T F
    f32x16 Ea = zero16();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const kf16x8 am = krow_perm(Am + cl * KAL + 16 * hh + 4 * g);
      if (!tw) {
        // V at tokens kperm(hh, g, 0..7), column 32 cw + cl
        const int r0 = 16 * hh + 4 * g + ((lane & 15) >> 2);
        const int col = 32 * cw + 16 * (G & 1) + 4 * (lane & 3);
        const ki16x4 v0 = ktr4(Vh + r0 * KRL + col);
        const ki16x4 v1 = ktr4(Vh + (r0 + 8) * KRL + col);
        ku32x4 w;
        w[0] = kpk(kf(v0[0]) - Y[8 * hh + 0], kf(v0[1]) - Y[8 * hh + 1]);
        w[1] = kpk(kf(v0[2]) - Y[8 * hh + 2], kf(v0[3]) - Y[8 * hh + 3]);
        w[2] = kpk(kf(v1[0]) - Y[8 * hh + 4], kf(v1[1]) - Y[8 * hh + 5]);
        w[3] = kpk(kf(v1[2]) - Y[8 * hh + 6], kf(v1[3]) - Y[8 * hh + 7]);
        Ea = kmfma(am, __builtin_bit_cast(kf16x8, w), Ea);
      } else {
        Ea = kmfma(am, kacc8(Y, hh), Ea);
      }
    }
#pragma unroll
    for (int t = 0; t < KNT; ++t) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 d4 = *reinterpret_cast<const float4*>(Dg + 32 * t + 8 * q4 + 4 * g);
        X[t][4 * q4 + 0] *= d4.x;
        X[t][4 * q4 + 1] *= d4.y;
        X[t][4 * q4 + 2] *= d4.z;
        X[t][4 * q4 + 3] *= d4.w;
      }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const kf16x8 eb = tw ? -kacc8(Ea, hh) : kacc8(Ea, hh);
      const int r0 = 16 * hh + 4 * g + ((lane & 15) >> 2);
#pragma unroll
      for (int t = 0; t < KNT; ++t) {
        // K-^T rows = channels 32t + cl, tokens kperm(hh, g, 0..7)
        const int col = 32 * t + 16 * (G & 1) + 4 * (lane & 3);
        const ki16x4 k0 = ktr4(Kb + r0 * KRL + col);
        const ki16x4 k1 = ktr4(Kb + (r0 + 8) * KRL + col);
        const ki16x8 kk = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
        X[t] = kmfma(__builtin_bit_cast(kf16x8, kk), eb, X[t]);
      }
    }
    // keep XT inside fp16's range as an operand
    if (tw) {
      float m = 0.f;
#pragma unroll
      for (int t = 0; t < KNT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(X[t][q]));
      m = kwave_max(m);
      int e;
      (void)frexpf(m, &e);
      e = (m > 0.f) ? (e < -120 ? -120 : e) : 0;
      const float sc = ldexpf(1.f, -e);
#pragma unroll
      for (int t = 0; t < KNT; ++t) X[t] *= sc;
      E += e;
    }
  }

  // ---- write-out: S(C|0); That_C = XT 2^(E - sum log2 m); lambda_C
  if (lane == 0) Mu[wave] = musum;
  __syncthreads();
  float mtot = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) mtot += Mu[w];
  const float sc = tw ? exp2f(float(E) - mtot) : 1.f;
  bool bad = false;
  float* out = (tw ? a.T_hat : a.S0) + unit * int64_t(KD) * KD;
  const int col = 32 * cw + cl;
#pragma unroll
  for (int t = 0; t < KNT; ++t)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 32 * t + acc_row(q, g);
      const float v = X[t][q] * sc;
      bad |= not_finite(v);
      out[int64_t(row) * KD + col] = v;
    }
  report_nonfinite(a.nonfinite, bad);
  if (threadIdx.x == 0) a.log_scale[unit] = mtot * kLn2;
}

}  // namespace

hipError_t launch_build_kda_chunk(const BuildArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_seg) * a.batch * a.heads;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(build_kda_chunk_kernel, dim3(unsigned(blocks)), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace pic
