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
// accumulators for the whole segment.  Each wave owns a quarter of the
// chunk's tokens when staging (4 tokens, two channels per lane).  The chunks
// run through a two-stage software pipeline with two barriers per chunk and
// the operand tiles double-buffered in LDS:
//   stage 1 of chunk i: every wave forms Y = K^ S (or K^ XT) and the per-wave
//     gate products of chunk i+1; wave 0 also forms L of chunk i on the
//     matrix cores and inverts I + diag(b) L in fp32 by 16 x 16 blocks;
//   stage 2 of chunk i: the S waves form E = A (V - Y) and
//     S <- gamma (.) S + K-^T E, the XT waves F = A Y and
//     XT <- gamma (.) XT - K-^T F; every wave then writes its tokens' rows of
//     chunk i+1's tiles (K^, K-, the two halves of L's factors, V) and issues
//     the loads of chunk i+2.
// So the vector work of staging a chunk overlaps the matrix-core work of
// applying the one before.
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
// The K- and V tiles, read only transposed (ds_read_b64_tr_b16), have rows of
// KTL = 144 halves (288 bytes) with their 16-column pieces permuted: piece p
// (columns 16p .. 16p+15) at slot (p >> 1) + 4 (p & 1).  A transposed read
// serves two 16-lane groups together, reading the two 16-column halves of one
// 32-column tile from the same four rows; with the 288-byte stride the four
// rows of a group fall 8 banks apart and the permutation puts the other
// group's half 32 banks further, so the two groups never share a bank.
constexpr int KTL = 144;
constexpr int KLL = 36;          // row stride (floats) of L
constexpr int KAL = 40;          // row stride (halves) of A
constexpr int KXS = 24;          // row stride (halves) of the diagonal blocks' rows

constexpr int K_TILE = KC * KRL * 2;
// one buffer of a chunk's tiles (token-major rows of KRL halves)
constexpr int T_KH = 0;                 // K^ = k (.) g_t          fp16
constexpr int KT_TILE = KC * KTL * 2;
constexpr int T_KB = T_KH + K_TILE;     // K- = k (.) gamma / g_t  fp16 (KTL rows)
constexpr int T_VR = T_KB + KT_TILE;    // V                        bf16 as loaded (KTL rows)
constexpr int T_KA = T_VR + KT_TILE;    // k (.) g_t / g_m          fp16
constexpr int T_KC = T_KA + K_TILE;     // k (.) g_m / g_t          fp16
constexpr int T_DG = T_KC + K_TILE;     // gamma [KD] fp32
constexpr int T_BT = T_DG + KD * 4;     // beta of the chunk's tokens [C] (0 past the end)
constexpr int T_QT = T_BT + KC * 4;     // per-wave gate products [8][KD]
constexpr int T_BUF = T_QT + 8 * KD * 4;
constexpr int O_L = 2 * T_BUF;                  // L [C][KLL] fp32, then the solve's rows [C][KXS] fp16
constexpr int O_A = O_L + (KC + 16) * KLL * 4;  // A [C][KAL] fp16
constexpr int O_MU = O_A + KC * KAL * 2;        // per-wave sums of log2 m_t [8]
constexpr int K_LDS = O_MU + 32;
static_assert(K_LDS <= 160 * 1024, "one workgroup per CU");
static_assert(T_BUF % 16 == 0 && T_DG % 16 == 0 && T_BT % 16 == 0 && T_QT % 16 == 0 &&
              O_L % 16 == 0 && O_A % 16 == 0 && (KRL * 2) % 16 == 0, "alignment");
static_assert(KC * KXS * 2 <= 16 * KLL * 4, "the solve's rows fit behind L");

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

// maximum of x over lane pairs (l, l ^ 16) and then (l, l ^ 32), for x >= 0:
// the 16-lane swap of two copies of x gives the even rows in one result and
// the odd rows in the other, the 32-lane swap the low and the high halves, so
// the larger of the two results pairs every lane with its partner.  The
// comparison is on the bit patterns as signed integers, which orders
// non-negative floats as their values do (and puts any negative value below
// them); the compiler folds a float maximum of the two swap results to the
// first of them.
__device__ __forceinline__ float kswap_max(float x) {
  const int a = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
  const int m = max(int(r[0]), int(r[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  return __builtin_bit_cast(float, max(int(q[0]), int(q[1])));
}

// maximum over the 64 lanes (uniform result): within rows of 16 by DPP,
// across rows by the 16- and 32-lane swaps
__device__ __forceinline__ float kwave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  x = kswap_max(x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// maxima over the 64 lanes of four values per lane (one per token): the quad
// exchanges halve the tokens twice, then the lanes with the same lane % 4
// combine; lane l ends with the maximum of token 2 (l & 1) + ((l >> 1) & 1)
__device__ __forceinline__ float ktoken_max4(const float (&v)[4], int lane) {
  const bool o1 = lane & 1, o2 = lane & 2;
  float a = o1 ? v[2] : v[0], b = o1 ? v[3] : v[1];
  const float sa = o1 ? v[0] : v[2], sb = o1 ? v[1] : v[3];
  a = fmaxf(a, dpp_f<0xB1>(sa));  // lane ^ 1
  b = fmaxf(b, dpp_f<0xB1>(sb));
  float k = o2 ? b : a;
  k = fmaxf(k, dpp_f<0x4E>(o2 ? a : b));  // lane ^ 2
  k = fmaxf(k, dpp_f<0x124>(k));          // row_ror:4
  k = fmaxf(k, dpp_f<0x128>(k));          // row_ror:8
  return kswap_max(k);  // across rows
}

// One row of X_bb = (I + N_bb)^{-1} for a 16 x 16 diagonal block, from
// X_bb (I + N_bb) = I with N = diag(beta) L: steps i = 15 .. 1,
// acc[r] -= (acc[i] beta_i) L[i][r] for r < i.  Row i of the block of L is a
// broadcast read issued KPF steps ahead of its use.
constexpr int KPF = 3;
__device__ __forceinline__ void ksubst16(float (&acc)[16], const float* lrow0, const float (&bt)[16]) {
  float4 buf[KPF + 1][4];
#pragma unroll
  for (int p = 0; p < KPF; ++p)
#pragma unroll
    for (int r4 = 0; r4 < (15 - p + 3) / 4; ++r4)
      buf[p][r4] = *reinterpret_cast<const float4*>(lrow0 + (15 - p) * KLL + 4 * r4);
#pragma unroll
  for (int i = 15; i >= 1; --i) {
    const int slot = (15 - i) % (KPF + 1);
    const int ip = i - KPF;
    if (ip >= 1) {
      const int ps = (15 - ip) % (KPF + 1);
#pragma unroll
      for (int r4 = 0; r4 < (ip + 3) / 4; ++r4)
        buf[ps][r4] = *reinterpret_cast<const float4*>(lrow0 + ip * KLL + 4 * r4);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float x = acc[i] * bt[i];
    // highest r first: acc[i - 1] is the next step's pivot
#pragma unroll
    for (int r = i - 1; r >= 0; --r) {
      const float4& b4 = buf[slot][r >> 2];
      const float nv = (r & 3) == 0 ? b4.x : (r & 3) == 1 ? b4.y : (r & 3) == 2 ? b4.z : b4.w;
      acc[r] = fmaf(-nv, x, acc[r]);
    }
  }
}

typedef _Float16 kf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 kmfma16x32(const kf16x8& a, const kf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 kmfma16(const kf16x4& a, const kf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ kf16x4 kh4(float x0, float x1, float x2, float x3) {
  const ku32x2 w = {kpk(x0, x1), kpk(x2, x3)};
  return __builtin_bit_cast(kf16x4, w);
}

__device__ __forceinline__ int64_t krfl64(int64_t v) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(uint64_t(v) >> 32))));
  return int64_t((uint64_t(hi) << 32) | lo);
}

template <class T>
__device__ __forceinline__ T kgload(const T* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}

__global__ __launch_bounds__(512) void build_kda_chunk_kernel(BuildArgs a) {
  __shared__ __attribute__((aligned(16))) char sm[K_LDS];
  float* Lm = reinterpret_cast<float*>(sm + O_L);
  _Float16* Am = reinterpret_cast<_Float16*>(sm + O_A);
  float* Mu = reinterpret_cast<float*>(sm + O_MU);
  auto kt = [&](int buf, int off) { return reinterpret_cast<_Float16*>(sm + buf * T_BUF + off); };
  auto kf32 = [&](int buf, int off) { return reinterpret_cast<float*>(sm + buf * T_BUF + off); };

  const int H = a.heads, BH = a.batch * H;
  const int seg = seg_in_order(a, int(build_unit(a, blockIdx.x) / BH));
  const int bh = int(build_unit(a, blockIdx.x) % BH), b = bh / H, h = bh % H;
  // segment bounds as wave-uniform values (scalar addressing of the token rows)
  const int64_t t_begin = krfl64(seg_offset(a, seg));
  const int64_t ntok = krfl64(seg_offset(a, seg + 1)) - t_begin;
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
  float musum = 0.f;  // lanes 0-3: sum of log2 m_t over one token slot of this wave

  // ---- raw inputs of a chunk in registers, channels 2 lane and 2 lane + 1
  // of this wave's tokens: wave 0 (which inverts the chunk's system) stages
  // none, waves 1-3 the first half of the chunk (5, 5 and 6 tokens), waves
  // 4-7 four tokens each of the second half
  constexpr int TW = 6;
  const int tcnt = wave == 0 ? 0 : wave == 3 ? 6 : wave < 3 ? 5 : 4;
  const int tq = wave < 4 ? 5 * (wave - 1) : 16 + 4 * (wave - 4);
  unsigned rk[TW], rv[TW];
  f32x2 ra[TW];
  float rb = 0.f;  // wave 0, lanes 0-31: beta of token lane
  auto load_raw = [&](int ci) __attribute__((always_inline)) {
    const int len = chunk_len(ci);
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      if (tt >= tcnt) break;
      // row pointers as wave-uniform (scalar) bases, the lane as the offset
      const int64_t r = int64_t(ci) * KC + min(tq + tt, len - 1);
      const int64_t e = krfl64(r * H * KD);
      rk[tt] = kgload(reinterpret_cast<const unsigned*>(kb + e) + lane);
      rv[tt] = kgload(reinterpret_cast<const unsigned*>(vb + e) + lane);
      ra[tt] = kgload(reinterpret_cast<const f32x2*>(ab + e) + lane);
    }
    if (wave == 0 && lane < KC) {
      const int64_t r = int64_t(ci) * KC + min(lane, len - 1);
      rb = bb ? kgload(bb + r * H) : 1.f;
    }
  };

  // ---- gate products of chunk ci's tokens (gates past the end are 1): the
  // wave's totals to Qt, beta to Bt, and the tokens' largest gates into musum
  auto gates = [&](int ci) __attribute__((always_inline)) {
    const int len = chunk_len(ci), buf = ci & 1;
    float p0 = 1.f, p1 = 1.f, mx[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) mx[tt] = 1.f;  // (log2 1 = 0: no contribution)
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      if (tt >= tcnt) break;
      if (tq + tt >= len) ra[tt] = (f32x2){1.f, 1.f};  // (wave-uniform)
      p0 *= ra[tt][0];
      p1 *= ra[tt][1];
      mx[tt] = fmaxf(ra[tt][0], ra[tt][1]);
    }
    *reinterpret_cast<f32x2*>(kf32(buf, T_QT) + wave * KD + 2 * lane) = (f32x2){p0, p1};
    if (wave == 0 && lane < KC) kf32(buf, T_BT)[lane] = lane < len ? rb : 0.f;
    // m_t of the wave's tokens, four at a time: lanes 0-3 each count one
    if (tcnt > 0) {
      const float m0 = ktoken_max4(*reinterpret_cast<const float(*)[4]>(mx), lane);
      float lg = __builtin_amdgcn_logf(m0);
      if (tcnt > 4) lg += __builtin_amdgcn_logf(ktoken_max4(*reinterpret_cast<const float(*)[4]>(mx + 4), lane));
      musum += lane < 4 ? lg : 0.f;
    }
  };

  // ---- chunk ci's tiles from the raw registers and the waves' gate
  // products: g_t, gamma = g_31 and g_m = g_15 per channel
  auto tiles = [&](int ci) __attribute__((always_inline)) {
    const int buf = ci & 1;
    const float* qt = kf32(buf, T_QT);
    float pre0 = 1.f, pre1 = 1.f, tot0 = 1.f, tot1 = 1.f, mid0 = 1.f, mid1 = 1.f;
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(qt + qq * KD + 2 * lane);
      if (qq == 4) {
        mid0 = tot0;
        mid1 = tot1;
      }
      if (qq == wave) {  // the product over the waves before this one
        pre0 = tot0;
        pre1 = tot1;
      }
      tot0 *= v[0];
      tot1 *= v[1];
    }
    if (wave == 0) *reinterpret_cast<f32x2*>(kf32(buf, T_DG) + 2 * lane) = (f32x2){tot0, tot1};
    const float im0 = __builtin_amdgcn_rcpf(mid0), im1 = __builtin_amdgcn_rcpf(mid1);
    _Float16* kh = kt(buf, T_KH);
    _Float16* kbr = kt(buf, T_KB);
    _Float16* vr = kt(buf, T_VR);
    _Float16* ka = kt(buf, T_KA);
    _Float16* kc = kt(buf, T_KC);
    float g0 = pre0, g1 = pre1;
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      if (tt >= tcnt) break;
      g0 *= ra[tt][0];  // gates past the end were set to 1 by gates()
      g1 *= ra[tt][1];
      const float r0 = __builtin_amdgcn_rcpf(g0), r1 = __builtin_amdgcn_rcpf(g1);
      const float k0 = kbf_lo(rk[tt]), k1 = kbf_hi(rk[tt]);
      const float kg0 = k0 * g0, kg1 = k1 * g1, kr0 = k0 * r0, kr1 = k1 * r1;
      const int at = (tq + tt) * KRL + 2 * lane;
      // (K- and V rows: channels 2 lane, 2 lane + 1 at their permuted slot)
      const int att = (tq + tt) * KTL + 16 * ((lane >> 4) + 4 * ((lane >> 3) & 1)) + 2 * (lane & 7);
      *reinterpret_cast<unsigned*>(kh + at) = kpk(kg0, kg1);
      *reinterpret_cast<unsigned*>(kbr + att) = kpk(kr0 * tot0, kr1 * tot1);
      *reinterpret_cast<unsigned*>(ka + at) = kpk(kg0 * im0, kg1 * im1);
      *reinterpret_cast<unsigned*>(kc + at) = kpk(kr0 * mid0, kr1 * mid1);
      *reinterpret_cast<unsigned*>(vr + att) = rv[tt];
    }
  };

  // ---- pipeline prologue: chunk 0's tiles, chunk 1's loads
  if (n > 0) {
    load_raw(0);
    gates(0);
    __syncthreads();
    tiles(0);
    if (n > 1) load_raw(1);
    __syncthreads();
  }

#pragma unroll 1
  for (int ci = 0; ci < n; ++ci) {
    const int cb = ci & 1;
    const _Float16* Kh = kt(cb, T_KH);
    const _Float16* Kb = kt(cb, T_KB);
    const _Float16* Vr = kt(cb, T_VR);
    const float* Dg = kf32(cb, T_DG);
    const float* Bt = kf32(cb, T_BT);

    // Y = K^ X (before the chunk's decay), then X <- gamma (.) X
    f32x16 Y = zero16();
    auto form_y = [&]() __attribute__((always_inline)) {
      f32x16 Y1 = zero16();
#pragma unroll
      for (int ks = 0; ks < 2 * KNT; ks += 2) {
        const kf16x8 kh0 = krow_perm(Kh + cl * KRL + 16 * ks + 4 * g);
        const kf16x8 kh1 = krow_perm(Kh + cl * KRL + 16 * ks + 16 + 4 * g);
        Y = kmfma(kh0, kacc8(X[ks >> 1], 0), Y);
        Y1 = kmfma(kh1, kacc8(X[ks >> 1], 1), Y1);
      }
      Y += Y1;
    };
    auto form_y_decay = [&]() __attribute__((always_inline)) {
      form_y();
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
    };

    // ================= stage 1: Y and the decay (wave 0: L and A);
    // the gate products of chunk ci+1
    if (tw) {
      // keep XT inside fp16's range as an operand: rescaled by a power of
      // two when its largest entry has fallen below 2^-6, so that every
      // chunk's products see it within [2^-6, 1]
      float m0 = 0.f, m1 = 0.f;
#pragma unroll
      for (int t = 0; t < KNT; ++t)
#pragma unroll
        for (int q = 0; q < 16; q += 2) {
          m0 = fmaxf(m0, fabsf(X[t][q]));
          m1 = fmaxf(m1, fabsf(X[t][q + 1]));
        }
      const float m = kwave_max(fmaxf(m0, m1));
      if (m < 0.015625f) {
        int e;
        (void)frexpf(m, &e);
        e = (m > 0.f) ? (e < -120 ? -120 : e) : 0;
        const float sc = ldexpf(1.f, -e);
#pragma unroll
        for (int t = 0; t < KNT; ++t) X[t] *= sc;
        E += e;
      }
    }
    if (wave != 0) form_y_decay();
    if (wave == 0) {
      const _Float16* Ka = kt(cb, T_KA);
      const _Float16* Kc = kt(cb, T_KC);
      // the three 16 x 16 blocks of L = Ka Kc^T that the solve reads (rows
      // t, columns s: blocks 00, 10, 11), three independent 16x16x32
      // product chains; lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16]
      // and D[4(l/16)+e][l%16]
      {
        const int m = lane & 15, kq = lane >> 4;
        f32x4 l00 = {0.f, 0.f, 0.f, 0.f}, l10 = l00, l11 = l00;
#pragma unroll
        for (int ks = 0; ks < KNT; ++ks) {
          const int c = 32 * ks + 8 * kq;
          const kf16x8 a0 = *reinterpret_cast<const kf16x8*>(Ka + m * KRL + c);
          const kf16x8 a1 = *reinterpret_cast<const kf16x8*>(Ka + (16 + m) * KRL + c);
          const kf16x8 b0 = *reinterpret_cast<const kf16x8*>(Kc + m * KRL + c);
          const kf16x8 b1 = *reinterpret_cast<const kf16x8*>(Kc + (16 + m) * KRL + c);
          l00 = kmfma16x32(a0, b0, l00);
          l10 = kmfma16x32(a1, b0, l10);
          l11 = kmfma16x32(a1, b1, l11);
        }
        // rows of L: Lm[t][s] (only s < t is read)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * kq + e;
          Lm[r * KLL + m] = l00[e];
          Lm[(16 + r) * KLL + m] = l10[e];
          Lm[(16 + r) * KLL + 16 + m] = l11[e];
        }
      }
      // (I + diag(beta) L)^{-1} by 16 x 16 blocks.  Diagonal blocks: lane
      // 16 blk + jr (and its copy 32 lanes up) computes row jr of X_bb.
      const int blk = (lane >> 4) & 1, jr = lane & 15;
      float bt[16], acc[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 b4 = *reinterpret_cast<const float4*>(Bt + 16 * blk + 4 * q4);
        bt[4 * q4] = b4.x;
        bt[4 * q4 + 1] = b4.y;
        bt[4 * q4 + 2] = b4.z;
        bt[4 * q4 + 3] = b4.w;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = (r == jr) ? 1.f : 0.f;
      ksubst16(acc, Lm + 16 * blk * KLL + 16 * blk, bt);
      _Float16* Xs = reinterpret_cast<_Float16*>(Lm + KC * KLL);  // rows of X_00, X_11 (fp16)
      if (g == 0) {
        _Float16* xr = Xs + (16 * blk + jr) * KXS;
        *reinterpret_cast<ku32x4*>(xr) = (ku32x4){kpk(acc[0], acc[1]), kpk(acc[2], acc[3]),
                                                  kpk(acc[4], acc[5]), kpk(acc[6], acc[7])};
        *reinterpret_cast<ku32x4*>(xr + 8) =
            (ku32x4){kpk(acc[8], acc[9]), kpk(acc[10], acc[11]), kpk(acc[12], acc[13]),
                     kpk(acc[14], acc[15])};
      }
      // off-diagonal block X_10 = -X_11 (N_10 X_00): two 16x16x16 products;
      // lane l holds A[l%16][4(l/16)+e], B[4(l/16)+e][l%16], D[4(l/16)+e][l%16]
      const int m = lane & 15, kq = lane >> 4;
      f32x4 x10;
      {
        const float4 l4 = *reinterpret_cast<const float4*>(Lm + (16 + m) * KLL + 4 * kq);
        const float bm = Bt[16 + m];
        const kf16x4 n10 = kh4(bm * l4.x, bm * l4.y, bm * l4.z, bm * l4.w);
        const kf16x4 x00 = __builtin_bit_cast(kf16x4, ktr4(Xs + (4 * kq + (m >> 2)) * KXS + 4 * (m & 3)));
        const kf16x4 x11 = *reinterpret_cast<const kf16x4*>(Xs + (16 + m) * KXS + 4 * kq);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 y = kmfma16(n10, x00, z);
        x10 = kmfma16(x11, kh4(y[0], y[1], y[2], y[3]), z);
      }
      // A = X diag(beta): the diagonal blocks' rows (and zeros right of X_00),
      // then X_10
      if (g == 0) {
        _Float16* arow = Am + (16 * blk + jr) * KAL;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          const int k = 8 * h8;
          *reinterpret_cast<ku32x4*>(arow + 16 * blk + k) =
              (ku32x4){kpk(acc[k] * bt[k], acc[k + 1] * bt[k + 1]),
                       kpk(acc[k + 2] * bt[k + 2], acc[k + 3] * bt[k + 3]),
                       kpk(acc[k + 4] * bt[k + 4], acc[k + 5] * bt[k + 5]),
                       kpk(acc[k + 6] * bt[k + 6], acc[k + 7] * bt[k + 7])};
        }
        if (blk == 0) {
          const ku32x4 z4 = {0u, 0u, 0u, 0u};
          *reinterpret_cast<ku32x4*>(arow + 16) = z4;
          *reinterpret_cast<ku32x4*>(arow + 24) = z4;
        }
      }
      {
        const float bn = Bt[m];
#pragma unroll
        for (int e = 0; e < 4; ++e) Am[(16 + 4 * kq + e) * KAL + m] = static_cast<_Float16>(-x10[e] * bn);
      }
    }
    if (ci + 1 < n) gates(ci + 1);
    __syncthreads();  // A of chunk ci; the gate products of chunk ci+1

    // ================= stage 2: the state update; chunk ci+1's tiles
    if (wave == 0) form_y_decay();
    f32x16 Ea = zero16();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const kf16x8 am = krow_perm(Am + cl * KAL + 16 * hh + 4 * g);
      if (!tw) {
        // V at tokens kperm(hh, g, 0..7), column 32 cw + cl (bf16)
        const int r0 = 16 * hh + 4 * g + ((lane & 15) >> 2);
        const int col = 16 * cw + 64 * (G & 1) + 4 * (lane & 3);  // (permuted slots)
        const ki16x4 v0 = ktr4(Vr + r0 * KTL + col);
        const ki16x4 v1 = ktr4(Vr + (r0 + 8) * KTL + col);
        auto bf = [](short x) { return __uint_as_float(uint32_t(uint16_t(x)) << 16); };
        ku32x4 w;
        w[0] = kpk(bf(v0[0]) - Y[8 * hh + 0], bf(v0[1]) - Y[8 * hh + 1]);
        w[1] = kpk(bf(v0[2]) - Y[8 * hh + 2], bf(v0[3]) - Y[8 * hh + 3]);
        w[2] = kpk(bf(v1[0]) - Y[8 * hh + 4], bf(v1[1]) - Y[8 * hh + 5]);
        w[3] = kpk(bf(v1[2]) - Y[8 * hh + 6], bf(v1[3]) - Y[8 * hh + 7]);
        Ea = kmfma(am, __builtin_bit_cast(kf16x8, w), Ea);
      } else {
        Ea = kmfma(am, kacc8(Y, hh), Ea);
      }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const kf16x8 eb = tw ? -kacc8(Ea, hh) : kacc8(Ea, hh);
      const int r0 = 16 * hh + 4 * g + ((lane & 15) >> 2);
#pragma unroll
      for (int t = 0; t < KNT; ++t) {
        // K-^T rows = channels 32t + cl, tokens kperm(hh, g, 0..7)
        const int col = 16 * t + 64 * (G & 1) + 4 * (lane & 3);  // (permuted slots)
        const ki16x4 k0 = ktr4(Kb + r0 * KTL + col);
        const ki16x4 k1 = ktr4(Kb + (r0 + 8) * KTL + col);
        const ki16x8 kk = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
        X[t] = kmfma(__builtin_bit_cast(kf16x8, kk), eb, X[t]);
      }
    }
    if (ci + 1 < n) {
      tiles(ci + 1);
      if (ci + 2 < n) load_raw(ci + 2);
    }
    __syncthreads();  // chunk ci+1's tiles; this chunk's buffers are free
  }

  // ---- write-out: S(C|0); That_C = XT 2^(E - sum log2 m); lambda_C
  {
    const int mi = __builtin_bit_cast(int, musum);
    const float m4 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(mi, 0)) +
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(mi, 1)) +
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(mi, 2)) +
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(mi, 3));
    if (lane == 0) Mu[wave] = m4;
  }
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
