// k_dense_fp16.hip -- the independent prefill of every segment with per-token
// outputs o_t = S_t^T q_t, for the dense gated-delta form at fp16 operand
// precision (bf16 q/k/v), with or without That: the computation in which a
// segment's pair (lambda_C, That_C, S(C|0)) is built at its first prefill.
// [xix.ai HYPIC article (French), paragraph on linear layers: T_C as the
//  product of the segment's token transitions and S(C|0) from a zero start;
//  remio.ai HYPIC article (Japanese), section on how HYPIC composes
//  linear-attention states: the pair is built at the segment's first prefill.]
//
// Chunked form.  Within a sub-chunk of 32 tokens with inclusive gate products
// g_t and total gamma, dividing by the gates turns the gated delta rule into
// the plain one, whose product of rank-one factors is I - K^T A K with
//   X = (I + diag(beta) strictly-lower(K K^T))^{-1},  A = X diag(beta),
//   A' = X diag(beta gamma / g)  (the decays of the write terms).
// Per sub-chunk, with S the state before it:
//   Y = K S,  P = A' V - A (gamma Y)      (P = gamma E, E the delta errors)
//   S' = gamma S + K^T P
//   That' = That - K^T A K That           (the same with the gate left out)
//   o_t = (g_t / gamma) [ q_t^T gamma S + sum_{s <= t} (k_s . q_t) P_s ].
// S decays lazily: the consumers keep XS = S / G (G >= 2^-5, the product of
// the decays since the last eager step), so a lazy step is
//   XS' = XS + K^T (A' V / G' - A K XS),  G' = G gamma,
// with 1/G' folded into A' by the gate wave, and an eager step multiplies XS
// by G gamma first.  The output of token t is then
//   o_t = g_t G [ (Q XS)_t + sum_{s <= t} (k_s . q_t) P_s ]  (lazy) or
//   (g_t / gamma) [ ... ] (eager), its row scale also from the gate wave.
//
// Precision.  Every matrix-core product takes fp16 operands (11 significant
// bits) and accumulates in fp32; S and That stay fp32 in accumulators.  That
// is kept at a power-of-two column scale (re-normalised every fourth chunk;
// a power of two is exact and commutes with the left products).
//
// One workgroup of eight waves per (segment, layer, head).  Waves 0-3
// ("consumers") hold columns [32c, 32c+32) of S and run its chain (and the
// outputs).  Waves 4-7 hold columns [32p, 32p+32) of That and run its chain,
// and besides: wave 4 solves the triangular systems, waves 5 and 6 stage K
// (and Q) and form K K^T, wave 7 stages V and turns the gates into beta,
// beta gamma / g / G', the eager multipliers and the output row scales.
//
// Pipeline (cycle ci, two phases, a workgroup barrier before each): chunk j
// has K staged in phase A of cycle j-1 and K K^T formed in phase B; it is
// solved in cycle j (diagonal blocks in A, off-diagonal blocks and the
// matrices -A, A' in B); its sub-chunk 0 is chained in phase A of cycle j+1
// and sub-chunk 1 in phase B.  V rows of sub-chunk 0 (and Q's) are staged in
// phase B of cycle j, those of sub-chunk 1 in phase A of cycle j+1, so one
// buffer holds each.  Every global load of K and V is issued a cycle before
// its data is staged, those of Q a phase before.
//
// LDS layouts.  K and Q rows are stored with the middle 4-channel pieces of
// every 16-channel group swapped (channels 0-3, 8-11, 4-7, 12-15), so that
// one 16-byte read of a row at [16 ks + 8 g] gives the channels 16 ks + 4 g +
// {0..3, 8..11}: the permuted contraction order in which an accumulator
// feeds a B operand (mfma_util.hpp); the transposed reads (K^T operands)
// address the swapped pieces so that each lane still receives its own
// channel.  -A rows are stored with the same column swap.  V rows and A'
// rows are in natural order.  The row stride of K, Q and V (304 bytes =
// 76 words, 12 mod 64 banks) keeps both the 16-byte row reads of 16 lanes and
// the transposed 8-byte reads of 32 lanes on distinct banks; G rows take 36
// words (16-byte writes of 16 lanes on distinct banks).
#include <type_traits>

#include "mfma_util.hpp"
#include "pic_internal.hpp"

namespace pic {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int DP = 128;          // padded head size
constexpr int C = 64;            // tokens per chunk (two sub-chunks of 32)
constexpr int NT = DP / 32;      // 32-row tiles of a column block
constexpr int THREADS = 512;     // eight waves
constexpr int NKB = 3;           // K buffers (chunks alive at once)
constexpr int RLD = 152;         // row stride (halves) of K, Q, V
constexpr int GLD = 36;          // row stride (floats) of K K^T
constexpr int A_LD = 40;         // row stride (halves) of -A and A'
constexpr int XS_LD = 48;        // row stride (halves) of the solver's scratch
constexpr float kLazyLog2 = -5.f;

constexpr int ROWS_BYTES = C * RLD * 2;
constexpr int G_FLOATS = 2 * 32 * GLD;       // K K^T of both sub-chunks
constexpr int A_HALFS = C * A_LD;            // one 64-row matrix
constexpr int L_K = 0;
constexpr int L_V = L_K + NKB * ROWS_BYTES;
constexpr int L_Q = L_V + ROWS_BYTES;
constexpr int L_G = L_Q + ROWS_BYTES;        // two chunks
constexpr int L_NA = L_G + 2 * G_FLOATS * 4; // -A, two chunks
constexpr int L_AP = L_NA + 2 * A_HALFS * 2; // A', two chunks
constexpr int L_XS = L_AP + 2 * A_HALFS * 2; // solver scratch (4 tiles of 16 rows)
constexpr int L_GB = L_XS + 4 * 16 * XS_LD * 2;
constexpr int L_GBR = L_GB + 2 * C * 4;
constexpr int L_OSC = L_GBR + 2 * C * 4;     // output row scales, four chunks
constexpr int L_EM = L_OSC + 4 * C * 4;      // eager multipliers [4][2], final log2 G
constexpr int LDS_TOTAL = L_EM + 12 * 4;
static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget of a CU");
static_assert(L_V % 16 == 0 && L_Q % 16 == 0 && L_G % 16 == 0 && L_NA % 16 == 0 &&
              L_AP % 16 == 0 && L_XS % 16 == 0 && L_GB % 16 == 0 && L_OSC % 16 == 0 &&
              (RLD * 2) % 16 == 0 && (GLD * 4) % 16 == 0 && (A_LD * 2) % 16 == 0,
              "alignment");

__shared__ __attribute__((aligned(16))) char dfp_smem[LDS_TOTAL];

// a workgroup barrier that no instruction is scheduled across (register-only
// matrix-core products would otherwise move into the next phase)
#define PIC_BARRIER()                    \
  do {                                   \
    __builtin_amdgcn_sched_barrier(0);   \
    __syncthreads();                     \
    __builtin_amdgcn_sched_barrier(0);   \
  } while (0)

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ f32x16 mfma16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16(const f16x4& a, const f16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ unsigned pk_h2(float x0, float x1) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x0, x1}, f16x2));
}
__device__ __forceinline__ f16x4 h4(float x0, float x1, float x2, float x3) {
  const u32x2 w = {pk_h2(x0, x1), pk_h2(x2, x3)};
  return __builtin_bit_cast(f16x4, w);
}
// accumulator registers 8h .. 8h+7 as an fp16 operand
__device__ __forceinline__ f16x8 acc_h8(const f32x16& a, int h) {
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = pk_h2(a[8 * h + 2 * j], a[8 * h + 2 * j + 1]);
  return __builtin_bit_cast(f16x8, w);
}
// two bf16 values in a word -> two fp16 values in a word
__device__ __forceinline__ unsigned bf2h_word(unsigned w) {
  return pk_h2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}
__device__ __forceinline__ f16x8 lds_h8(const _Float16* p) {
  return *reinterpret_cast<const f16x8*>(p);
}
// transposed read: in each group of 16 lanes, lane i receives 16-bit element
// (i & 3) of the 8 bytes addressed by lane 4j + (i >> 2), j = 0..3
__device__ __forceinline__ i16x4 lds_tr4(const _Float16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}
__device__ __forceinline__ f16x8 tr_h8(const _Float16* p0, const _Float16* p1) {
  const i16x4 lo = lds_tr4(p0), hi = lds_tr4(p1);
  const i16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(f16x8, r);
}
template <class T>
__device__ __forceinline__ T gload(const T* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}
template <class T>
__device__ __forceinline__ void gstore(T* p, T v) {
  *(__attribute__((address_space(1))) T*)(p) = v;
}
__device__ __forceinline__ uint4 gload_u4(const void* p) {
  const u32x4 w = *(const __attribute__((address_space(1))) u32x4*)(p);
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t rfl64(int64_t v) {
  const uint32_t lo = uint32_t(rfl(int(uint32_t(v)))), hi = uint32_t(rfl(int(uint64_t(v) >> 32)));
  return int64_t((uint64_t(hi) << 32) | lo);
}
template <class T>
__device__ __forceinline__ T* rflp(T* p) {
  return reinterpret_cast<T*>(rfl64(reinterpret_cast<int64_t>(p)));
}
// maximum over the 64 lanes (uniform result)
__device__ __forceinline__ float wave_max(float x) {
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
// the swap of the middle 4-channel pieces of a 16-channel group, on the
// index of a 4-channel piece (0 1 2 3 -> 0 2 1 3)
__device__ __forceinline__ int swap_piece(int q) { return ((q & 1) << 1) | ((q >> 1) & 1); }

// Staging of rows: 16 items of 16 bytes per lane cover a chunk -- item i is
// row (lane >> 4) + 4 i, channels 8 (lane & 15) .. +7 -- so each load reads
// four whole 256-byte rows.  Rows past the chunk's end read its last row
// (beta is zero on them, so they only meet zero coefficients; their outputs
// are not written); channels past the head size are zeroed.
template <int NI>
__device__ __forceinline__ void load_rows(uint4 (&pr)[NI], const __bf16* base, int HD, int len,
                                          int i0, int lane) {
  if (len == C) {
    const __bf16* p = base + (lane >> 4) * HD;
#pragma unroll
    for (int i = 0; i < NI; ++i) pr[i] = gload_u4(p + 4 * (i0 + i) * HD);
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      pr[i] = gload_u4(base + min((lane >> 4) + 4 * (i0 + i), len - 1) * HD);
  }
}
// natural channel order (V)
template <int NI>
__device__ __forceinline__ void stage_nat(_Float16* dst, const uint4 (&pr)[NI], int d, int i0,
                                          int lane) {
  const int cg = lane & 15;
  const bool okc = 8 * cg < d;
  _Float16* row = dst + (lane >> 4) * RLD + 8 * cg;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint4 x = pr[i];
    const uint4 h = okc ? make_uint4(bf2h_word(x.x), bf2h_word(x.y), bf2h_word(x.z), bf2h_word(x.w))
                        : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(row + 4 * (i0 + i) * RLD) = h;
  }
}
// swapped middle pieces (K, Q): channels 8 cg + 0..3 and + 4..7 of the lane
// go to positions 16 (cg / 2) + 4 swap(2 (cg & 1)) and + 4 swap(2 (cg & 1) + 1)
template <int NI>
__device__ __forceinline__ void stage_perm(_Float16* dst, const uint4 (&pr)[NI], int d, int i0,
                                           int lane) {
  const int cg = lane & 15;
  const bool okc = 8 * cg < d;
  const int p0 = 16 * (cg >> 1) + 4 * swap_piece(2 * (cg & 1));
  const int p1 = 16 * (cg >> 1) + 4 * swap_piece(2 * (cg & 1) + 1);
  _Float16* row = dst + (lane >> 4) * RLD;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint4 x = pr[i];
    const u32x2 a = okc ? (u32x2){bf2h_word(x.x), bf2h_word(x.y)} : (u32x2){0u, 0u};
    const u32x2 b = okc ? (u32x2){bf2h_word(x.z), bf2h_word(x.w)} : (u32x2){0u, 0u};
    _Float16* r = row + 4 * (i0 + i) * RLD;
    *reinterpret_cast<u32x2*>(r + p0) = a;
    *reinterpret_cast<u32x2*>(r + p1) = b;
  }
}

// Back substitution of X_bb (I + L_bb) = I for one row of a 16x16 diagonal
// block, steps i = 15 .. 1: acc[r] -= X[row][i] L[i][r] for r < i, where
// L[i][r] = beta_i G[i][r].  Row i of the block of G is a broadcast read,
// issued PF steps ahead of its use; bt holds beta of the block's tokens.
constexpr int PF = 3;
__device__ __forceinline__ void subst16(float (&acc)[16], const float* grow0, const float (&bt)[16]) {
  float4 buf[PF + 1][4];
#pragma unroll
  for (int p = 0; p < PF; ++p)
#pragma unroll
    for (int r4 = 0; r4 < (15 - p + 3) / 4; ++r4)
      buf[p][r4] = *reinterpret_cast<const float4*>(grow0 + (15 - p) * GLD + 4 * r4);
#pragma unroll
  for (int i = 15; i >= 1; --i) {
    const int slot = (15 - i) % (PF + 1);
    const int ip = i - PF;
    if (ip >= 1) {
      const int ps = (15 - ip) % (PF + 1);
#pragma unroll
      for (int r4 = 0; r4 < (ip + 3) / 4; ++r4)
        buf[ps][r4] = *reinterpret_cast<const float4*>(grow0 + ip * GLD + 4 * r4);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float x = acc[i] * bt[i];
#pragma unroll
    for (int r4 = 0; r4 < (i + 3) / 4; ++r4) {
      const float nv[4] = {buf[slot][r4].x, buf[slot][r4].y, buf[slot][r4].z, buf[slot][r4].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * r4 + e < i) acc[4 * r4 + e] = fmaf(-nv[e], x, acc[4 * r4 + e]);
    }
  }
}

// Per-block values and the fields of the call the roles read.  Each role is
// its own non-inlined function, so that the register allocator sees one role
// at a time.
struct Ctx {
  int64_t t_begin, t_end, N, unit;
  int n, b, h;
};
struct Core {
  int heads, dk, dv;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  float* log_scale;
  float* T_hat;
  float* S0;
  __bf16* O;
  unsigned* nonfinite;
};

#define PIC_DFP_PROLOGUE                                                        \
  _Float16* Kb0 = reinterpret_cast<_Float16*>(dfp_smem + L_K);                  \
  _Float16* Vb = reinterpret_cast<_Float16*>(dfp_smem + L_V);                   \
  _Float16* Qb = reinterpret_cast<_Float16*>(dfp_smem + L_Q);                   \
  float* Gm0 = reinterpret_cast<float*>(dfp_smem + L_G);                        \
  _Float16* NA0 = reinterpret_cast<_Float16*>(dfp_smem + L_NA);                 \
  _Float16* AP0 = reinterpret_cast<_Float16*>(dfp_smem + L_AP);                 \
  _Float16* Xs = reinterpret_cast<_Float16*>(dfp_smem + L_XS);                  \
  float* gb0 = reinterpret_cast<float*>(dfp_smem + L_GB);                       \
  float* gbr0 = reinterpret_cast<float*>(dfp_smem + L_GBR);                     \
  float* osc0 = reinterpret_cast<float*>(dfp_smem + L_OSC);                     \
  float* em0 = reinterpret_cast<float*>(dfp_smem + L_EM);                       \
  const int H = rfl(a.heads), dk = rfl(a.dk), dv = rfl(a.dv);                   \
  const int b = rfl(x.b), h = rfl(x.h), n = rfl(x.n);                           \
  const int64_t t_begin = rfl64(x.t_begin), t_end = rfl64(x.t_end);             \
  const int64_t N = rfl64(x.N), unit = rfl64(x.unit);                           \
  const int lane = threadIdx.x & 63, g = lane >> 5, cl = lane & 31;             \
  const int wid = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));        \
  const int ti = lane & 15, tg = lane >> 4;                                     \
  const int tr_row = ti >> 2;                                                   \
  /* transposed reads of V (natural channels) and of K (swapped pieces) */      \
  const int tr_col = 16 * (tg & 1) + 4 * (ti & 3);                              \
  const int trk_col = 16 * (tg & 1) + 4 * swap_piece(ti & 3);                   \
  auto chunk_len = [&](int j) {                                                 \
    const int64_t c0 = t_begin + int64_t(j) * C;                                \
    return (t_end - c0 < C) ? int(t_end - c0) : C;                              \
  };                                                                            \
  auto row0 = [&](int j) { return (int64_t(b) * N + t_begin + int64_t(j) * C) * H + h; }; \
  (void)Kb0; (void)Vb; (void)Qb; (void)Gm0; (void)NA0; (void)AP0; (void)Xs;    \
  (void)gb0; (void)gbr0; (void)osc0; (void)em0; (void)H; (void)dk; (void)dv;   \
  (void)b; (void)h; (void)N; (void)unit; (void)g; (void)cl; (void)wid;          \
  (void)chunk_len; (void)row0; (void)t_begin; (void)t_end; (void)tr_row;        \
  (void)tr_col; (void)trk_col; (void)ti; (void)tg

// ===========================================================================
// That chain (waves 4-7, columns [32p, 32p+32)): Y = K That, N = -A Y,
// That += K^T N; re-normalised by a power of two every fourth chunk
// ===========================================================================
struct ThatState {
  f32x16 XT[NT];
  int E;
};

__device__ __forceinline__ void that_init(ThatState& st, int p, int dk, int g, int cl) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = t * 32 + acc_row(q, g), col = p * 32 + cl;
      st.XT[t][q] = (row == col && row < dk) ? 1.f : 0.f;
    }
  st.E = 0;
}

__device__ __forceinline__ void that_renorm(ThatState& st) {
  float m = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(st.XT[t][q]));
  m = wave_max(m);
  int e;
  (void)frexpf(m, &e);
  e = (m > 0.f) ? (e < -120 ? -120 : e) : 0;
  const float sc = ldexpf(1.f, -e);
#pragma unroll
  for (int t = 0; t < NT; ++t) st.XT[t] *= sc;
  st.E += e;
}

// ===========================================================================
// roles
// ===========================================================================
template <bool TRACK_T, bool OUTPUT>
__device__ __noinline__ void consumer_role(const Core& a, const Ctx& x);
template <bool TRACK_T, bool OUTPUT>
__device__ __noinline__ void solver_role(const Core& a, const Ctx& x);
template <bool TRACK_T, bool OUTPUT>
__device__ __noinline__ void kwave_role(const Core& a, const Ctx& x);
template <bool TRACK_T, bool OUTPUT>
__device__ __noinline__ void vwave_role(const Core& a, const Ctx& x);

template <bool TRACK_T, bool OUTPUT>
__global__ __launch_bounds__(THREADS) void dense_fp16_kernel(BuildArgs a) {
  const int BH = a.batch * a.heads;
  const int seg = seg_in_order(a, int(build_unit(a, blockIdx.x) / BH));
  const int bh = int(build_unit(a, blockIdx.x) % BH);
  Ctx x;
  x.b = bh / a.heads;
  x.h = bh % a.heads;
  x.t_begin = seg_offset(a, seg);
  x.t_end = seg_offset(a, seg + 1);
  x.N = a.n_tokens;
  x.n = int((x.t_end - x.t_begin + C - 1) / C);
  x.unit = (int64_t(seg) * a.batch + x.b) * a.heads + x.h;
  const Core core{a.heads, a.dk,      a.dv,    a.q,  a.k,  a.v,
                  a.alpha, a.beta,    a.log_scale, a.T_hat, a.S0,
                  static_cast<__bf16*>(a.O), a.nonfinite};
  const int wid = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  if (wid < 4)
    consumer_role<TRACK_T, OUTPUT>(core, x);
  else if (wid == 4)
    solver_role<TRACK_T, OUTPUT>(core, x);
  else if (wid < 7)
    kwave_role<TRACK_T, OUTPUT>(core, x);
  else
    vwave_role<TRACK_T, OUTPUT>(core, x);
}

// ---------------------------------------------------------------------------
// the That step of sub-chunk s of chunk j (waves 4-7)
// ---------------------------------------------------------------------------
#define PIC_DFP_THAT_STEP(st, s, j)                                                  \
  do {                                                                               \
    const _Float16* kb_ = Kb0 + ((j) % NKB) * (C * RLD);                             \
    const _Float16* na_ = NA0 + ((j) & 1) * A_HALFS;                                 \
    const _Float16* krow_ = kb_ + (32 * (s) + cl) * RLD + 8 * g;                     \
    f16x8 kr_[2 * NT];                                                               \
    _Pragma("unroll") for (int ks = 0; ks < 3; ++ks) kr_[ks] = lds_h8(krow_ + 16 * ks); \
    f16x8 nA_[2];                                                                    \
    _Pragma("unroll") for (int hh = 0; hh < 2; ++hh)                                 \
      nA_[hh] = lds_h8(na_ + (32 * (s) + cl) * A_LD + 16 * hh + 8 * g);              \
    f32x16 Y_ = zero16();                                                            \
    _Pragma("unroll") for (int ks = 0; ks < 2 * NT; ++ks) {                          \
      if (ks + 3 < 2 * NT) kr_[ks + 3] = lds_h8(krow_ + 16 * (ks + 3));              \
      Y_ = mfma16(kr_[ks], acc_h8((st).XT[ks >> 1], ks & 1), Y_);                    \
      __builtin_amdgcn_sched_barrier(0);                                             \
    }                                                                                \
    const _Float16* kbase_ = kb_ + (32 * (s) + 4 * g + tr_row) * RLD + trk_col;      \
    f16x8 kf_[2][NT];                                                                \
    _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                 \
      const _Float16* p0_ = kbase_ + 32 * t;                                         \
      kf_[0][t] = tr_h8(p0_, p0_ + 8 * RLD);                                         \
    }                                                                                \
    f32x16 Nn_ = zero16();                                                           \
    _Pragma("unroll") for (int hh = 0; hh < 2; ++hh)                                 \
      Nn_ = mfma16(nA_[hh], acc_h8(Y_, hh), Nn_);                                    \
    __builtin_amdgcn_sched_barrier(0);                                               \
    _Pragma("unroll") for (int hh = 0; hh < 2; ++hh) {                               \
      const f16x8 nb_ = acc_h8(Nn_, hh);                                             \
      if (hh == 0) {                                                                 \
        _Pragma("unroll") for (int t = 0; t < NT; ++t) {                             \
          const _Float16* p0_ = kbase_ + 16 * RLD + 32 * t;                          \
          kf_[1][t] = tr_h8(p0_, p0_ + 8 * RLD);                                     \
        }                                                                            \
      }                                                                              \
      _Pragma("unroll") for (int t = 0; t < NT; ++t)                                 \
        (st).XT[t] = mfma16(kf_[hh][t], nb_, (st).XT[t]);                            \
      __builtin_amdgcn_sched_barrier(0);                                             \
    }                                                                                \
  } while (0)

#define PIC_DFP_THAT_STORE(st, p)                                                    \
  do {                                                                               \
    const int ncol_ = (p) * 32 + cl;                                                 \
    bool bad_ = false;                                                               \
    if (ncol_ < dk) {                                                                \
      float* out_ = rflp(a.T_hat) + unit * int64_t(dk) * dk;                         \
      _Pragma("unroll") for (int t = 0; t < NT; ++t)                                 \
      _Pragma("unroll") for (int q = 0; q < 16; ++q) {                               \
        const int row_ = t * 32 + acc_row(q, g);                                     \
        const float v_ = ldexpf((st).XT[t][q], (st).E);                              \
        bad_ |= not_finite(v_);                                                      \
        if (row_ < dk) gstore(out_ + int64_t(row_) * dk + ncol_, v_);                \
      }                                                                              \
    }                                                                                \
    report_nonfinite(a.nonfinite, bad_);                                             \
  } while (0)

// ===========================================================================
// consumers: columns [32c, 32c+32) of S (and of the outputs)
// ===========================================================================
template <bool TRACK_T, bool OUTPUT>
__device__ __noinline__ void consumer_role(const Core& a, const Ctx& x) {
  PIC_DFP_PROLOGUE;
  const int c = wid;
  bool obad = false;  // a stored output or state value is not finite
  f32x16 XS[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) XS[t] = zero16();

  // sub-chunk s of chunk j
  auto chain = [&](int s, int j) {
    const _Float16* kb = Kb0 + (j % NKB) * (C * RLD);
    const _Float16* na = NA0 + (j & 1) * A_HALFS;
    const _Float16* ap = AP0 + (j & 1) * A_HALFS;
    // K-row fragments (A operand of K XS and of K Q^T) and Q-row fragments
    // (A operand of Q XS, B operand of K Q^T), streamed three steps ahead
    const _Float16* krow = kb + (32 * s + cl) * RLD + 8 * g;
    const _Float16* qrow = Qb + (32 * s + cl) * RLD + 8 * g;
    f16x8 kr[2 * NT], qr[2 * NT];
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      kr[ks] = lds_h8(krow + 16 * ks);
      if constexpr (OUTPUT) qr[ks] = lds_h8(qrow + 16 * ks);
    }
    const int emi = rfl(__float_as_int(em0[(j & 3) * 2 + s]));
    if (emi >= 0) {  // eager step (uniform)
      const float em = __int_as_float(emi);
#pragma unroll
      for (int t = 0; t < NT; ++t) XS[t] *= em;
    }
    // Y = K XS; with the outputs also Q XS (the inter-chunk part) and
    // KQ[s'][t] = k_s' . q_t
    f32x16 Y = zero16(), O = zero16(), KQ = zero16();
#pragma unroll
    for (int ks = 0; ks < 2 * NT; ++ks) {
      if (ks + 3 < 2 * NT) {
        kr[ks + 3] = lds_h8(krow + 16 * (ks + 3));
        if constexpr (OUTPUT) qr[ks + 3] = lds_h8(qrow + 16 * (ks + 3));
      }
      const f16x8 sb = acc_h8(XS[ks >> 1], ks & 1);
      Y = mfma16(kr[ks], sb, Y);
      if constexpr (OUTPUT) {
        O = mfma16(qr[ks], sb, O);
        KQ = mfma16(kr[ks], qr[ks], KQ);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // P = A' V (the W seed, with the lazy 1/G') - A Y
    f32x16 P = zero16();
    {
      // V^T fragment: lane (g, m) needs V[token 16 kk + 8 g + 0..7][32 c + m]
      const _Float16* vbase = Vb + (8 * g + tr_row) * RLD + 32 * c + tr_col;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const f16x8 ph = lds_h8(ap + (32 * s + cl) * A_LD + 16 * kk + 8 * g);
        const _Float16* p0 = vbase + (32 * s + 16 * kk) * RLD;
        P = mfma16(ph, tr_h8(p0, p0 + 4 * RLD), P);
      }
    }
    f16x8 nA[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) nA[hh] = lds_h8(na + (32 * s + cl) * A_LD + 16 * hh + 8 * g);
    const _Float16* kbase = kb + (32 * s + 4 * g + tr_row) * RLD + trk_col;
    f16x8 kf[2][NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const _Float16* p0 = kbase + 32 * t;
      kf[0][t] = tr_h8(p0, p0 + 8 * RLD);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) P = mfma16(nA[hh], acc_h8(Y, hh), P);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (OUTPUT) {
      // causal mask of KQ: keep s' <= t (lane column t = cl, row s' = acc_row)
#pragma unroll
      for (int q = 0; q < 16; ++q) KQ[q] = (acc_row(q, g) <= cl) ? KQ[q] : 0.f;
    }
    // XS += K^T P, O += KQ^T P (the K^T fragments of the second half are
    // read while the first half's products run)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const f16x8 mb = acc_h8(P, hh);
      if (hh == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const _Float16* p0 = kbase + 16 * RLD + 32 * t;
          kf[1][t] = tr_h8(p0, p0 + 8 * RLD);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) XS[t] = mfma16(kf[hh][t], mb, XS[t]);
      if constexpr (OUTPUT) O = mfma16(acc_h8(KQ, hh), mb, O);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (OUTPUT) {
      // row scales and the stores (bf16, rows of this sub-chunk inside the segment)
      const float* osc = osc0 + (j & 3) * C + 32 * s;
      const int len = chunk_len(j) - 32 * s;
      const int ncol = 32 * c + cl;
      __bf16* ob = rflp(a.O) + (row0(j) + int64_t(32 * s) * H) * dv + ncol;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 sc = *reinterpret_cast<const float4*>(osc + 8 * i + 4 * g);
        const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * i + 4 * g + e;
          if (r < len && ncol < dv) {
            const float v = O[4 * i + e] * scv[e];
            obad |= not_finite(v);
            gstore(ob + int64_t(r) * H * dv, static_cast<__bf16>(v));
          }
        }
      }
    }
  };

  PIC_BARRIER();  // cycle -1, phase A
  PIC_BARRIER();  //           phase B
  PIC_BARRIER();  // cycle 0,  phase A
  PIC_BARRIER();  //           phase B
#pragma unroll 1
  for (int ci = 1; ci <= n; ++ci) {
    PIC_BARRIER();  // phase A
    chain(0, ci - 1);
    PIC_BARRIER();  // phase B
    chain(1, ci - 1);
  }
  // S(C|0) = 2^lg XS (lg the final log2 G of the lazy decay)
  const int ncol = c * 32 + cl;
  if (ncol < dv) {
    float* out = rflp(a.S0) + unit * int64_t(dk) * dv;
    const float gs = n >= 1 ? exp2f(em0[8]) : 1.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = t * 32 + acc_row(q, g);
        const float v = float(XS[t][q]) * gs;
        obad |= not_finite(v);
        if (row < dk) gstore(out + int64_t(row) * dv + ncol, v);
      }
  }
  report_nonfinite(a.nonfinite, obad);
}

// ===========================================================================
// solver wave (also That columns [0, 32)): X_s = (I + L_s)^{-1} of both
// sub-chunks.  Phase A: the four 16x16 diagonal blocks by back substitution,
// lane 32 s + 16 b + j owning row j of block b of sub-chunk s; the rows go
// to the scratch (fp16).  Phase B: the off-diagonal block X_10 = -X_11 L_10
// X_00 of each sub-chunk with two 16x16x16 matrix-core products, then
// -A = -X diag(beta) (columns swapped as the K rows) and A' = X diag(beta r).
// ===========================================================================
template <bool TRACK_T, bool OUTPUT>
__device__ __noinline__ void solver_role(const Core& a, const Ctx& x) {
  PIC_DFP_PROLOGUE;
  const int s = lane >> 5, blk = (lane >> 4) & 1, jr = lane & 15;
  float acc[16], bt[16];
  ThatState st;
  if constexpr (TRACK_T) that_init(st, 0, dk, g, cl);
  // position of column col (0..31) of -A in its row: pieces 1 and 2 of each
  // 16-column group swapped
  auto na_pos = [](int col) { return 16 * (col >> 4) + 4 * swap_piece((col >> 2) & 3) + (col & 3); };

  auto phase_a = [&](int ci) {
    if (ci >= 0 && ci < n) {
      const float* gm = Gm0 + (ci & 1) * G_FLOATS;
      const float* gbp = gb0 + (ci & 1) * C;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 b4 = *reinterpret_cast<const float4*>(gbp + 32 * s + 16 * blk + 4 * q);
        bt[4 * q] = b4.x; bt[4 * q + 1] = b4.y; bt[4 * q + 2] = b4.z; bt[4 * q + 3] = b4.w;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = (r == jr) ? 1.f : 0.f;
      subst16(acc, gm + s * 32 * GLD + (16 * blk) * GLD + 16 * blk, bt);
      _Float16* xr = Xs + ((2 * s + blk) * 16 + jr) * XS_LD;
      *reinterpret_cast<uint4*>(xr) = make_uint4(pk_h2(acc[0], acc[1]), pk_h2(acc[2], acc[3]),
                                                 pk_h2(acc[4], acc[5]), pk_h2(acc[6], acc[7]));
      *reinterpret_cast<uint4*>(xr + 8) = make_uint4(pk_h2(acc[8], acc[9]), pk_h2(acc[10], acc[11]),
                                                     pk_h2(acc[12], acc[13]), pk_h2(acc[14], acc[15]));
    }
  };
  auto phase_b = [&](int ci) {
    if (ci >= 0 && ci < n) {
      const float* gm = Gm0 + (ci & 1) * G_FLOATS;
      const float* gbp = gb0 + (ci & 1) * C;
      const float* grp = gbr0 + (ci & 1) * C;
      _Float16* na = NA0 + (ci & 1) * A_HALFS;
      _Float16* ap = AP0 + (ci & 1) * A_HALFS;
      // off-diagonal blocks; 16x16x16 layouts: lane l holds A[l%16][4(l/16)+e],
      // B[4(l/16)+e][l%16], D[4(l/16)+e][l%16], e = 0..3
      const int m = lane & 15, kq = lane >> 4;
      f32x4 X10[2];
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const float4 g4 = *reinterpret_cast<const float4*>(gm + ss * 32 * GLD + (16 + m) * GLD + 4 * kq);
        const float bm = gbp[32 * ss + 16 + m];
        const f16x4 l10 = h4(bm * g4.x, bm * g4.y, bm * g4.z, bm * g4.w);
        const _Float16* t00 = Xs + (2 * ss) * 16 * XS_LD;
        const _Float16* t11 = Xs + (2 * ss + 1) * 16 * XS_LD;
        const f16x4 x00 = __builtin_bit_cast(f16x4, lds_tr4(t00 + (4 * kq + (m >> 2)) * XS_LD + 4 * (m & 3)));
        const f16x4 x11 = *reinterpret_cast<const f16x4*>(t11 + m * XS_LD + 4 * kq);
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        y = mfma16x16(l10, x00, y);
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        X10[ss] = mfma16x16(x11, h4(y[0], y[1], y[2], y[3]), z);
      }
      // this lane's row of its diagonal block: -A and A' entries; the other
      // half of the row is zero (block 0) or the off-diagonal block (block 1)
      const int row = 32 * s + 16 * blk + jr;
      float rk[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 r4 = *reinterpret_cast<const float4*>(grp + 32 * s + 16 * blk + 4 * q);
        rk[4 * q] = r4.x; rk[4 * q + 1] = r4.y; rk[4 * q + 2] = r4.z; rk[4 * q + 3] = r4.w;
      }
      // -A: pieces of 4 columns, stored with pieces 1 and 2 swapped
      _Float16* narow = na + row * A_LD + 16 * blk;
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        const int k = 4 * pc;
        *reinterpret_cast<u32x2*>(narow + 4 * swap_piece(pc)) =
            (u32x2){pk_h2(-acc[k] * bt[k], -acc[k + 1] * bt[k + 1]),
                    pk_h2(-acc[k + 2] * bt[k + 2], -acc[k + 3] * bt[k + 3])};
      }
      _Float16* aprow = ap + row * A_LD;
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int k = 8 * h8;
        *reinterpret_cast<uint4*>(aprow + 16 * blk + k) =
            make_uint4(pk_h2(acc[k] * rk[k], acc[k + 1] * rk[k + 1]),
                       pk_h2(acc[k + 2] * rk[k + 2], acc[k + 3] * rk[k + 3]),
                       pk_h2(acc[k + 4] * rk[k + 4], acc[k + 5] * rk[k + 5]),
                       pk_h2(acc[k + 6] * rk[k + 6], acc[k + 7] * rk[k + 7]));
      }
      if (blk == 0) {
        const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(na + row * A_LD + 16) = z4;
        *reinterpret_cast<uint4*>(na + row * A_LD + 24) = z4;
        *reinterpret_cast<uint4*>(aprow + 16) = z4;
        *reinterpret_cast<uint4*>(aprow + 24) = z4;
      }
      // off-diagonal blocks: lane l holds (X11 L10 X00)[4 kq + e][m] = -X10
      // of each sub-chunk
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const float bn = gbp[32 * ss + m], rn = grp[32 * ss + m];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 32 * ss + 16 + 4 * kq + e;
          na[r * A_LD + na_pos(m)] = _Float16(X10[ss][e] * bn);
          ap[r * A_LD + m] = _Float16(-X10[ss][e] * rn);
        }
      }
    }
  };

  for (int ci = -1; ci <= 0; ++ci) {
    PIC_BARRIER();
    phase_a(ci);
    PIC_BARRIER();
    phase_b(ci);
  }
#pragma unroll 1
  for (int ci = 1; ci <= n; ++ci) {
    PIC_BARRIER();
    phase_a(ci);
    if constexpr (TRACK_T) PIC_DFP_THAT_STEP(st, 0, ci - 1);
    PIC_BARRIER();
    phase_b(ci);
    if constexpr (TRACK_T) {
      PIC_DFP_THAT_STEP(st, 1, ci - 1);
      if ((ci & 3) == 0) that_renorm(st);
    }
  }
  if constexpr (TRACK_T) PIC_DFP_THAT_STORE(st, 0);
}

// ===========================================================================
// K waves (also That columns [32, 64) and [64, 96)): K rows of chunk ci+1
// (half each) and, for the outputs, Q rows; K K^T of sub-chunk pw
// ===========================================================================
template <bool TRACK_T, bool OUTPUT>
__device__ __noinline__ void kwave_role(const Core& a, const Ctx& x) {
  PIC_DFP_PROLOGUE;
  const int pw = wid - 5;  // 0 or 1
  const int HDk = H * dk;
  const int kch = min(8 * (lane & 15), dk - 8);
  const __bf16* kp = rflp(static_cast<const __bf16*>(a.k));
  const __bf16* qp = rflp(static_cast<const __bf16*>(a.q));
  ThatState st;
  if constexpr (TRACK_T) that_init(st, 1 + pw, dk, g, cl);
  // K rows: items 8 pw .. 8 pw + 7 of a chunk, loaded a cycle ahead; Q
  // rows: items 4 pw .. + 3 of each sub-chunk's eight (sub-chunk 0: items
  // 0-7, sub-chunk 1: 8-15), each half loaded one phase ahead, so that the
  // two halves never hold registers at the same time
  uint4 prk[8], prq[4];
  if (n > 0) load_rows(prk, kp + row0(0) * dk + kch, HDk, chunk_len(0), 8 * pw, lane);
  auto phase_a = [&](int ci) {
    if (ci + 1 < n) stage_perm(Kb0 + ((ci + 1) % NKB) * (C * RLD), prk, dk, 8 * pw, lane);
    if (ci + 2 < n) load_rows(prk, kp + row0(ci + 2) * dk + kch, HDk, chunk_len(ci + 2), 8 * pw, lane);
    if constexpr (OUTPUT) {
      // Q rows of sub-chunk 1 of chunk ci-1 (loaded in the last phase B),
      // then those of sub-chunk 0 of chunk ci (staged in the next phase)
      if (ci - 1 >= 0 && ci - 1 < n) stage_perm(Qb, prq, dk, 8 + 4 * pw, lane);
      if (ci >= 0 && ci < n) load_rows(prq, qp + row0(ci) * dk + kch, HDk, chunk_len(ci), 4 * pw, lane);
    }
  };
  auto phase_b = [&](int ci) {
    if (ci + 1 < n) {
      // K K^T of sub-chunk pw of chunk ci+1 (fp32; symmetric: the lane's
      // accumulator column is written as a row)
      const _Float16* kb = Kb0 + ((ci + 1) % NKB) * (C * RLD);
      f32x16 g0 = zero16(), g1 = zero16();
#pragma unroll
      for (int ks = 0; ks < 2 * NT; ++ks) {
        const f16x8 ak = lds_h8(kb + (32 * pw + cl) * RLD + 16 * ks + 8 * g);
        if (ks & 1)
          g1 = mfma16(ak, ak, g1);
        else
          g0 = mfma16(ak, ak, g0);
      }
      float* row = Gm0 + ((ci + 1) & 1) * G_FLOATS + pw * 32 * GLD + cl * GLD + 4 * g;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
        *reinterpret_cast<float4*>(row + 8 * k4) =
            make_float4(g0[4 * k4] + g1[4 * k4], g0[4 * k4 + 1] + g1[4 * k4 + 1],
                        g0[4 * k4 + 2] + g1[4 * k4 + 2], g0[4 * k4 + 3] + g1[4 * k4 + 3]);
    }
    if constexpr (OUTPUT) {
      // Q rows of sub-chunk 0 of chunk ci, then those of its sub-chunk 1
      if (ci >= 0 && ci < n) {
        stage_perm(Qb, prq, dk, 4 * pw, lane);
        load_rows(prq, qp + row0(ci) * dk + kch, HDk, chunk_len(ci), 8 + 4 * pw, lane);
      }
    }
  };

  for (int ci = -1; ci <= 0; ++ci) {
    PIC_BARRIER();
    phase_a(ci);
    PIC_BARRIER();
    phase_b(ci);
  }
#pragma unroll 1
  for (int ci = 1; ci <= n; ++ci) {
    PIC_BARRIER();
    phase_a(ci);
    if constexpr (TRACK_T) PIC_DFP_THAT_STEP(st, 0, ci - 1);
    PIC_BARRIER();
    phase_b(ci);
    if constexpr (TRACK_T) {
      PIC_DFP_THAT_STEP(st, 1, ci - 1);
      if ((ci & 3) == 0) that_renorm(st);
    }
  }
  if constexpr (TRACK_T) PIC_DFP_THAT_STORE(st, 1 + pw);
}

// ===========================================================================
// V wave (also That columns [96, 128)): V rows by sub-chunk, the gates
// ===========================================================================
template <bool TRACK_T, bool OUTPUT>
__device__ __noinline__ void vwave_role(const Core& a, const Ctx& x) {
  PIC_DFP_PROLOGUE;
  const float* alpha = rflp(a.alpha);
  const float* beta = rflp(a.beta);
  const float* bsrc = beta ? beta : alpha;
  const __bf16* vp = rflp(static_cast<const __bf16*>(a.v));
  const int HDv = H * dv;
  const int vch = min(8 * (lane & 15), dv - 8);
  ThatState st;
  if constexpr (TRACK_T) that_init(st, 3, dk, g, cl);
  uint4 prv0[8], prv1[8];  // V rows of sub-chunk 0 (items 0-7) and 1 (8-15)
  float pa[2] = {1.f, 1.f}, pb[2] = {0.f, 0.f};
  float lam = 0.f, lg = 0.f;  // lg: log2 G of the lazy decay (uniform)
  auto load_gates = [&](int j, float& ra, float& rb) {
    const int64_t gi = row0(j) + int64_t(min(lane, chunk_len(j) - 1)) * H;
    ra = gload(alpha + gi);
    rb = gload(bsrc + gi);
  };
  if (n > 0) load_rows(prv0, vp + row0(0) * dv + vch, HDv, chunk_len(0), 0, lane);
  if (n > 0) load_gates(0, pa[0], pb[0]);
  if (n > 1) load_gates(1, pa[1], pb[1]);

  auto phase_a = [&](int ci) {
    if (ci - 1 >= 0 && ci - 1 < n) stage_nat(Vb, prv1, dv, 8, lane);
    if (ci >= 0 && ci < n) load_rows(prv1, vp + row0(ci) * dv + vch, HDv, chunk_len(ci), 8, lane);
  };
  // gates of chunk jn = ci+1 (slot P of the loaded gates)
  auto gates = [&](int jn, float& ra, float& rb) {
    const int len = chunk_len(jn);
    const float x2 = half_wave_scan(lane < len ? log2f(ra) : 0.f);
    const int xi = __builtin_bit_cast(int, x2);
    const float e0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 31));
    const float e1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 63));
    const float bend = g ? e1 : e0;
    const float bt = lane < len ? (beta ? rb : 1.f) : 0.f;  // masked beta
    // lazy decay of S: a lazy step keeps S / G with G <- G gamma (its W seed
    // takes 1/G, folded into beta * r), an eager step (em >= 0) multiplies S
    // by G gamma and restarts G at 1.  Output row scale of token t: g_t G
    // before the step (lazy) or g_t / gamma (eager)
    float em[2], sl[2], oo[2];
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const float e = ss ? e1 : e0;
      if (lg + e >= kLazyLog2) {
        oo[ss] = lg;
        lg += e;
        em[ss] = -1.f;
        sl[ss] = -lg;
      } else {
        oo[ss] = -e;
        em[ss] = exp2f(lg + e);
        lg = 0.f;
        sl[ss] = 0.f;
      }
    }
    gb0[(jn & 1) * C + lane] = bt;
    gbr0[(jn & 1) * C + lane] = bt * exp2f(bend - x2 + (g ? sl[1] : sl[0]));
    if constexpr (OUTPUT) osc0[(jn & 3) * C + lane] = exp2f(x2 + (g ? oo[1] : oo[0]));
    if (lane == 0) {
      em0[(jn & 3) * 2] = em[0];
      em0[(jn & 3) * 2 + 1] = em[1];
      if (jn == n - 1) em0[8] = lg;  // S(C|0) = 2^lg x the consumers' state
    }
    lam += e0 + e1;
    if (jn + 2 < n) load_gates(jn + 2, ra, rb);
  };
  auto phase_b = [&](int ci) {
    if (ci + 1 < n) {
      if ((ci + 1) & 1)
        gates(ci + 1, pa[1], pb[1]);
      else
        gates(ci + 1, pa[0], pb[0]);
    }
    if (ci >= 0 && ci < n) stage_nat(Vb, prv0, dv, 0, lane);
    if (ci + 1 < n) load_rows(prv0, vp + row0(ci + 1) * dv + vch, HDv, chunk_len(ci + 1), 0, lane);
  };

  for (int ci = -1; ci <= 0; ++ci) {
    PIC_BARRIER();
    phase_a(ci);
    PIC_BARRIER();
    phase_b(ci);
  }
#pragma unroll 1
  for (int ci = 1; ci <= n; ++ci) {
    PIC_BARRIER();
    phase_a(ci);
    if constexpr (TRACK_T) PIC_DFP_THAT_STEP(st, 0, ci - 1);
    PIC_BARRIER();
    phase_b(ci);
    if constexpr (TRACK_T) {
      PIC_DFP_THAT_STEP(st, 1, ci - 1);
      if ((ci & 3) == 0) that_renorm(st);
    }
  }
  if (lane == 0) gstore(rflp(a.log_scale) + unit, lam * kLn2);
  if constexpr (TRACK_T) PIC_DFP_THAT_STORE(st, 3);
}

template <bool TRACK_T, bool OUTPUT>
hipError_t launch(const BuildArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_seg) * a.batch * a.heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((dense_fp16_kernel<TRACK_T, OUTPUT>), dim3(unsigned(blocks)), dim3(THREADS),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_prefill(const BuildArgs& a, bool track_T, hipStream_t s) {
  return track_T ? launch<true, true>(a, s) : launch<false, true>(a, s);
}

}  // namespace pic
