// k_build_dense_h16.hip -- build of the dense gated-delta pair
// (lambda_C, That_C, S(C|0)) for bf16 k/v at fp16 operand precision
// (PIC_PREC_FP16): every matrix-core product takes single fp16 operands and
// accumulates in fp32; the running That and S stay fp32 in accumulators.
// Same chunked arithmetic as k_build_dense.hip (derivation there), on
// sub-chunks of 32 tokens:
//   X_s = (I + diag(beta) strictly-lower(K_s K_s^T))^{-1}
//   A_s = X_s diag(beta),  A'_s = X_s diag(beta r),  U_s = A_s K_s,  W_s = A'_s V_s
//   That <- That - K_s^T (U_s That),   S <- gamma_s S + K_s^T (W_s - U_s (gamma_s S)).
// [xix.ai HYPIC article (French), paragraph on linear layers: T_C as the
//  product of the segment's token transitions and S(C|0) from a zero start;
//  dense delta-rule transitions are the heaviest family.]
//
// Precision.  fp16 keeps 11 significant bits (bf16: 8), so one fp16 product
// per operand pair replaces the three split-bf16 products of the fp32-accurate
// kernels.  The ungated product That shrinks steadily along a segment (its
// norm is ~1e-4 after 4096 tokens at the usual gates), far below fp16's
// normal range, so each consumer wave keeps its columns of That scaled by a
// power of two (a column scaling commutes with left multiplication, and a
// power of two is exact) and re-normalises them every fourth chunk; the
// exponent is applied when That is written.  S is decayed lazily: the
// consumers keep S / G with G >= 2^-5 the product of the chunk decays since
// the last eager multiply, so most sub-chunks need no pass over S (the 1/G
// of the W seed is folded into beta * r by the gate wave).  S / G, U, W and
// the keys stay within fp16's range for unit-norm keys and |S| below ~2e3.
//
// One workgroup per (segment, layer, head): four consumer waves, each holding
// columns [32c, 32c+32) of both That and S in MFMA accumulators for the whole
// segment, and four producer waves.  Producer wave 0 ("solver") computes the
// two 32x32 triangular inverses of a chunk: the 16x16 diagonal blocks by back
// substitution, one row per lane, reading rows of L as broadcast LDS loads a
// few steps ahead, then the off-diagonal blocks X_10 = -X_11 L_10 X_00 with
// 16x16x16 matrix-core products: no workgroup barrier inside the solve; it
// also forms two of the eight U^T = K^T A^T tiles.  Two K waves stage the K
// rows (half each), form the other six U^T tiles and G = K K^T (one
// sub-chunk each); the last wave stages V and turns the gates into the
// masked beta, beta * r and the sub-chunk decays.
//
// LDS holds K and V row-major in fp16.  Every transposed operand fragment
// (K^T for U^T and for K^T N, V^T for W) is read with ds_read_b64_tr_b16: in
// each group of 16 lanes, lane i receives, for j = 0..3, 16-bit element
// (i & 3) of the 8 bytes addressed by lane 4j + (i >> 2).  So when lane
// 4j + q of the group addresses row r_j, columns c0 + 4q .. c0 + 4q + 3, lane
// i receives rows r_0..r_3 of column c0 + i: a column of the tile, i.e. a
// row of its transpose.  The row stride (288 bytes) puts the 16 addresses of
// a group on distinct banks.  The LDS serves the two groups of a half wave
// together, and they read the two 16-column halves of one 32-column tile from
// the same rows: so the columns of a row are stored permuted, the 16-column
// piece p (columns 16p .. 16p+15) at piece slot (p >> 1) + 4 (p & 1), which
// puts the two halves of tile t 128 bytes apart (slots t and t + 4) and their
// banks apart.  G = K K^T sums over all columns and reads them in stored order.
//
// Pipeline: cycle ci has two phases separated by workgroup barriers.
//   phase A: consumers chain sub-chunk 1 of chunk ci-2
//            K waves:  K rows of chunk ci+1 to LDS; U^T tiles 0-5 of chunk
//                      ci-1 -> -U fragments
//            V wave:   V rows of chunk ci-1
//            solver:   diagonal blocks of chunk ci; U^T tiles 6, 7 of ci-1
//   phase B: consumers: W seed and chain of sub-chunk 0 of chunk ci-1, then
//                       the W seed of its sub-chunk 1 (kept for phase A)
//            K waves:  G of chunk ci+1 (wave s: sub-chunk s)
//            V wave:   the gates of chunk ci+1
//            solver:   off-diagonal blocks of chunk ci -> A, A'
// so a chunk is staged in cycle j-1, solved in cycle j, and chained in cycles
// j+1 and j+2.  K is kept for four chunks; -U fragments, A/A', G and the
// masked gates for two; V for one.  Every global load (K and V rows, gates)
// is issued two cycles before its data is staged, into one of two register
// sets.  The solver applies beta to the rows of G
// (L = diag(beta) strictly-lower(G)); G = K K^T is symmetric, so each lane
// writes its accumulator column as a row with four 16-byte stores.
#include <type_traits>

#include "mfma_util.hpp"
#include "pic_internal.hpp"

namespace pic {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Barriers.  Nothing is scheduled across a workgroup barrier: register-only
// work (matrix-core products) is otherwise free to move past it, and products
// of one phase that slip into the next delay that phase's own work.
//
// Optional phase timing (built only with -DPIC_PHASE_TIMING, into a separate
// diagnostic library): every wave adds up, per phase of the pipeline cycle,
// its busy clocks (from the barrier that opens the phase to its arrival at the
// one that closes it) and the phase's length (release to release), in a few
// words of LDS per wave, so that the timers take no registers from the roles
// (kept in registers, they spilled to scratch, whose waits distorted the
// phases).  Clocks are the counter read by s_memtime.
#ifdef PIC_PHASE_TIMING
}  // namespace
__device__ unsigned long long* pic_phase_out;  // [block][wave][8], blocks < pic_phase_blocks
__device__ int pic_phase_blocks;
namespace {
// per wave: busy A, busy B, length A, length B, last release, cycles, start
__shared__ unsigned h16_tm[8][8];
#define PIC_PHASE_DECL                                                      \
  do {                                                                      \
    if ((threadIdx.x & 63) == 0) {                                          \
      const unsigned t_ = unsigned(__builtin_amdgcn_s_memtime());          \
      unsigned* m_ = h16_tm[threadIdx.x >> 6];                              \
      m_[0] = m_[1] = m_[2] = m_[3] = m_[5] = 0u;                           \
      m_[4] = m_[6] = t_;                                                   \
    }                                                                       \
  } while (0)
// barrier that opens phase `ph` (and closes the other one)
#define PIC_BAR(ph)                                                         \
  do {                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                      \
    const unsigned a_ = unsigned(__builtin_amdgcn_s_memtime());            \
    __syncthreads();                                                        \
    const unsigned r_ = unsigned(__builtin_amdgcn_s_memtime());            \
    if ((threadIdx.x & 63) == 0) {                                          \
      unsigned* m_ = h16_tm[threadIdx.x >> 6];                              \
      const unsigned o_ = m_[4];                                            \
      m_[1 - (ph)] += a_ - o_;                                              \
      m_[3 - (ph)] += r_ - o_;                                              \
      m_[4] = r_;                                                           \
      m_[5] += (ph);                                                        \
    }                                                                       \
    __builtin_amdgcn_sched_barrier(0);                                      \
  } while (0)
#define PIC_PHASE_SAVE                                                                   \
  do {                                                                                   \
    if (int(blockIdx.x) < pic_phase_blocks && (threadIdx.x & 63) == 0) {                \
      const unsigned* m_ = h16_tm[threadIdx.x >> 6];                                     \
      unsigned long long* o =                                                            \
          pic_phase_out + (blockIdx.x * (THREADS / 64) + (threadIdx.x >> 6)) * 8;        \
      o[0] = m_[2];                                                                      \
      o[1] = m_[2] - m_[0];                                                              \
      o[2] = m_[3];                                                                      \
      o[3] = m_[3] - m_[1];                                                              \
      o[4] = unsigned(__builtin_amdgcn_s_memtime()) - m_[6];                            \
      o[5] = m_[5];                                                                      \
    }                                                                                    \
  } while (0)
#else
#define PIC_PHASE_DECL
#define PIC_BAR(ph)                        \
  do {                                     \
    __builtin_amdgcn_sched_barrier(0);     \
    __syncthreads();                       \
    __builtin_amdgcn_sched_barrier(0);     \
  } while (0)
#define PIC_PHASE_SAVE
#endif

constexpr int DP = 128;        // padded head size
constexpr int C = 64;          // tokens staged per chunk
constexpr int NT = DP / 32;    // consumer waves = 32-row tiles
constexpr int NHW = 3;         // producer waves besides the solver (two K, one V)
constexpr int THREADS = (NT + 1 + NHW) * 64;
constexpr int NKB = 4;         // K buffers (chunks alive at once)

constexpr int RLD = DP + 16;   // row stride (halves) of K and V
constexpr float kLazyLog2 = -5.f;  // lazy decay of S: G >= 2^-5
constexpr int A_LD = 40;       // A, A' rows (fp16, 32 tokens + pad)

constexpr int ROWS_BYTES = C * RLD * 2;
constexpr int L_K = 0;
constexpr int L_V = L_K + NKB * ROWS_BYTES;
constexpr int L_NM = L_V + ROWS_BYTES;
constexpr int NM_FLOATS = 2 * 32 * 32;          // L of both sub-chunks
constexpr int L_AB = L_NM + 2 * NM_FLOATS * 4;
constexpr int AB_HALFS = 2 * 64 * A_LD;         // A rows then A' rows
constexpr int L_UF = L_AB + 2 * AB_HALFS * 2;
constexpr int UF_BYTES = 2 * NT * 2 * 64 * 16;  // [s][t][h][lane] x 16 B
constexpr int L_GB = L_UF + 2 * UF_BYTES;       // beta (masked), two chunks
constexpr int L_GBR = L_GB + 2 * C * 4;         // beta * r, two chunks
constexpr int L_GG = L_GBR + 2 * C * 4;         // eager multiplier ring [4][2], final log2 scale
constexpr int LDS_TOTAL = L_GG + 12 * 4;
static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget of a CU");
static_assert(L_V % 16 == 0 && L_NM % 16 == 0 && L_AB % 16 == 0 && L_UF % 16 == 0 &&
              L_GB % 16 == 0 && L_GBR % 16 == 0 && (RLD * 2) % 16 == 0, "alignment");

__device__ __forceinline__ f32x16 mfma16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ unsigned pk_h2(float x0, float x1) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x0, x1}, f16x2));
}

// accumulator registers 8h .. 8h+7 (times SGN) as an fp16 operand
template <int SGN = 1>
__device__ __forceinline__ f16x8 acc_h8(const f32x16& a, int h) {
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = pk_h2(SGN * a[8 * h + 2 * j], SGN * a[8 * h + 2 * j + 1]);
  return __builtin_bit_cast(f16x8, w);
}

// two bf16 values in a word -> two fp16 values in a word
__device__ __forceinline__ unsigned bf2h_word(unsigned w) {
  return pk_h2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}
__device__ __forceinline__ uint4 bf2h(const uint4& x) {
  return make_uint4(bf2h_word(x.x), bf2h_word(x.y), bf2h_word(x.z), bf2h_word(x.w));
}
__device__ __forceinline__ uint4 pick_u4(bool ok, const uint4& x) {
  return make_uint4(ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u, ok ? x.w : 0u);
}

__device__ __forceinline__ f16x8 lds_h8(const _Float16* p) {
  return *reinterpret_cast<const f16x8*>(p);
}

// transposed read (see the header): 4 fp16 values
__device__ __forceinline__ i16x4 lds_tr4(const _Float16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}
// an 8-value operand from two transposed reads
__device__ __forceinline__ f16x8 tr_h8(const _Float16* p0, const _Float16* p1) {
  const i16x4 lo = lds_tr4(p0), hi = lds_tr4(p1);
  const i16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(f16x8, r);
}

__device__ __forceinline__ int uf_off(int s, int t, int h, int lane) {
  return (((s * NT + t) * 2 + h) * 64 + lane) * 16;
}

// global-memory access through an explicitly global pointer (pointers that
// reach a role function through memory would otherwise be accessed with flat
// instructions, which also count against the LDS wait counter)
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

// maximum over the 64 lanes (uniform result)
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // lane ^ 1
  x = fmaxf(x, dpp_f<0x4E>(x));   // lane ^ 2
  x = fmaxf(x, dpp_f<0x141>(x));  // half-row mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row mirror
  const int xi = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// G's layout.  Row r (32 floats) of sub-chunk s holds its eight 4-float
// pieces swizzled: piece j at slot j ^ ((r >> 1) & 7) ^ 2s.  The Gram waves
// write a row per lane, the solver reads 16 rows x one piece per lane (the
// off-diagonal block) or one row per group of 16 lanes, four groups at once
// (the diagonal blocks); with the swizzle each of these touches distinct banks.
__device__ __forceinline__ int g_slot(int r, int j, int s) { return j ^ ((r >> 1) & 7) ^ (2 * s); }

// Back substitution of X_bb (I + L_bb) = I for one row of a 16x16 diagonal
// block, steps i = 15 .. 1: acc[r] -= X[row][i] L[i][r] for r < i, where
// L[i][r] = beta_i G[i][r].  Row i of the block of G is a broadcast read
// (the 16 lanes of a block read the same address), issued PF steps ahead of
// its use; bt holds beta of the block's 16 tokens.  gp[k] points at row 0 of
// the block, stored slot x ^ k with x = 4 blk ^ 2 s (the block's piece 4 blk
// + r4 of row i sits at stored slot x ^ (r4 ^ ((i >> 1) & 7))).
constexpr int PF = 3;
__device__ __forceinline__ void subst16(float (&acc)[16], const float* const (&gp)[8],
                                        const float (&bt)[16]) {
  float4 buf[PF + 1][4];
#pragma unroll
  for (int p = 0; p < PF; ++p)
#pragma unroll
    for (int r4 = 0; r4 < (15 - p + 3) / 4; ++r4)
      buf[p][r4] = *reinterpret_cast<const float4*>(gp[r4 ^ (((15 - p) >> 1) & 7)] + (15 - p) * 32);
#pragma unroll
  for (int i = 15; i >= 1; --i) {
    const int slot = (15 - i) % (PF + 1);
    const int ip = i - PF;  // row read now, used PF steps later
    if (ip >= 1) {
      const int ps = (15 - ip) % (PF + 1);
#pragma unroll
      for (int r4 = 0; r4 < (ip + 3) / 4; ++r4)
        buf[ps][r4] = *reinterpret_cast<const float4*>(gp[r4 ^ ((ip >> 1) & 7)] + ip * 32);
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

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16x16(const f16x4& a, const f16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x4 h4(float x0, float x1, float x2, float x3) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = {pk_h2(x0, x1), pk_h2(x2, x3)};
  return __builtin_bit_cast(f16x4, w);
}

// Staging of K / V rows: 16 items of 16 bytes per lane cover a chunk --
// item i is row (lane >> 4) + 4 i, channels 8 (lane & 15) .. +7 -- so each
// load instruction reads four whole 256-byte rows.  Rows past the chunk's end
// read its last row (a valid address) and are staged as they are: beta is
// zero on them, so their rows and columns of A, A', U and W, and their rows of
// N and M, are exactly zero, and a finite key or value row only ever meets
// zero coefficients.  Channels past the head size read a valid group and are
// zeroed (they would enter K K^T and the products over channels).
template <int NI>
__device__ __forceinline__ void load_rows(uint4 (&pr)[NI], const __bf16* base, int HD, int len,
                                          int i0, int lane) {
  // One code path for whole and short chunks: row (lane >> 4) + 4 (i0 + i),
  // clamped to the chunk's last row by an unsigned minimum of byte offsets
  // (the offsets grow with the row).  With a branch here the compiler tracks
  // the register sets' loads less precisely across the pipeline loop and
  // waits for loads of the set issued after the one being staged.
  const unsigned rb = unsigned(HD) * 2u;
  const unsigned lim = unsigned(len - 1) * rb;
  const unsigned o = unsigned((lane >> 4) + 4 * i0) * rb;
  const char* p = reinterpret_cast<const char*>(base);
#pragma unroll
  for (int i = 0; i < NI; ++i) pr[i] = gload_u4(p + min(o + unsigned(4 * i) * rb, lim));
}
// stored position (halves) of columns 8 cg .. 8 cg + 7 of a K or V row (the
// permutation of 16-column pieces in the header)
__device__ __forceinline__ int col_slot8(int cg) {
  return 16 * ((cg >> 2) + 4 * ((cg >> 1) & 1)) + 8 * (cg & 1);
}
template <int NI>
__device__ __forceinline__ void stage_rows(_Float16* dst, const uint4 (&pr)[NI], int d, int i0, int lane) {
  const int cg = lane & 15;
  _Float16* row = dst + (lane >> 4) * RLD + col_slot8(cg);
  if (d == DP) {
#pragma unroll
    for (int i = 0; i < NI; ++i) *reinterpret_cast<uint4*>(row + 4 * (i0 + i) * RLD) = bf2h(pr[i]);
  } else {
    const bool okc = 8 * cg < d;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<uint4*>(row + 4 * (i0 + i) * RLD) = pick_u4(okc, bf2h(pr[i]));
  }
}

// G_ss = K_s K_s^T of sub-chunk s from the K rows of a chunk (fp32).  G is
// symmetric: the lane's accumulator column cl is also row cl, with entries
// 8 k + 4 g + {0..3} in registers 4k .. 4k+3, so each lane writes its row
// with four 16-byte stores (pieces 2k + g, swizzled).
__device__ __forceinline__ void gram(float* gm, const _Float16* kb, int lane, int s) {
  const int g = lane >> 5, cl = lane & 31;
  {
    f32x16 acc0 = zero16(), acc1 = zero16();
#pragma unroll
    for (int ks = 0; ks < DP / 16; ++ks) {
      const f16x8 ak = lds_h8(kb + (32 * s + cl) * RLD + 16 * ks + 8 * g);
      if (ks & 1)
        acc1 = mfma16(ak, ak, acc1);
      else
        acc0 = mfma16(ak, ak, acc0);
    }
    float* row = gm + s * 1024 + cl * 32;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
      *reinterpret_cast<float4*>(row + 4 * g_slot(cl, 2 * k4 + g, s)) =
          make_float4(acc0[4 * k4] + acc1[4 * k4], acc0[4 * k4 + 1] + acc1[4 * k4 + 1],
                      acc0[4 * k4 + 2] + acc1[4 * k4 + 2], acc0[4 * k4 + 3] + acc1[4 * k4 + 3]);
  }
}

// U^T tiles tile0 .. tile0+NTL-1 of chunk j -> -U fragments.  Tile i covers
// sub-chunk i / NT, columns 32 (i % NT) ..  K^T fragment: lane (g, m) needs
// K[token 32 s + 16 kk + 8 g + 0..7][32 t + m].  All operands are read before
// the products, so the reads of the tiles overlap.
template <int NTL>
__device__ __forceinline__ void ut_tiles(const _Float16* kb, const _Float16* Ah, char* uf, int tile0,
                                         int lane) {
  const int g = lane >> 5, cl = lane & 31;
  const int ti = lane & 15, tg = lane >> 4;
  const int tr_row = ti >> 2, tr_col = 64 * (tg & 1) + 4 * (ti & 3);  // (stored slots)
  const _Float16* kbase = kb + (8 * g + tr_row) * RLD + tr_col;
  f16x8 kf[NTL][2], ah[NTL][2];
#pragma unroll
  for (int i = 0; i < NTL; ++i) {
    const int t = (tile0 + i) % NT, s = (tile0 + i) / NT;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const _Float16* p0 = kbase + (32 * s + 16 * kk) * RLD + 16 * t;
      kf[i][kk] = tr_h8(p0, p0 + 4 * RLD);
      ah[i][kk] = lds_h8(Ah + (32 * s + cl) * A_LD + 16 * kk + 8 * g);
    }
  }
#pragma unroll
  for (int i = 0; i < NTL; ++i) {
    const int t = (tile0 + i) % NT, s = (tile0 + i) / NT;
    f32x16 acc = zero16();
    acc = mfma16(kf[i][0], ah[i][0], acc);
    acc = mfma16(kf[i][1], ah[i][1], acc);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      *reinterpret_cast<f16x8*>(uf + uf_off(s, t, hh, lane)) = acc_h8<-1>(acc, hh);
  }
}

// wave-uniform copies (values that reach a role through memory would
// otherwise be treated as per-lane, turning uniform branches into exec masks)
__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t rfl64(int64_t v) {
  const uint32_t lo = uint32_t(rfl(int(uint32_t(v)))), hi = uint32_t(rfl(int(uint64_t(v) >> 32)));
  return int64_t((uint64_t(hi) << 32) | lo);
}
template <class T>
__device__ __forceinline__ T* rflp(T* p) {
  return reinterpret_cast<T*>(rfl64(reinterpret_cast<int64_t>(p)));
}

// Per-block values shared by the three roles.  Each role is its own
// non-inlined function, so that the register allocator sees one role at a
// time (inlined into one body, the three live-range sets interfere).
struct Ctx {
  int64_t t_begin, t_end, N, unit;
  int n, b, h;
};

// The fields of the call that the roles read.  The roles take this (not the
// kernel's argument block, which also carries the plan tables) so that the
// per-lane copy the calls make stays small.
struct Core {
  int heads, dk, dv;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  float* log_scale;
  float* T_hat;
  float* S0;
  unsigned* nonfinite;
};

// the workgroup's LDS, at file scope so that every role function addresses
// it directly (LDS instructions, not flat ones)
__shared__ __attribute__((aligned(16))) char h16_smem[LDS_TOTAL];

__device__ __noinline__ void consumer_role(const Core& a, const Ctx& x);
__device__ __noinline__ void solver_role(const Core& a, const Ctx& x);
__device__ __noinline__ void kstage_role(const Core& a, const Ctx& x);
__device__ __noinline__ void vstage_role(const Core& a, const Ctx& x);

__global__ __launch_bounds__(THREADS) void build_dense_h16_kernel(BuildArgs a) {
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
  const Core core{a.heads, a.dk, a.dv,      a.k,    a.v,  a.alpha,
                  a.beta,  a.log_scale, a.T_hat, a.S0, a.nonfinite};
  const int wid = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  if (wid < NT)
    consumer_role(core, x);
  else if (wid == NT)
    solver_role(core, x);
  else if (wid < NT + NHW)
    kstage_role(core, x);
  else
    vstage_role(core, x);
}

#define PIC_H16_ROLE_PROLOGUE                                                   \
  _Float16* Kb0 = reinterpret_cast<_Float16*>(h16_smem + L_K);                  \
  _Float16* Vb = reinterpret_cast<_Float16*>(h16_smem + L_V);                   \
  float* Nm0 = reinterpret_cast<float*>(h16_smem + L_NM);                       \
  _Float16* AB0 = reinterpret_cast<_Float16*>(h16_smem + L_AB);                 \
  char* Uf0 = h16_smem + L_UF;                                                  \
  float* gb0 = reinterpret_cast<float*>(h16_smem + L_GB);                       \
  float* gbr0 = reinterpret_cast<float*>(h16_smem + L_GBR);                     \
  float* gg = reinterpret_cast<float*>(h16_smem + L_GG);                        \
  const int H = rfl(a.heads), dk = rfl(a.dk), dv = rfl(a.dv);                   \
  const int b = rfl(x.b), h = rfl(x.h), n = rfl(x.n);                           \
  const int64_t t_begin = rfl64(x.t_begin), t_end = rfl64(x.t_end);             \
  const int64_t N = rfl64(x.N), unit = rfl64(x.unit);                           \
  const __bf16* kp = rflp(static_cast<const __bf16*>(a.k));                     \
  const __bf16* vp = rflp(static_cast<const __bf16*>(a.v));                     \
  const float* alpha = rflp(a.alpha);                                           \
  const float* beta = rflp(a.beta);                                             \
  float* out_lam = rflp(a.log_scale);                                           \
  float* out_T = rflp(a.T_hat);                                                 \
  float* out_S = rflp(a.S0);                                                    \
  const int lane = threadIdx.x & 63, g = lane >> 5, cl = lane & 31;             \
  const int wid = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));        \
  /* transposed reads: group lane ti supplies row ti >> 2 of a 4-row block   */ \
  /* and columns 4 (ti & 3) .. +3 of the group's 16-column half (stored at   */ \
  /* slot t or t + 4 of tile t: add 16 t)                                     */ \
  const int ti = lane & 15, tg = lane >> 4;                                     \
  const int tr_row = ti >> 2, tr_col = 64 * (tg & 1) + 4 * (ti & 3);            \
  auto chunk_len = [&](int j) {                                                 \
    const int64_t c0 = t_begin + int64_t(j) * C;                                \
    return (t_end - c0 < C) ? int(t_end - c0) : C;                              \
  };                                                                            \
  (void)Kb0; (void)Vb; (void)Nm0; (void)AB0; (void)Uf0; (void)gb0;   \
  (void)gbr0; (void)gg; (void)H; (void)dk; (void)dv; (void)b; (void)h; (void)N; \
  (void)unit; (void)g; (void)cl; (void)wid; (void)chunk_len; (void)t_begin;     \
  (void)t_end; (void)kp; (void)vp; (void)alpha; (void)beta; (void)out_lam;      \
  (void)out_T; (void)out_S; (void)tr_row; (void)tr_col

// ===========================================================================
// consumer wave c: columns [32c, 32c+32) of That (scaled by 2^E) and S
// ===========================================================================
__device__ __noinline__ void consumer_role(const Core& a, const Ctx& x) {
  PIC_H16_ROLE_PROLOGUE;
  PIC_PHASE_DECL;
  const int c = wid;
  f32x16 XT[NT], XS[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    XS[t] = zero16();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = t * 32 + acc_row(q, g), col = c * 32 + cl;
      XT[t][q] = (row == col && row < dk) ? 1.f : 0.f;
    }
  }
  int E = 0;

  // Lazy decay of S.  XS holds S / G, where G is the product of the
  // sub-chunk decays gamma since the last eager step, so that a lazy step
  // needs no pass over the state: S' = gamma S + K^T (W - U gamma S) becomes
  // XS' = XS + K^T (W / G' - U XS) with G' = G gamma, and the 1/G' of the W
  // seed is already folded into beta * r by the gate wave.  When G gamma would
  // drop below 2^kLazyLog2 the step is eager instead: XS *= G gamma, G = 1.
  // So |XS| <= 2^-kLazyLog2 |S| (the fp16 operand range bounds |S|).

  // sub-chunk s of chunk j, seed P = W / G' (this wave's columns):
  // [eager: S *= em]; N = -U That, M = W - U S; That += K^T N, S += K^T M
  auto chain_sub = [&](int s, int j, f32x16 P) {
    const char* uf = Uf0 + (j & 1) * UF_BYTES;
    const _Float16* kb = Kb0 + (j % NKB) * (C * RLD);
    // every -U fragment of the sub-chunk, read before anything waits
    f16x8 uu[2 * NT];
#pragma unroll
    for (int ks = 0; ks < 2 * NT; ++ks)
      uu[ks] = *reinterpret_cast<const f16x8*>(uf + uf_off(s, ks >> 1, ks & 1, lane));
    const int emi = rfl(__float_as_int(gg[(j & 3) * 2 + s]));
    if (emi >= 0) {  // eager step (uniform)
      const float em = __int_as_float(emi);
#pragma unroll
      for (int t = 0; t < NT; ++t) XS[t] *= em;
    }
    // K^T fragment of K-step hh, tile t: lane (g, m) needs K[token][32t + m]
    // for tokens kperm(hh, g, 0..7) = 16 hh + 4 g + {0..3, 8..11} of the
    // sub-chunk -- the row order of the N / M accumulator halves
    const _Float16* kbase = kb + (32 * s + 4 * g + tr_row) * RLD + tr_col;
    f16x8 kf[2][NT];
    f32x16 PN = zero16();
    // k-steps in source order (a scheduling barrier after each), so that the
    // -U fragments die one by one and the K^T reads of the second stage are
    // issued while the first stage still has matrix work queued
#pragma unroll
    for (int ks = 0; ks < 2 * NT; ++ks) {
      const int t = ks >> 1, hh = ks & 1;
      const f16x8 tb = acc_h8(XT[t], hh), sb = acc_h8(XS[t], hh);
      PN = mfma16(uu[ks], tb, PN);
      P = mfma16(uu[ks], sb, P);
      if (ks == 3 || ks == 5) {
        const int kh = ks == 3 ? 0 : 1;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const _Float16* p0 = kbase + 16 * kh * RLD + 16 * tt;
          kf[kh][tt] = tr_h8(p0, p0 + 8 * RLD);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const f16x8 nb = acc_h8(PN, hh), mb = acc_h8(P, hh);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        XT[t] = mfma16(kf[hh][t], nb, XT[t]);
        XS[t] = mfma16(kf[hh][t], mb, XS[t]);
      }
    }
  };

  // W seed of sub-chunk s of chunk j: M_s = A'_s V_s (this wave's columns;
  // A' carries the lazy 1/G')
  auto seed = [&](int j, int s) {
    const _Float16* Ap = AB0 + (j & 1) * AB_HALFS + 64 * A_LD;
    // V^T fragment: lane (g, n) needs V[token 16 kk + 8 g + 0..7][32 c + n]
    const _Float16* vbase = Vb + (8 * g + tr_row) * RLD + 16 * c + tr_col;
    f32x16 acc = zero16();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const f16x8 ph = lds_h8(Ap + (32 * s + cl) * A_LD + 16 * kk + 8 * g);
      const _Float16* p0 = vbase + (32 * s + 16 * kk) * RLD;
      const f16x8 vf = tr_h8(p0, p0 + 4 * RLD);
      acc = mfma16(ph, vf, acc);
    }
    return acc;
  };
  // re-normalise this wave's columns of That by a power of two -- branch-free,
  // so that no copy of the state is made
  auto renorm = [&]() {
    float m = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(XT[t][q]));
    m = wave_max(m);
    int e;
    (void)frexpf(m, &e);
    e = (m > 0.f) ? (e < -120 ? -120 : e) : 0;
    const float sc = ldexpf(1.f, -e);
#pragma unroll
    for (int t = 0; t < NT; ++t) XT[t] *= sc;
    E += e;
  };

  // Cycles -1 .. n+1 of the pipeline, peeled so that the steady-state loop
  // has no branch around the chain (see the schedule at the top).
  PIC_BAR(0);  // cycle -1, phase A
  PIC_BAR(1);  //           phase B
  PIC_BAR(0);  // cycle 0,  phase A
  PIC_BAR(1);  //           phase B
  if (n >= 1) {
    PIC_BAR(0);  // cycle 1, phase A
    PIC_BAR(1);  //          phase B
    renorm();
    chain_sub(0, 0, seed(0, 0));
    f32x16 PM1 = seed(0, 1);  // (V of the chunk is replaced in the next phase)
    int ci = 2;
    // (the re-normalisation of That every fourth chunk sits at the end of
    // phase A; That's norm shrinks by about 0.87 per chunk at the usual gates,
    // so four chunks stay far inside fp16's range)
#pragma unroll 1
    for (; ci + 1 <= n; ci += 2) {
      PIC_BAR(0);  // phase A
      chain_sub(1, ci - 2, PM1);
      PIC_BAR(1);  // phase B
      chain_sub(0, ci - 1, seed(ci - 1, 0));
      PM1 = seed(ci - 1, 1);
      PIC_BAR(0);  // phase A
      chain_sub(1, ci - 1, PM1);
      if (((ci >> 1) & 1) == 0) renorm();  // every fourth chunk
      PIC_BAR(1);  // phase B
      chain_sub(0, ci, seed(ci, 0));
      PM1 = seed(ci, 1);
    }
    if (ci <= n) {
      PIC_BAR(0);  // phase A
      chain_sub(1, ci - 2, PM1);
      PIC_BAR(1);  // phase B
      chain_sub(0, ci - 1, seed(ci - 1, 0));
      PM1 = seed(ci - 1, 1);
    }
    PIC_BAR(0);  // cycle n+1, phase A
    chain_sub(1, n - 1, PM1);
    PIC_BAR(1);  //            phase B
  } else {
    PIC_BAR(0);  // cycle 1, phase A
    PIC_BAR(1);  //          phase B
  }

  PIC_PHASE_SAVE;
  // write this wave's columns of S(C|0) (= 2^lg XS, lg the final log2 G of
  // the lazy decay) and That_C
  const int ncol = c * 32 + cl;
  bool bad = false;
  if (ncol < dv) {
    float* out = out_S + unit * int64_t(dk) * dv;
    const float gs = n >= 1 ? exp2f(gg[8]) : 1.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = t * 32 + acc_row(q, g);
        const float v = float(XS[t][q]) * gs;
        bad |= not_finite(v);
        if (row < dk) gstore(out + int64_t(row) * dv + ncol, v);
      }
  }
  if (ncol < dk) {
    float* out = out_T + unit * int64_t(dk) * dk;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = t * 32 + acc_row(q, g);
        const float v = ldexpf(XT[t][q], E);
        bad |= not_finite(v);
        if (row < dk) gstore(out + int64_t(row) * dk + ncol, v);
      }
  }
  report_nonfinite(a.nonfinite, bad);
}

// ===========================================================================
// solver wave: X_s = (I + L_s)^{-1} of both sub-chunks.  Phase A: the four
// 16x16 diagonal blocks by back substitution, lane 32 s + 16 b + j owning
// row j of block b of sub-chunk s; the rows go to a scratch tile (fp16).
// Phase B: the off-diagonal block X_10 = -X_11 L_10 X_00 of each sub-chunk
// with two 16x16x16 matrix-core products (their B operands are read
// transposed from the scratch tile; the first product's accumulators are
// already the second one's B operand), then A = X diag(beta) and
// A' = X diag(beta r) to LDS.  The scratch is the A/A' buffer of the chunk
// being solved: its previous chunk was last read in the cycle before.
// ===========================================================================
constexpr int XS_LD = 48;  // scratch row stride (halves): 96 bytes, so that the
                           // four rows of a transposed read hit distinct banks
__device__ __noinline__ void solver_role(const Core& a, const Ctx& x) {
  PIC_H16_ROLE_PROLOGUE;
  PIC_PHASE_DECL;
  const int s = lane >> 5, blk = (lane >> 4) & 1, jr = lane & 15;
  float acc[16], bt[16];
#pragma unroll 1
  for (int ci = -1; ci <= n + 1; ++ci) {
    const bool solve = ci >= 0 && ci < n;
    const float* gm = Nm0 + (ci & 1) * NM_FLOATS;          // G of both sub-chunks
    const float* gbp = gb0 + (ci & 1) * C;                 // masked beta
    const float* grp = gbr0 + (ci & 1) * C;                // beta * r
    _Float16* ab = AB0 + (ci & 1) * AB_HALFS;              // scratch, then A / A'
    PIC_BAR(0);  // phase A
    if (solve) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 b4 = *reinterpret_cast<const float4*>(gbp + 32 * s + 16 * blk + 4 * q);
        bt[4 * q] = b4.x; bt[4 * q + 1] = b4.y; bt[4 * q + 2] = b4.z; bt[4 * q + 3] = b4.w;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = (r == jr) ? 1.f : 0.f;
      const float* gp[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) gp[k] = gm + s * 1024 + (16 * blk) * 32 + 4 * ((4 * blk ^ 2 * s) ^ k);
      subst16(acc, gp, bt);
      // row jr of block blk -> scratch tile (s, blk)
      _Float16* xr = ab + ((2 * s + blk) * 16 + jr) * XS_LD;
      *reinterpret_cast<uint4*>(xr) = make_uint4(pk_h2(acc[0], acc[1]), pk_h2(acc[2], acc[3]),
                                                 pk_h2(acc[4], acc[5]), pk_h2(acc[6], acc[7]));
      *reinterpret_cast<uint4*>(xr + 8) = make_uint4(pk_h2(acc[8], acc[9]), pk_h2(acc[10], acc[11]),
                                                     pk_h2(acc[12], acc[13]), pk_h2(acc[14], acc[15]));
    }
    // U^T tiles 6, 7 of chunk ci-1
    if (ci - 1 >= 0 && ci - 1 < n) {
      const int j = ci - 1;
      ut_tiles<2>(Kb0 + (j % NKB) * (C * RLD), AB0 + (j & 1) * AB_HALFS, Uf0 + (j & 1) * UF_BYTES,
                  6, lane);
    }
    PIC_BAR(1);  // phase B
    if (solve) {
      // off-diagonal blocks; 16x16x16 layouts: lane l holds A[l%16][4(l/16)+e],
      // B[4(l/16)+e][l%16], D[4(l/16)+e][l%16], e = 0..3
      const int m = lane & 15, kq = lane >> 4;
      f32x4 X10[2];
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const float4 g4 =
            *reinterpret_cast<const float4*>(gm + ss * 1024 + (16 + m) * 32 + 4 * g_slot(16 + m, kq, ss));
        const float bm = gbp[32 * ss + 16 + m];
        const f16x4 l10 = h4(bm * g4.x, bm * g4.y, bm * g4.z, bm * g4.w);
        const _Float16* t00 = ab + (2 * ss) * 16 * XS_LD;
        const _Float16* t11 = ab + (2 * ss + 1) * 16 * XS_LD;
        const f16x4 x00 = __builtin_bit_cast(f16x4, lds_tr4(t00 + (4 * kq + (m >> 2)) * XS_LD + 4 * (m & 3)));
        const f16x4 x11 = *reinterpret_cast<const f16x4*>(t11 + m * XS_LD + 4 * kq);
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        y = mfma16x16(l10, x00, y);
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        X10[ss] = mfma16x16(x11, h4(y[0], y[1], y[2], y[3]), z);
      }
      // rows of the diagonal blocks (this lane's row of block blk), the other
      // half of the row: zeros (block 0) or the off-diagonal block (block 1,
      // written below)
      const int row = 32 * s + 16 * blk + jr;
      _Float16* arow = ab + row * A_LD;
      _Float16* brow = arow + 64 * A_LD;
      const float* bk = bt;  // beta of the block's tokens (phase A)
      float rk[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 r4 = *reinterpret_cast<const float4*>(grp + 32 * s + 16 * blk + 4 * q);
        rk[4 * q] = r4.x; rk[4 * q + 1] = r4.y; rk[4 * q + 2] = r4.z; rk[4 * q + 3] = r4.w;
      }
      uint4 wa[2], wb[2];
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int k = 8 * h8;
        wa[h8] = make_uint4(pk_h2(acc[k] * bk[k], acc[k + 1] * bk[k + 1]),
                            pk_h2(acc[k + 2] * bk[k + 2], acc[k + 3] * bk[k + 3]),
                            pk_h2(acc[k + 4] * bk[k + 4], acc[k + 5] * bk[k + 5]),
                            pk_h2(acc[k + 6] * bk[k + 6], acc[k + 7] * bk[k + 7]));
        wb[h8] = make_uint4(pk_h2(acc[k] * rk[k], acc[k + 1] * rk[k + 1]),
                            pk_h2(acc[k + 2] * rk[k + 2], acc[k + 3] * rk[k + 3]),
                            pk_h2(acc[k + 4] * rk[k + 4], acc[k + 5] * rk[k + 5]),
                            pk_h2(acc[k + 6] * rk[k + 6], acc[k + 7] * rk[k + 7]));
      }
      // (the scratch reads above precede these stores in the wave's LDS
      // order, so they see the scratch before it is overwritten)
      *reinterpret_cast<uint4*>(arow + 16 * blk) = wa[0];
      *reinterpret_cast<uint4*>(arow + 16 * blk + 8) = wa[1];
      *reinterpret_cast<uint4*>(brow + 16 * blk) = wb[0];
      *reinterpret_cast<uint4*>(brow + 16 * blk + 8) = wb[1];
      if (blk == 0) {
        const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(arow + 16) = z4;
        *reinterpret_cast<uint4*>(arow + 24) = z4;
        *reinterpret_cast<uint4*>(brow + 16) = z4;
        *reinterpret_cast<uint4*>(brow + 24) = z4;
      }
      // off-diagonal blocks: lane l holds X10[4 kq + e][m] of each sub-chunk
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const float bn = gbp[32 * ss + m], rn = grp[32 * ss + m];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 32 * ss + 16 + 4 * kq + e;
          ab[r * A_LD + m] = _Float16(-X10[ss][e] * bn);
          ab[(64 + r) * A_LD + m] = _Float16(-X10[ss][e] * rn);
        }
      }
    }
  }
  PIC_PHASE_SAVE;
}

// ===========================================================================
// K waves: K rows (half each), U^T tiles, G; V wave: V rows and the gates
// ===========================================================================
__device__ __noinline__ void kstage_role(const Core& a, const Ctx& x) {
  PIC_H16_ROLE_PROLOGUE;
  PIC_PHASE_DECL;
  const int pw = wid - NT - 1;  // 0 or 1
  const int HDk = H * dk;       // element stride between tokens
  const int kch = min(8 * (lane & 15), dk - 8);
  // K rows: K wave pw stages rows [32 pw, 32 pw + 32) of each chunk (items
  // 8 pw .. 8 pw + 7), loaded two cycles ahead
  const int i0 = 8 * pw;
  uint4 pr0[8], pr1[8];  // two chunks' rows (even and odd chunks)
  auto row0 = [&](int j) { return (int64_t(b) * N + t_begin + int64_t(j) * C) * H + h; };
  // pr holds the rows of chunk ci+1; once staged, it takes chunk ci+3.  The
  // chunk index is clamped rather than the load skipped, so that every cycle
  // issues the same loads and the wait before a staging covers only the set
  // being staged.
  auto cycle = [&](int ci, uint4 (&pr)[8]) __attribute__((always_inline)) {
    // ---------------- phase A: K rows of chunk ci+1, load chunk ci+3's;
    // U^T tiles 3 pw .. 3 pw + 2 of chunk ci-1
    PIC_BAR(0);
    if (ci + 1 < n)
      stage_rows(Kb0 + ((ci + 1) % NKB) * (C * RLD), pr, dk, i0, lane);
    {
      const int jl = min(ci + 3, n - 1);
      load_rows(pr, kp + row0(jl) * dk + kch, HDk, chunk_len(jl), i0, lane);
    }
    if (ci - 1 >= 0 && ci - 1 < n) {
      const int j = ci - 1;
      ut_tiles<3>(Kb0 + (j % NKB) * (C * RLD), AB0 + (j & 1) * AB_HALFS, Uf0 + (j & 1) * UF_BYTES,
                  3 * pw, lane);
    }
    // ---------------- phase B: G of sub-chunk pw of chunk ci+1
    PIC_BAR(1);
    if (ci + 1 < n)
      gram(Nm0 + ((ci + 1) & 1) * NM_FLOATS, Kb0 + ((ci + 1) % NKB) * (C * RLD), lane, pw);
  };
  if (n > 0) {
    load_rows(pr0, kp + row0(0) * dk + kch, HDk, chunk_len(0), i0, lane);
    load_rows(pr1, kp + row0(min(1, n - 1)) * dk + kch, HDk, chunk_len(min(1, n - 1)), i0, lane);
    int ci = -1;
#pragma unroll 1
    for (; ci + 1 <= n + 1; ci += 2) {
      cycle(ci, pr0);
      cycle(ci + 1, pr1);
    }
    if (ci <= n + 1) cycle(ci, pr0);
  } else {
#pragma unroll 1
    for (int ci = -1; ci <= n + 1; ++ci) {
      PIC_BAR(0);
      PIC_BAR(1);
    }
  }
  PIC_PHASE_SAVE;
}

// V rows and gates (the last wave)
__device__ __noinline__ void vstage_role(const Core& a, const Ctx& x) {
  PIC_H16_ROLE_PROLOGUE;
  PIC_PHASE_DECL;
  const float* bsrc = beta ? beta : alpha;
  const int HDv = H * dv;  // element stride between tokens
  const int vch = min(8 * (lane & 15), dv - 8);
  uint4 prv[2][16];  // V rows of two chunks (items 0..15), loaded two cycles ahead
  // alpha, beta of lane's token for two chunks, indexed by chunk parity, so
  // that no register holding a pending load is copied
  float pa[2] = {1.f, 1.f}, pb[2] = {0.f, 0.f};
  float lam = 0.f;
  float lg = 0.f;  // log2 G of the lazy decay, uniform
  auto row0 = [&](int j) { return (int64_t(b) * N + t_begin + int64_t(j) * C) * H + h; };
  auto load_gates = [&](int j, float& ra, float& rb) {
    const int64_t gi = row0(j) + int64_t(min(lane, chunk_len(j) - 1)) * H;
    ra = gload(alpha + gi);
    rb = gload(bsrc + gi);
  };

  // one pipeline cycle; P = parity of chunk ci+1 (compile-time register slot)
  auto cycle = [&](int ci, auto par) {
    constexpr int P = decltype(par)::value;
    // ---------------- phase A: V rows of chunk ci-1, then load chunk ci+1's
    // into the same set (clamped, as the K rows)
    PIC_BAR(0);
    if (ci - 1 >= 0 && ci - 1 < n) stage_rows(Vb, prv[P], dv, 0, lane);
    {
      const int jl = min(ci + 1, n - 1);
      load_rows(prv[P], vp + row0(jl) * dv + vch, HDv, chunk_len(jl), 0, lane);
    }
    // ---------------- phase B: gates of chunk ci+1
    PIC_BAR(1);
    if (ci + 1 < n) {
      // log2 prefix per sub-chunk (one per half wave)
      const int jn = ci + 1;
      const int len = chunk_len(jn);
      const float x2 = half_wave_scan(lane < len ? log2f(pa[P]) : 0.f);
      const int xi = __builtin_bit_cast(int, x2);
      const float e0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 31));
      const float e1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 63));
      const float bend = g ? e1 : e0;
      const float bt = lane < len ? (beta ? pb[P] : 1.f) : 0.f;  // masked beta
      // lazy decay of S (see the consumer): per sub-chunk, either the
      // consumers keep S / G with G <- G gamma (lazy: the W seed takes 1/G),
      // or, when G gamma would drop below 2^kLazyLog2, they multiply S by
      // G gamma and G restarts at 1 (eager: em >= 0)
      float em[2], sl[2];
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const float e = ss ? e1 : e0;
        if (lg + e >= kLazyLog2) {
          lg += e;
          em[ss] = -1.f;
          sl[ss] = -lg;
        } else {
          em[ss] = exp2f(lg + e);
          lg = 0.f;
          sl[ss] = 0.f;
        }
      }
      gb0[(jn & 1) * C + lane] = bt;
      gbr0[(jn & 1) * C + lane] = bt * exp2f(bend - x2 + (g ? sl[1] : sl[0]));
      if (lane == 0) {
        gg[(jn & 3) * 2] = em[0];
        gg[(jn & 3) * 2 + 1] = em[1];
        if (jn == n - 1) gg[8] = lg;  // S(C|0) = 2^lg x the consumers' S
      }
      lam += e0 + e1;
    }
    // the slot of chunk ci+1 now takes chunk ci+3 (clamped)
    load_gates(min(ci + 3, n - 1), pa[P], pb[P]);
  };

  if (n > 0) {
    load_gates(0, pa[0], pb[0]);
    load_gates(min(1, n - 1), pa[1], pb[1]);
    // chunk ci+1 has parity (ci+1) & 1: cycles -1, 1, 3, ... use slot 0
    int ci = -1;
#pragma unroll 1
    for (; ci + 1 <= n + 1; ci += 2) {
      cycle(ci, std::integral_constant<int, 0>{});
      cycle(ci + 1, std::integral_constant<int, 1>{});
    }
    if (ci <= n + 1) cycle(ci, std::integral_constant<int, 0>{});
  } else {
#pragma unroll 1
    for (int ci = -1; ci <= n + 1; ++ci) {
      PIC_BAR(0);
      PIC_BAR(1);
    }
  }
  if (lane == 0) gstore(out_lam + unit, lam * kLn2);
  PIC_PHASE_SAVE;
}

}  // namespace

hipError_t launch_build_dense_h16(const BuildArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_seg) * a.batch * a.heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(build_dense_h16_kernel, dim3(unsigned(blocks)), dim3(THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace pic

#ifdef PIC_PHASE_TIMING
// Diagnostic library only: where the dense fp16 build writes its per-wave
// phase clocks ([block][wave][8]: length of phase A, wait at its end, length
// of phase B, wait at its end, total clocks, cycles, 2 unused) for blocks
// below `blocks`.
extern "C" int pic_phase_timing_set(void* dev_buf, int blocks) {
  if (hipMemcpyToSymbol(HIP_SYMBOL(pic::pic_phase_out), &dev_buf, sizeof(dev_buf)) != hipSuccess)
    return -7;
  if (hipMemcpyToSymbol(HIP_SYMBOL(pic::pic_phase_blocks), &blocks, sizeof(blocks)) != hipSuccess)
    return -7;
  return 0;
}
#endif
