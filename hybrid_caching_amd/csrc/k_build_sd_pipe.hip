// k_build_sd_pipe.hip -- build of the scalar-decay and diagonal-gate pairs
// (lambda_C, S(C|0)) for bf16 k/v, streaming: the contraction is on
// split-bf16 MFMA, the next chunk is staged into a second LDS buffer while
// the current one is contracted, and the inputs of the chunks after that are
// in flight in registers.  Same arithmetic as k_build_scalar_diag.hip (which
// serves fp32 inputs).
// [xix.ai HYPIC article (French), paragraph on linear layers: T_C is the
//  product of the token transitions, S(C|0) the final state from zero; decay
//  (RetNet, Mamba2) and gating (GLA) families.  remio.ai (Japanese), section on
//  state composition: scalar and diagonal transition forms.]
//
// For a block of tokens with w_t = prod_{s > t in the block} alpha_s (per key
// channel for the diagonal form) and gamma = prod over the block:
//   S <- gamma (.) S + Kw^T V,   Kw_t = w_t (.) k_t   (factors <= 1)
// A chunk is 64 tokens.  The scalar form takes the whole chunk as one block;
// the diagonal form takes the 16 (or 32) tokens one wave stages as a block,
// so that its per-channel suffix products stay inside the wave, and rescales
// the state between the blocks of a chunk.
//
// Loads.  Every load instruction reads whole 128-byte lines of token rows
// (16 lanes x 16 bytes of k or v, 16 lanes x 16 bytes of gates, or 16 lanes x
// 8 bytes); instructions that scatter 8- or 16-byte pieces over many rows
// stall the issue of vector memory instructions.  Chunk j's inputs are loaded
// into register set j % 2, two chunks before chunk j is staged.  Every load
// instruction of the steady state is issued unconditionally (chunk indices
// past the end are clamped to the last chunk), so the wait before a staging
// step covers only the register set it stages.
//
// Pipeline: step j reads chunk j's operand fragments (LDS buffer j & 1),
// stages chunk j+1 into the other buffer, issues the loads of chunk j+3 into
// the register set it has just staged, contracts chunk j; one barrier.
#include <type_traits>

#include "mfma_util.hpp"
#include "pic_internal.hpp"

namespace pic {
namespace {

constexpr int kCs = 64;  // tokens per chunk

__device__ __forceinline__ int opaque_i(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// log2 and exp2 on the hardware instructions.  Gates are clamped to the
// smallest normal float before the logarithm (the instruction does not take
// denormal inputs; a gate of 0 would give -inf and then NaN weights).  For
// x >= 0 the integer order of the bit patterns is the float order, so the
// clamp is one integer max.  exp2 of an argument below -126 gives 0, which is
// where the weight of a token is below fp32's normal range anyway.
__device__ __forceinline__ float log2_gate(float x) {
  return __builtin_amdgcn_logf(__int_as_float(max(__float_as_int(x), 0x00800000)));
}
__device__ __forceinline__ float exp2_w(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf_at(const uint4& a, int j) {
  const unsigned w = (j < 2) ? a.x : (j < 4) ? a.y : (j < 6) ? a.z : a.w;
  return (j & 1) ? bf_hi(w) : bf_lo(w);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives, for
// j = 0..3, 16-bit element (i & 3) of the 8 bytes addressed by lane
// 4j + (i >> 2).  When lane 4j + q of the group addresses row r0 + j, columns
// c0 + 4q .. c0 + 4q + 3 of a row-major tile, lane i receives rows
// r0 .. r0+3 of column c0 + i.
__device__ __forceinline__ i16x4 lds_tr4(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}
__device__ __forceinline__ bf16x8 tr_bf8(const __bf16* p0, const __bf16* p1) {
  const i16x4 lo = lds_tr4(p0), hi = lds_tr4(p1);
  const i16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// shared set-up of one (segment, layer, head) unit
struct Unit {
  int seg, b, h, n_chunks;
  int64_t n_tok, unit;
};
__device__ __forceinline__ Unit unit_of(const BuildArgs& a) {
  Unit u;
  const int H = a.heads, BH = a.batch * H;
  u.seg = a.d_order[blockIdx.x / BH];
  const int bh = blockIdx.x % BH;
  u.b = bh / H;
  u.h = bh % H;
  const int64_t t_begin = a.d_offsets[u.seg];
  u.n_tok = a.d_offsets[u.seg + 1] - t_begin;
  u.n_chunks = int((u.n_tok + kCs - 1) / kCs);
  u.unit = (int64_t(u.seg) * a.batch + u.b) * H + u.h;
  return u;
}
__device__ __forceinline__ int chunk_len(const Unit& u, int ci) {
  const int64_t rest = u.n_tok - int64_t(ci) * kCs;
  return rest < kCs ? int(rest) : kCs;
}
// element offset of token t_begin of this (layer, head) in a [B][N][H][d] tensor
__device__ __forceinline__ int64_t row0(const BuildArgs& a, const Unit& u, int d) {
  return ((int64_t(u.b) * a.n_tokens + a.d_offsets[u.seg]) * a.heads + u.h) * d;
}

// Runs the two-chunk-deep pipeline: load(set, chunk) issues the loads of a
// chunk into register set `set` (a std::integral_constant), stage(set, chunk,
// buffer) stages it, frags(chunk, buffer) reads a chunk's operand fragments
// into a value that contract(value, chunk) consumes.
template <class LoadF, class StageF, class FragF, class ContractF>
__device__ __forceinline__ void run_pipeline(int n_chunks, LoadF&& load, StageF&& stage,
                                             FragF&& frags, ContractF&& contract) {
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  if (n_chunks <= 0) return;
  const int last = n_chunks - 1;
  load(S0(), 0);
  load(S1(), min(1, last));
  stage(S0(), 0, 0);
  load(S0(), min(2, last));
  __syncthreads();
  auto step = [&](auto D, int cj) __attribute__((always_inline)) {
    using DN = std::integral_constant<int, (decltype(D)::value + 1) & 1>;
    auto fr = frags(cj, cj & 1);
    if (cj + 1 < n_chunks) stage(DN(), cj + 1, (cj + 1) & 1);
    load(DN(), min(cj + 3, last));
    contract(fr, cj);
    __syncthreads();
  };
  int cj = 0;
#pragma unroll 1
  for (; cj + 1 < n_chunks; cj += 2) {
    step(S0(), cj);
    step(S1(), cj + 1);
  }
  if (cj < n_chunks) step(S0(), cj);
}

// write this wave's tiles of S (rows mt*32.., columns (nt0+k)*32..)
template <int TPW>
__device__ __forceinline__ void write_tiles(const f32x16 (&S)[TPW], float* out, int mt, int nt0,
                                            int dk, int dv) {
  const int lane = threadIdx.x & 63, g = lane >> 5, cl = lane & 31;
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int col = (nt0 + k) * 32 + cl;
    if (col < dv) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mt * 32 + acc_row(r, g);
        if (row < dk) out[int64_t(row) * dv + col] = S[k][r];
      }
    }
  }
}

// ============================================================ scalar decay
//
// Thread mapping: lanes along channels, DP/8 lanes per token row, each thread
// tokens t0 = 2 * (tid / (DP/8)) and t0+1, channels i0 .. i0+7.  The weights
// of the chunk's 64 tokens come from one 64-lane scan that every wave does
// for itself (lane = token), and reach the threads by ds_bpermute.  Kw (hi,
// lo) and V are staged token-major (16-byte pieces of rows); the contraction
// reads its transposed operand fragments with ds_read_b64_tr_b16.
template <int DP>
struct ScalarLds {
  static constexpr int RLD = DP + 16;              // row stride (bf16): the 16 addresses of a
                                                   // transposed read's lane group hit distinct banks
  static constexpr int KH = 0;                     // Kw hi [C][RLD]
  static constexpr int KL = KH + kCs * RLD * 2;    // Kw lo
  static constexpr int VR = KL + kCs * RLD * 2;    // V
  static constexpr int TOTAL = VR + kCs * RLD * 2;
};

struct ScalarRegs {
  uint4 k0, k1, v0, v1;
  float a;  // gate of token `lane` of the chunk
};

template <int DP>
__global__ __launch_bounds__(4 * DP) void build_scalar_pipe_kernel(BuildArgs a) {
  using L = ScalarLds<DP>;
  constexpr int C = kCs, NTH = 4 * DP, NW = NTH / 64, RLD = L::RLD;
  constexpr int NTC = DP / 32, TILES = NTC * NTC, TPW = (TILES + NW - 1) / NW;
  constexpr int GPR = DP / 8;  // threads per token row
  static_assert((C / 2) * GPR == NTH, "two tokens x 8 channels per thread");
  static_assert(NTC % TPW == 0, "the tiles of a wave share one row of tiles");
  __shared__ __attribute__((aligned(16))) char smem[2 * L::TOTAL];

  const Unit u = unit_of(a);
  const int H = a.heads, dk = a.dk, dv = a.dv;
  const int sk = H * dk, sv = H * dv;
  const __bf16* kbase = static_cast<const __bf16*>(a.k) + row0(a, u, dk);
  const __bf16* vbase = static_cast<const __bf16*>(a.v) + row0(a, u, dv);
  const float* abase = a.alpha + row0(a, u, 1);

  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const bool has_tiles = wave * TPW < TILES;
  const int mt = (wave * TPW) / NTC, nt0 = (wave * TPW) % NTC;

  f32x16 S[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) S[k] = zero16();
  float lam = 0.f, gnext = 1.f;
  ScalarRegs regs[2];

  // Tokens past the end of the segment read its last token (a valid
  // address) and get weight 0; channels past dk / dv read the last channels
  // and only feed rows / columns of S that are not written.
  auto load = [&](auto SET, int ci) __attribute__((always_inline)) {
    ScalarRegs& st = regs[decltype(SET)::value];
    const int tid = opaque_i(threadIdx.x), lane = tid & 63;
    const int t0 = 2 * (tid / GPR), i0 = 8 * (tid % GPR);
    const int len = chunk_len(u, ci);
    const unsigned ta = unsigned(min(t0, len - 1)), tb = unsigned(min(t0 + 1, len - 1));
    const unsigned ik = unsigned(min(i0, dk - 8)), iv = unsigned(min(i0, dv - 8));
    const int64_t off = int64_t(ci) * C;
    const char* kc = reinterpret_cast<const char*>(kbase + off * sk);
    const char* vc = reinterpret_cast<const char*>(vbase + off * sv);
    const char* ac = reinterpret_cast<const char*>(abase + off * H);
    st.k0 = *reinterpret_cast<const uint4*>(kc + (ta * unsigned(sk) + ik) * 2u);
    st.k1 = *reinterpret_cast<const uint4*>(kc + (tb * unsigned(sk) + ik) * 2u);
    st.v0 = *reinterpret_cast<const uint4*>(vc + (ta * unsigned(sv) + iv) * 2u);
    st.v1 = *reinterpret_cast<const uint4*>(vc + (tb * unsigned(sv) + iv) * 2u);
    st.a = *reinterpret_cast<const float*>(ac + unsigned(min(lane, len - 1)) * unsigned(H) * 4u);
  };

  auto stage_t = [&](auto TAIL, const ScalarRegs& st, int ci, char* sb) __attribute__((always_inline)) {
    constexpr bool tail = decltype(TAIL)::value;
    __bf16* Kh = reinterpret_cast<__bf16*>(sb + L::KH);
    __bf16* Kl = reinterpret_cast<__bf16*>(sb + L::KL);
    __bf16* Vr = reinterpret_cast<__bf16*>(sb + L::VR);
    const int tid = opaque_i(threadIdx.x), lane = tid & 63;
    const int t0 = 2 * (tid / GPR), i0 = 8 * (tid % GPR);
    const int len = chunk_len(u, ci);
    const bool ok = !tail || lane < len;
    const float incl = wave_inclusive_scan(ok ? log2_gate(st.a) : 0.f);
    const float tot =
        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
    const float wt = ok ? exp2_w(tot - incl) : 0.f;  // product of the later gates of the chunk
    const float w0 = __shfl(wt, t0, 64), w1 = __shfl(wt, t0 + 1, 64);
    lam += tot;
    gnext = exp2_w(tot);
    float x0[8], x1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x0[j] = w0 * bf_at(st.k0, j);
      x1[j] = w1 * bf_at(st.k1, j);
    }
    bf16x8 h0, l0, h1, l1;
    split8(x0, h0, l0);
    split8(x1, h1, l1);
    *reinterpret_cast<bf16x8*>(Kh + t0 * RLD + i0) = h0;
    *reinterpret_cast<bf16x8*>(Kl + t0 * RLD + i0) = l0;
    *reinterpret_cast<bf16x8*>(Kh + (t0 + 1) * RLD + i0) = h1;
    *reinterpret_cast<bf16x8*>(Kl + (t0 + 1) * RLD + i0) = l1;
    *reinterpret_cast<uint4*>(Vr + t0 * RLD + i0) = st.v0;
    *reinterpret_cast<uint4*>(Vr + (t0 + 1) * RLD + i0) = st.v1;
  };
  auto stage = [&](auto SET, int ci, int buf) __attribute__((always_inline)) {
    char* sb = smem + buf * L::TOTAL;
    if (chunk_len(u, ci) == C)
      stage_t(std::false_type(), regs[decltype(SET)::value], ci, sb);
    else
      stage_t(std::true_type(), regs[decltype(SET)::value], ci, sb);
  };

  struct Frags {
    bf16x8 ah[C / 16], al[C / 16], vb[TPW][C / 16];
    float g;
  };
  auto frags = [&](int, int buf) __attribute__((always_inline)) {
    Frags fr;
    fr.g = gnext;  // decay of the chunk being contracted (staged one step ago)
    if (has_tiles) {
      const char* sb = smem + buf * L::TOTAL;
      const __bf16* Kh = reinterpret_cast<const __bf16*>(sb + L::KH);
      const __bf16* Kl = reinterpret_cast<const __bf16*>(sb + L::KL);
      const __bf16* Vr = reinterpret_cast<const __bf16*>(sb + L::VR);
      const int lane = opaque_i(threadIdx.x) & 63;
      // lane 4j + q of a 16-lane group addresses token row r0 + j, columns c0 + 4q
      const int rsub = (lane & 15) >> 2, csub = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) {
        const int r0 = 16 * ks + 8 * (lane >> 5) + rsub;
        const int ca = r0 * RLD + mt * 32 + csub;
        fr.ah[ks] = tr_bf8(Kh + ca, Kh + ca + 4 * RLD);
        fr.al[ks] = tr_bf8(Kl + ca, Kl + ca + 4 * RLD);
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
          const int cv = r0 * RLD + (nt0 + k) * 32 + csub;
          fr.vb[k][ks] = tr_bf8(Vr + cv, Vr + cv + 4 * RLD);
        }
      }
    }
    return fr;
  };
  auto contract = [&](const Frags& fr, int) __attribute__((always_inline)) {
    if (!has_tiles) return;
#pragma unroll
    for (int k = 0; k < TPW; ++k) S[k] *= fr.g;
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks)
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        S[k] = mfma32(fr.al[ks], fr.vb[k][ks], S[k]);
        S[k] = mfma32(fr.ah[ks], fr.vb[k][ks], S[k]);
      }
  };

  run_pipeline(u.n_chunks, load, stage, frags, contract);

  if (has_tiles) write_tiles<TPW>(S, a.S0 + u.unit * int64_t(dk) * dv, mt, nt0, dk, dv);
  if (threadIdx.x == 0) a.log_scale[u.unit] = lam * kLn2;
}

// ============================================================ diagonal gates
//
// Thread mapping: a wave covers PL lanes x 4 channels of a token row and RW
// rows of 4 consecutive tokens (lane = PL * r + p: tokens 4r .. 4r+3 of the
// wave's block, channels 4p .. 4p+3 of its channel part); the waves split
// the head's channels into CP parts and the chunk into TG blocks of 4 * RW
// tokens.  Per channel, the log2 gates are summed over a lane's 4 tokens,
// then over the later rows of the block by ds_bpermute; a lane's weights are
// one exp2 of the sum over later rows times its own later gates.  Kw^T (hi,
// lo) and V^T go to LDS as channel rows (8 bytes per channel and lane); the
// block decays go to a small table that the contraction applies to S
// between the blocks.
template <int DP>
struct DiagShape {
  static constexpr int PL = DP / 4 < 16 ? DP / 4 : 16;  // lanes per token row
  static constexpr int RW = 64 / PL;                    // token quads per wave
  static constexpr int CP = DP / (4 * PL);              // channel parts
  static constexpr int NW = DP / 16;                    // waves
  static constexpr int TG = NW / CP;                    // token blocks per chunk
  static constexpr int BT = 4 * RW;                     // tokens per block
  static_assert(TG * BT == kCs, "the blocks cover the chunk");
  static_assert(BT % 16 == 0, "a block is a whole number of MFMA K-steps");
};

template <int DP>
struct DiagLds {
  static constexpr int KT = kCs + 8;                 // bf16 row stride of the channel rows
  static constexpr int KH = 0;                       // Kw^T hi [DP][KT]
  static constexpr int KL = KH + DP * KT * 2;        // Kw^T lo
  static constexpr int VT = KL + DP * KT * 2;        // V^T
  static constexpr int GM = VT + DP * KT * 2;        // block decays [TG][DP]
  static constexpr int TOTAL = GM + DiagShape<DP>::TG * DP * 4;
};

struct DiagRegs {
  uint2 k[4], v[4];
  float4 a[4];
};

template <int DP>
__global__ __launch_bounds__(4 * DP) void build_diag_pipe_kernel(BuildArgs a) {
  using L = DiagLds<DP>;
  using Sh = DiagShape<DP>;
  constexpr int C = kCs, NTH = 4 * DP, NW = NTH / 64, KT = L::KT;
  constexpr int PL = Sh::PL, RW = Sh::RW, CP = Sh::CP, TG = Sh::TG, BT = Sh::BT;
  constexpr int NTC = DP / 32, TILES = NTC * NTC, TPW = (TILES + NW - 1) / NW;
  static_assert(NW == Sh::NW, "wave count");
  static_assert(NTC % TPW == 0, "the tiles of a wave share one row of tiles");
  static_assert(TG * DP * 4 <= 2 * DiagLds<DP>::TOTAL, "lambda table fits the LDS buffers");
  __shared__ __attribute__((aligned(16))) char smem[2 * L::TOTAL];

  const Unit u = unit_of(a);
  const int H = a.heads, dk = a.dk, dv = a.dv;
  const int sk = H * dk, sv = H * dv;
  const __bf16* kbase = static_cast<const __bf16*>(a.k) + row0(a, u, dk);
  const __bf16* vbase = static_cast<const __bf16*>(a.v) + row0(a, u, dv);
  const float* abase = a.alpha + row0(a, u, dk);

  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const bool has_tiles = wave * TPW < TILES;
  const int mt = (wave * TPW) / NTC, nt0 = (wave * TPW) % NTC;
  const int part = wave % CP, tg = wave / CP;

  f32x16 S[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) S[k] = zero16();
  float lam[4] = {0.f, 0.f, 0.f, 0.f};
  DiagRegs regs[2];

  // lane -> (row r, channels c0 .. c0+3, first token t4 of the lane in the chunk)
  auto lane_map = [&](int& r, int& c0, int& t4) __attribute__((always_inline)) {
    const int lane = opaque_i(threadIdx.x) & 63;
    const int p = lane % PL;
    r = lane / PL;
    c0 = 4 * (PL * part + p);
    t4 = BT * tg + 4 * r;
  };

  auto load = [&](auto SET, int ci) __attribute__((always_inline)) {
    DiagRegs& st = regs[decltype(SET)::value];
    int r, c0, t4;
    lane_map(r, c0, t4);
    const int len = chunk_len(u, ci);
    const unsigned ck = unsigned(min(c0, dk - 4)), cv = unsigned(min(c0, dv - 4));
    const int64_t off = int64_t(ci) * C;
    const char* kc = reinterpret_cast<const char*>(kbase + off * sk);
    const char* vc = reinterpret_cast<const char*>(vbase + off * sv);
    const char* ac = reinterpret_cast<const char*>(abase + off * sk);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned t = unsigned(min(t4 + q, len - 1));
      st.k[q] = *reinterpret_cast<const uint2*>(kc + (t * unsigned(sk) + ck) * 2u);
      st.v[q] = *reinterpret_cast<const uint2*>(vc + (t * unsigned(sv) + cv) * 2u);
      st.a[q] = *reinterpret_cast<const float4*>(ac + (t * unsigned(sk) + ck) * 4u);
    }
  };

  auto stage_t = [&](auto TAIL, const DiagRegs& st, int ci, char* sb) __attribute__((always_inline)) {
    constexpr bool tail = decltype(TAIL)::value;
    __bf16* Kh = reinterpret_cast<__bf16*>(sb + L::KH);
    __bf16* Kl = reinterpret_cast<__bf16*>(sb + L::KL);
    __bf16* Vt = reinterpret_cast<__bf16*>(sb + L::VT);
    float* gm = reinterpret_cast<float*>(sb + L::GM);
    int r, c0, t4;
    lane_map(r, c0, t4);
    const int lane = opaque_i(threadIdx.x) & 63;
    const int len = chunk_len(u, ci);
    float gv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float gg[4], l[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = !tail || t4 + q < len;
        const float x = st.a[q][j];
        gg[q] = ok ? x : 1.f;
        l[q] = ok ? log2_gate(x) : 0.f;
      }
      const float quad = (l[0] + l[1]) + (l[2] + l[3]);
      // sum over the rows r' >= r of the block (same lane position)
      float incl = quad;
#pragma unroll
      for (int s = 1; s < RW; s <<= 1) {
        const float o = __shfl(incl, lane + s * PL, 64);
        incl += (r + s < RW) ? o : 0.f;
      }
      const float base = exp2_w(incl - quad);  // product of the gates of later rows
      float w[4];
      w[3] = base;
      w[2] = base * gg[3];
      w[1] = w[2] * gg[2];
      w[0] = w[1] * gg[1];
      if (tail) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (t4 + q >= len) w[q] = 0.f;
      }
      lam[j] += incl;  // the block total on rows r == 0, which hold lambda
      gv[j] = exp2_w(incl);
      // channel c0 + j: Kw hi / lo and V of tokens t4 .. t4+3
      float kw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const unsigned word = (j < 2) ? st.k[q].x : st.k[q].y;
        kw[q] = w[q] * ((j & 1) ? bf_hi(word) : bf_lo(word));
      }
      unsigned h01, l01, h23, l23;
      split2(kw[0], kw[1], h01, l01);
      split2(kw[2], kw[3], h23, l23);
      const int at = (c0 + j) * KT + t4;
      *reinterpret_cast<uint2*>(Kh + at) = make_uint2(h01, h23);
      *reinterpret_cast<uint2*>(Kl + at) = make_uint2(l01, l23);
      const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
      const unsigned v01 = (j < 2) ? __builtin_amdgcn_perm(st.v[1].x, st.v[0].x, sel)
                                   : __builtin_amdgcn_perm(st.v[1].y, st.v[0].y, sel);
      const unsigned v23 = (j < 2) ? __builtin_amdgcn_perm(st.v[3].x, st.v[2].x, sel)
                                   : __builtin_amdgcn_perm(st.v[3].y, st.v[2].y, sel);
      *reinterpret_cast<uint2*>(Vt + at) = make_uint2(v01, v23);
    }
    if (r == 0) *reinterpret_cast<float4*>(gm + tg * DP + c0) = make_float4(gv[0], gv[1], gv[2], gv[3]);
  };
  auto stage = [&](auto SET, int ci, int buf) __attribute__((always_inline)) {
    char* sb = smem + buf * L::TOTAL;
    if (chunk_len(u, ci) == C)
      stage_t(std::false_type(), regs[decltype(SET)::value], ci, sb);
    else
      stage_t(std::true_type(), regs[decltype(SET)::value], ci, sb);
  };

  struct Frags {
    bf16x8 ah[C / 16], al[C / 16], vb[TPW][C / 16];
    int buf;
  };
  auto frags = [&](int, int buf) __attribute__((always_inline)) {
    Frags fr;
    fr.buf = buf;
    if (has_tiles) {
      const char* sb = smem + buf * L::TOTAL;
      const __bf16* Kh = reinterpret_cast<const __bf16*>(sb + L::KH);
      const __bf16* Kl = reinterpret_cast<const __bf16*>(sb + L::KL);
      const __bf16* Vt = reinterpret_cast<const __bf16*>(sb + L::VT);
      const int lane = opaque_i(threadIdx.x) & 63;
      const int g = lane >> 5, cl = lane & 31;
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) {
        const int ka = (mt * 32 + cl) * KT + 16 * ks + 8 * g;
        fr.ah[ks] = lds_load8(Kh + ka);
        fr.al[ks] = lds_load8(Kl + ka);
#pragma unroll
        for (int k = 0; k < TPW; ++k)
          fr.vb[k][ks] = lds_load8(Vt + ((nt0 + k) * 32 + cl) * KT + 16 * ks + 8 * g);
      }
    }
    return fr;
  };
  // per block: S <- gamma_block (.) S (rows), then the block's K-steps
  auto contract = [&](const Frags& fr, int) __attribute__((always_inline)) {
    if (!has_tiles) return;
    const float* gm = reinterpret_cast<const float*>(smem + fr.buf * L::TOTAL + L::GM);
    const int g = (opaque_i(threadIdx.x) & 63) >> 5;
#pragma unroll
    for (int bi = 0; bi < TG; ++bi) {
      float f[16];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const float4 x = *reinterpret_cast<const float4*>(gm + bi * DP + mt * 32 + 8 * qq + 4 * g);
        f[4 * qq] = x.x; f[4 * qq + 1] = x.y; f[4 * qq + 2] = x.z; f[4 * qq + 3] = x.w;
      }
#pragma unroll
      for (int k = 0; k < TPW; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[k][r] *= f[r];
#pragma unroll
      for (int ks = bi * (BT / 16); ks < (bi + 1) * (BT / 16); ++ks)
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
          S[k] = mfma32(fr.al[ks], fr.vb[k][ks], S[k]);
          S[k] = mfma32(fr.ah[ks], fr.vb[k][ks], S[k]);
        }
    }
  };

  run_pipeline(u.n_chunks, load, stage, frags, contract);

  if (has_tiles) write_tiles<TPW>(S, a.S0 + u.unit * int64_t(dk) * dv, mt, nt0, dk, dv);
  // lambda: rows r == 0 hold their block's totals; the TG blocks of each
  // channel are summed through LDS (free after the pipeline's last barrier)
  int r, c0, t4;
  lane_map(r, c0, t4);
  float* lb = reinterpret_cast<float*>(smem);
  if (r == 0) *reinterpret_cast<float4*>(lb + tg * DP + c0) = make_float4(lam[0], lam[1], lam[2], lam[3]);
  __syncthreads();
  if (r == 0 && tg == 0 && c0 < dk) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 0.f;
#pragma unroll
      for (int bi = 0; bi < TG; ++bi) s += lb[bi * DP + c0 + j];
      a.log_scale[u.unit * dk + c0 + j] = s * kLn2;
    }
  }
}

template <int DP, bool DIAG>
hipError_t launch_sdp_t(const BuildArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_seg) * a.batch * a.heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (DIAG)
    hipLaunchKernelGGL((build_diag_pipe_kernel<DP>), dim3(unsigned(blocks)), dim3(4 * DP), 0, s, a);
  else
    hipLaunchKernelGGL((build_scalar_pipe_kernel<DP>), dim3(unsigned(blocks)), dim3(4 * DP), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_sd_pipe(const BuildArgs& a, hipStream_t s) {
  const int d = a.dk > a.dv ? a.dk : a.dv;
  const bool diag = a.form == kDiag;
  if (d <= 32) return diag ? launch_sdp_t<32, true>(a, s) : launch_sdp_t<32, false>(a, s);
  if (d <= 64) return diag ? launch_sdp_t<64, true>(a, s) : launch_sdp_t<64, false>(a, s);
  return diag ? launch_sdp_t<128, true>(a, s) : launch_sdp_t<128, false>(a, s);
}

}  // namespace pic
