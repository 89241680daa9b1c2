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
#ifndef SD_DEPTH_SCALAR
#define SD_DEPTH_SCALAR 2
#endif
#ifndef SD_DEPTH_DIAG
#define SD_DEPTH_DIAG 2
#endif

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
  u.seg = seg_in_order(a, int(build_unit(a, blockIdx.x) / BH));
  const int bh = int(build_unit(a, blockIdx.x) % BH);
  u.b = bh / H;
  u.h = bh % H;
  const int64_t t_begin = seg_offset(a, u.seg);
  u.n_tok = seg_offset(a, u.seg + 1) - t_begin;
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
  return ((int64_t(u.b) * a.n_tokens + seg_offset(a, u.seg)) * a.heads + u.h) * d;
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<I + 1, N>(f);
  }
}

// Runs the pipeline with DEPTH register sets: load(set, chunk) issues the
// loads of a chunk into register set `set` (a std::integral_constant; chunk
// j lives in set j % DEPTH), stage(set, chunk, buffer) stages it,
// frags(chunk, buffer) reads a chunk's operand fragments into a value that
// contract(value, chunk) consumes.  Step j: frags of chunk j (buffer j & 1),
// stage chunk j+1 (buffer (j+1) & 1), load chunk j+1+DEPTH into the set just
// staged, contract chunk j, barrier.
template <int DEPTH, class LoadF, class StageF, class FragF, class ContractF>
__device__ __forceinline__ void run_pipeline(int n_chunks, LoadF&& load, StageF&& stage,
                                             FragF&& frags, ContractF&& contract) {
  if (n_chunks <= 0) return;
  const int last = n_chunks - 1;
  static_for<0, DEPTH>([&](auto S) { load(S, min(decltype(S)::value, last)); });
  stage(std::integral_constant<int, 0>(), 0, 0);
  load(std::integral_constant<int, 0>(), min(DEPTH, last));
  __syncthreads();
  auto step = [&](auto D, int cj) __attribute__((always_inline)) {
    using DN = std::integral_constant<int, (decltype(D)::value + 1) % DEPTH>;
    auto fr = frags(cj, cj & 1);
    if (cj + 1 < n_chunks) stage(DN(), cj + 1, (cj + 1) & 1);
    load(DN(), min(cj + 1 + DEPTH, last));
    contract(fr, cj);
    __syncthreads();
  };
  int cj = 0;
#pragma unroll 1
  for (; cj + DEPTH <= n_chunks; cj += DEPTH)
    static_for<0, DEPTH>([&](auto D) { step(D, cj + decltype(D)::value); });
  static_for<0, DEPTH - 1>([&](auto D) {
    if (cj + decltype(D)::value < n_chunks) step(D, cj + decltype(D)::value);
  });
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
// Producer and consumer waves.  DP/32 consumer waves each hold one row of
// 32x32 tiles of S (all DP/32 column tiles) in MFMA registers for the whole
// segment; they read operand fragments and issue MFMAs.  Consumer wave 0
// also turns the gates into the chunk's token weights, two chunks ahead
// (a 64-lane scan, lane = token; it has the time, the MFMA waves wait on
// the staging), and leaves them in a small LDS table.  As many producer
// waves load and stage: producer thread (R, i0) takes the four consecutive
// tokens 4R .. 4R+3 of the chunk, channels i0 .. i0+7; load instruction p
// reads token 4R+p of every R, i.e. whole token rows.  A producer reads its
// four weights with one broadcast LDS load, stages Kw (hi, lo) and V
// token-major, and issues the loads of a later chunk into each token's
// registers as soon as that token is staged.  The consumers read their
// transposed operand fragments with ds_read_b64_tr_b16.
//
// Step j (one barrier): consumers contract chunk j (buffer j & 1, table
// j % 3); consumer wave 0 writes the weights of chunk j+2 (table (j+2) % 3);
// producers stage chunk j+1 (buffer (j+1) & 1, weights from table
// (j+1) % 3) and load chunk j+3.
#ifndef SD_SCALAR_T
#define SD_SCALAR_T 0
#endif
// element offset of tokens t .. of channel row `row` (t a multiple of 4); the
// 16-byte chunks of a row are XOR-swizzled by the row's 8-row group
template <int KT>
__device__ __forceinline__ int ch_at(int row, int t) {
  return row * KT + 8 * ((t >> 3) ^ ((row >> 3) & 7)) + (t & 7);
}
template <int DP>
struct ScalarLds {
  static constexpr bool T = SD_SCALAR_T;     // channel rows (else token rows)
  static constexpr int KT = kCs + 8;         // channel rows: bf16 stride
  static constexpr int RLD = DP + 16;        // token rows: bf16 stride; the 16 addresses of a
                                             // transposed read's lane group hit distinct banks
  static constexpr int TILE = T ? DP * KT * 2 : kCs * RLD * 2;
  static constexpr int KH = 0;               // Kw hi [C][RLD]
  static constexpr int KL = KH + TILE;       // Kw lo
  static constexpr int VR = KL + TILE;       // V
  static constexpr int TOTAL = VR + TILE;    // one of two buffers
  static constexpr int WT = 2 * TOTAL;       // weight tables [3][C + 4]
  static constexpr int ALL = WT + 3 * (kCs + 4) * 4;
};

template <int DP>
__global__ __launch_bounds__(4 * DP) void build_scalar_pipe_kernel(BuildArgs a) {
  using L = ScalarLds<DP>;
  constexpr int C = kCs, RLD = L::RLD;
  constexpr int NC = DP / 32;     // consumer waves = rows of tiles
  constexpr int GPR = DP / 8;     // producer threads per token row
  static_assert(NC * 64 / GPR * 4 == C, "the producers cover the chunk");
  static_assert(2 * NC * 64 == 4 * DP, "block size");
  __shared__ __attribute__((aligned(16))) char smem[L::ALL];
  float* wtab = reinterpret_cast<float*>(smem + L::WT);

  const Unit u = unit_of(a);
  const int H = a.heads, dk = a.dk, dv = a.dv;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int n = u.n_chunks, last = n - 1;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  if (wave < NC) {
    // ---------------- consumers
    const int mt = wave, lane = threadIdx.x & 63;
    const bool scan_wave = wave == 0;
    // the scan wave (products plus the weights two chunks ahead) is the
    // busiest of the block: it issues ahead of the producer on its SIMD
    if (scan_wave) __builtin_amdgcn_s_setprio(1);
    const float* abase = a.alpha + row0(a, u, 1);
    float areg[2] = {1.f, 1.f}, lam = 0.f;
    // gate of token `lane` of chunk ci (clamped inside the segment)
    auto load_gate = [&](auto SET, int ci) __attribute__((always_inline)) {
      const int len = chunk_len(u, ci);
      const char* ac = reinterpret_cast<const char*>(abase + int64_t(ci) * C * H);
      areg[decltype(SET)::value] =
          *reinterpret_cast<const float*>(ac + unsigned(min(lane, len - 1)) * unsigned(H) * 4u);
    };
    // weights of chunk ci into table ci & 1: w_t = product of the gates after
    // t in the chunk (0 past its end), then the chunk's decay
    // Lazy decay: the consumers hold S' = S / 2^G, G the log2 decay since a
    // reference point, so a chunk needs no rescaling of S: its token weights
    // become 2^(-G_prev - prefix_t) (prefix_t: log2 gates of the chunk through
    // token t).  When G_prev + (the chunk's decay) would drop below -kLazy,
    // the reference moves to the chunk's end: S' is scaled once by
    // 2^(G_prev + decay) before the chunk and the weights are the plain
    // 2^(decay - prefix_t) <= 1.  Weights stay below 2^kLazy.
    constexpr float kLazy = 32.f;
    float Gref = 0.f;
    // weights of chunk ci (gates from register set SET) into table `tab`:
    // [0, C) token weights (0 past the chunk's end), [C] the factor to scale
    // S' by before the chunk, [C+1] G after the chunk.  Chunks past the last
    // (ci >= n) are computed but leave G and lambda unchanged.
    auto weights = [&](auto SET, int ci, int tab) __attribute__((always_inline)) {
      const bool real = ci < n;
      ci = min(ci, last);
      const int len = chunk_len(u, ci);
      const bool ok = lane < len;
      const float incl = wave_inclusive_scan(ok ? log2_gate(areg[decltype(SET)::value]) : 0.f);
      const float tot =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
      const bool move = Gref + tot < -kLazy;
      const float e0 = move ? tot : -Gref;  // weight exponent = e0 - prefix_t
      float* wt = wtab + tab * (C + 4);
      wt[lane] = ok ? exp2_w(e0 - incl) : 0.f;
      const float Gnew = move ? 0.f : Gref + tot;
      if (lane == 0) {
        wt[C] = move ? exp2_w(Gref + tot) : 1.f;
        wt[C + 1] = Gnew;
      }
      if (real) {
        Gref = Gnew;
        lam += tot;
      }
    };

    f32x16 S[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) S[k] = zero16();
    float Gs = 0.f;  // S = 2^Gs S' after the chunks contracted so far
    if (n > 0) {
      // every consumer wave issues the gate loads (a load inside the scan
      // wave's branch makes the compiler wait for all of them at the join);
      // only the scan wave uses them
      load_gate(I0(), 0);
      load_gate(I1(), min(1, last));
      if (scan_wave) weights(I0(), 0, 0);
      load_gate(I0(), min(2, last));
      if (scan_wave) weights(I1(), 1, 1);
      load_gate(I1(), min(3, last));
      __syncthreads();  // weights of chunks 0 and 1
      __syncthreads();  // chunk 0 staged
      auto step = [&](auto D, int cj) __attribute__((always_inline)) {
        const char* sb = smem + (cj & 1) * L::TOTAL;
        const __bf16* Kh = reinterpret_cast<const __bf16*>(sb + L::KH);
        const __bf16* Kl = reinterpret_cast<const __bf16*>(sb + L::KL);
        const __bf16* Vr = reinterpret_cast<const __bf16*>(sb + L::VR);
        const float pre = wtab[(cj % 3) * (C + 4) + C];
        Gs = wtab[(cj % 3) * (C + 4) + C + 1];
        // lane 4j + q of a 16-lane group addresses token row r0 + j, columns c0 + 4q
        const int l = opaque_i(threadIdx.x) & 63;
        const int rsub = (l & 15) >> 2, csub = 16 * ((l >> 4) & 1) + 4 * (l & 3);
        bf16x8 ah[C / 16], al[C / 16], vb[NC][C / 16];
        if (L::T) {
          const int cl = l & 31, t8 = 8 * (l >> 5);
#pragma unroll
          for (int ks = 0; ks < C / 16; ++ks) {
            const int ka = ch_at<L::KT>(mt * 32 + cl, 16 * ks + t8);
            ah[ks] = lds_load8(Kh + ka);
            al[ks] = lds_load8(Kl + ka);
#pragma unroll
            for (int k = 0; k < NC; ++k) vb[k][ks] = lds_load8(Vr + ch_at<L::KT>(k * 32 + cl, 16 * ks + t8));
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < C / 16; ++ks) {
            const int r0 = 16 * ks + 8 * (l >> 5) + rsub;
            const int ca = r0 * RLD + mt * 32 + csub;
            ah[ks] = tr_bf8(Kh + ca, Kh + ca + 4 * RLD);
            al[ks] = tr_bf8(Kl + ca, Kl + ca + 4 * RLD);
#pragma unroll
            for (int k = 0; k < NC; ++k) {
              const int cv = r0 * RLD + k * 32 + csub;
              vb[k][ks] = tr_bf8(Vr + cv, Vr + cv + 4 * RLD);
            }
          }
        }
        if (__builtin_amdgcn_readfirstlane(__float_as_int(pre)) != __float_as_int(1.f)) {
#pragma unroll
          for (int k = 0; k < NC; ++k) S[k] *= pre;
        }
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks)
#pragma unroll
          for (int k = 0; k < NC; ++k) {
            S[k] = mfma32(al[ks], vb[k][ks], S[k]);
            S[k] = mfma32(ah[ks], vb[k][ks], S[k]);
          }
        if (scan_wave) weights(D, cj + 2, (cj + 2) % 3);
        load_gate(D, min(cj + 4, last));
        __syncthreads();
      };
      int cj = 0;
#pragma unroll 1
      for (; cj + 2 <= n; cj += 2) {
        step(I0(), cj);
        step(I1(), cj + 1);
      }
      if (cj < n) step(I0(), cj);
    }
    const float fin = exp2_w(Gs);
#pragma unroll
    for (int k = 0; k < NC; ++k) S[k] *= fin;
    write_tiles<NC>(S, a.S0 + u.unit * int64_t(dk) * dv, mt, 0, dk, dv);
    if (threadIdx.x == 0) a.log_scale[u.unit] = lam * kLn2;
    return;
  }

  // ---------------- producers (issue ahead of the consumer waves 1..3 that
  // share their SIMDs, like the scan wave)
  __builtin_amdgcn_s_setprio(1);
  const int ptid = int(threadIdx.x) - NC * 64;
  const int R = ptid / GPR, i0 = 8 * (ptid % GPR);
  const int sk = H * dk, sv = H * dv;
  const unsigned ik = unsigned(min(i0, dk - 8)), iv = unsigned(min(i0, dv - 8));
  const __bf16* kbase = static_cast<const __bf16*>(a.k) + row0(a, u, dk);
  const __bf16* vbase = static_cast<const __bf16*>(a.v) + row0(a, u, dv);
  struct Set {
    uint4 k[4], v[4];  // tokens 4R+p of a chunk
  };
  Set regs[2];

  // Tokens past the end of the segment read its last token (a valid
  // address; their weight is 0); channels past dk / dv read the last
  // channels and only feed rows / columns of S that are not written.
  auto load_tok = [&](auto SET, int ci, auto P) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    const int len = chunk_len(u, ci);
    const unsigned t = unsigned(min(4 * R + p, len - 1));
    const int64_t off = int64_t(ci) * C;
    const char* kc = reinterpret_cast<const char*>(kbase + off * sk);
    const char* vc = reinterpret_cast<const char*>(vbase + off * sv);
    Set& rs = regs[decltype(SET)::value];
    rs.k[p] = *reinterpret_cast<const uint4*>(kc + (t * unsigned(sk) + ik) * 2u);
    rs.v[p] = *reinterpret_cast<const uint4*>(vc + (t * unsigned(sv) + iv) * 2u);
  };
  // stage chunk cs from register set SET into buffer cs & 1, reloading each
  // token's registers with chunk cl as soon as the token is staged
  auto stage = [&](auto SET, int cs, int cl) __attribute__((always_inline)) {
    constexpr int st = decltype(SET)::value;
    char* sb = smem + (cs & 1) * L::TOTAL;
    __bf16* Kh = reinterpret_cast<__bf16*>(sb + L::KH);
    __bf16* Kl = reinterpret_cast<__bf16*>(sb + L::KL);
    __bf16* Vr = reinterpret_cast<__bf16*>(sb + L::VR);
    const float4 w4 = *reinterpret_cast<const float4*>(wtab + (cs % 3) * (C + 4) + 4 * R);
    if (L::T) {
      const Set& rs = regs[st];
      const float w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // channel i0 + j, tokens 4R .. 4R+3
        float x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = w[q] * bf_at(rs.k[q], j);
        unsigned h01, l01, h23, l23;
        split2(x[0], x[1], h01, l01);
        split2(x[2], x[3], h23, l23);
        const int at = ch_at<L::KT>(i0 + j, 4 * R);
        *reinterpret_cast<uint2*>(Kh + at) = make_uint2(h01, h23);
        *reinterpret_cast<uint2*>(Kl + at) = make_uint2(l01, l23);
        const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
        auto dw = [&](const uint4& v) { return (j < 2) ? v.x : (j < 4) ? v.y : (j < 6) ? v.z : v.w; };
        const unsigned v01 = __builtin_amdgcn_perm(dw(rs.v[1]), dw(rs.v[0]), sel);
        const unsigned v23 = __builtin_amdgcn_perm(dw(rs.v[3]), dw(rs.v[2]), sel);
        *reinterpret_cast<uint2*>(Vr + at) = make_uint2(v01, v23);
      }
      static_for<0, 4>([&](auto P) __attribute__((always_inline)) { load_tok(SET, cl, P); });
      return;
    }
    static_for<0, 4>([&](auto P) __attribute__((always_inline)) {
      constexpr int p = decltype(P)::value;
      const int t = 4 * R + p;
      const float wp = p == 0 ? w4.x : p == 1 ? w4.y : p == 2 ? w4.z : w4.w;
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = wp * bf_at(regs[st].k[p], j);
      bf16x8 hi, lo;
      split8(x, hi, lo);
      *reinterpret_cast<bf16x8*>(Kh + t * RLD + i0) = hi;
      *reinterpret_cast<bf16x8*>(Kl + t * RLD + i0) = lo;
      *reinterpret_cast<uint4*>(Vr + t * RLD + i0) = regs[st].v[p];
      load_tok(SET, cl, P);
    });
  };
  auto load_all = [&](auto SET, int ci) __attribute__((always_inline)) {
    static_for<0, 4>([&](auto P) __attribute__((always_inline)) { load_tok(SET, ci, P); });
  };

  if (n > 0) {
    load_all(I0(), 0);
    load_all(I1(), min(1, last));
    __syncthreads();  // weights of chunks 0 and 1
    stage(I0(), 0, min(2, last));
    __syncthreads();  // chunk 0 staged
    // The last step stages the chunk past the end (weights of a clamped
    // chunk, registers of the last one) into the buffer nobody reads any
    // more: every step runs the same code, so the register sets are never
    // merged at a join (the copies there would wait for every load in flight).
    auto step = [&](auto D, int cj) __attribute__((always_inline)) {
      using DN = std::integral_constant<int, (decltype(D)::value + 1) & 1>;
      stage(DN(), cj + 1, min(cj + 3, last));
      __syncthreads();
    };
    int cj = 0;
#pragma unroll 1
    for (; cj + 2 <= n; cj += 2) {
      step(I0(), cj);
      step(I1(), cj + 1);
    }
    if (cj < n) step(I0(), cj);
  }
}

// ============================================================ diagonal gates
//
// Producer and consumer waves, as for the scalar form.  DP/32 consumer waves
// each hold one row of 32x32 tiles of S and contract the chunk block by
// block, scaling S's rows by each block's decay first.  As many producer
// waves stage: a producer wave covers PL lanes x 4 channels of a token row
// and RW rows of 8 consecutive tokens (lane = PL * r + p: tokens 8r .. 8r+7
// of the wave's block, channels 4p .. 4p+3 of its channel part); the waves
// split the channels into CP parts and the chunk into TG blocks of 8 * RW
// tokens, so a channel's suffix sums of log2 alpha stay in one wave: a lane
// takes the log2 of the product of its 8 gates, then the sums over the later
// rows come by ds_bpermute.  A lane's weights are one exp2 of the sum over
// the later rows times its own later gates.  Kw^T (hi, lo) and V^T go to LDS
// as channel rows, one 16-byte store (8 tokens) per channel and array; the
// 16-byte pieces of a row are XOR-swizzled by the row's 8-row group.  The
// producers stage the gates and Kw; V is loaded and staged by the consumer
// wave of the same index with the same lane map (the producers set the pace
// of a step, the consumers are idle for half of it).  Loads: 16 lanes x 8
// bytes of k or v or 16 lanes x 16 bytes of gates per token row (whole
// 128-byte lines), nontemporal; a lane's offsets inside a chunk are fixed,
// so an address costs one add and one clamp.  Each part of a register set is
// reloaded as soon as the staging step is done with it.  Every step is one
// code path for every chunk (see stage below), with no branch around loads.
template <int DP>
struct DiagShape {
  static constexpr int NC = DP / 32;                    // consumer waves
  static constexpr int NP = DP / 32;                    // producer waves
  static constexpr int PL = DP / 4 < 16 ? DP / 4 : 16;  // lanes per token row
  static constexpr int RW = 64 / PL;                    // rows of 8 tokens per wave
  static constexpr int CP = DP / (4 * PL);              // channel parts
  static constexpr int TG = NP / CP;                    // token blocks per chunk
  static constexpr int BT = 8 * RW;                     // tokens per block
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


// Loads with the nontemporal hint: the inputs of a diagonal-gate unit (its
// own channels of k, v and the gates) are read exactly once.
typedef float ntf4 __attribute__((ext_vector_type(4)));
typedef unsigned ntu2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 nt_f4(const char* p) {
  const ntf4 t = __builtin_nontemporal_load(reinterpret_cast<const ntf4*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 nt_u2(const char* p) {
  const ntu2 t = __builtin_nontemporal_load(reinterpret_cast<const ntu2*>(p));
  return make_uint2(t.x, t.y);
}
struct DiagRegs {
  uint2 k[8];
  float4 a[8];
};

template <int DP>
__global__ __launch_bounds__(4 * DP) void build_diag_pipe_kernel(BuildArgs a) {
  using L = DiagLds<DP>;
  using Sh = DiagShape<DP>;
  constexpr int C = kCs, KT = L::KT;
  constexpr int NC = Sh::NC, PL = Sh::PL, RW = Sh::RW, CP = Sh::CP, TG = Sh::TG, BT = Sh::BT;
  static_assert((NC + Sh::NP) * 64 == 4 * DP, "block size");
  static_assert(TG * DP * 4 <= 2 * L::TOTAL, "lambda table fits the LDS buffers");
  __shared__ __attribute__((aligned(16))) char smem[2 * L::TOTAL];

  const Unit u = unit_of(a);
  const int H = a.heads, dk = a.dk, dv = a.dv;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int n = u.n_chunks, last = n - 1;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  if (wave < NC) {
    // ---------------- consumers: tiles (mt = wave, nt = 0 .. NC-1)
    const int mt = wave;
    f32x16 S[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) S[k] = zero16();
    // V: consumer wave w loads and stages the rows producer wave w would
    // (the same lane map), two chunks ahead in two register sets; the
    // consumers have the time (the producers set the pace of a step), and
    // their loads add to the bytes in flight.
    int vr, vc0, vt0;
    {
      const int lane = opaque_i(threadIdx.x) & 63;
      vr = lane / PL;
      vc0 = 4 * (PL * (wave % CP) + lane % PL);
      vt0 = BT * (wave / CP) + 8 * vr;
    }
    const int sv = H * dv;
    const __bf16* vbase = static_cast<const __bf16*>(a.v) + row0(a, u, dv);
    const unsigned rv = unsigned(sv) * 2u, cv2 = unsigned(min(vc0, dv - 4)) * 2u;
    const unsigned ov_ = unsigned(vt0) * rv + cv2;
    uint2 vreg[2][8];
    // chunks past the last read one row of the last chunk (data unused)
    auto load_v = [&](auto SET, int cq) __attribute__((always_inline)) {
      const int ci = min(cq, last);
      const char* vc = reinterpret_cast<const char*>(vbase + int64_t(ci) * C * sv);
      const unsigned lim = unsigned(cq > last ? 0 : chunk_len(u, ci) - 1) * rv + cv2;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        vreg[decltype(SET)::value][q] = nt_u2(vc + min(ov_ + unsigned(q) * rv, lim));
    };
    // V of tokens vt0 .. vt0+7 of chunk cs, channels vc0 .. vc0+3, as channel
    // rows into buffer cs & 1; zero past the end of the segment (so those
    // tokens add nothing whatever their weights)
    auto stage_v = [&](auto SET, int cs) __attribute__((always_inline)) {
      uint2(&rg)[8] = vreg[decltype(SET)::value];
      __bf16* Vt = reinterpret_cast<__bf16*>(smem + (cs & 1) * L::TOTAL + L::VT);
      const int len = chunk_len(u, cs);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const unsigned m = vt0 + q < len ? 0xffffffffu : 0u;
        rg[q].x &= m;
        rg[q].y &= m;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
        unsigned pv[4];
#pragma unroll
        for (int q = 0; q < 8; q += 2) {
          const unsigned v0 = (j < 2) ? rg[q].x : rg[q].y;
          const unsigned v1 = (j < 2) ? rg[q + 1].x : rg[q + 1].y;
          pv[q / 2] = __builtin_amdgcn_perm(v1, v0, sel);
        }
        *reinterpret_cast<uint4*>(Vt + ch_at<KT>(vc0 + j, vt0)) = make_uint4(pv[0], pv[1], pv[2], pv[3]);
      }
    };
    if (n > 0) {
      load_v(I0(), 0);
      load_v(I1(), 1);
      stage_v(I0(), 0);
      load_v(I0(), 2);
      __syncthreads();  // chunk 0 staged
      // step j: contract chunk j; stage V of chunk j+1 (set (j+1) & 1) and
      // reload that set with chunk j+3 (one code path for every step)
      auto cstep = [&](auto D, int cj) __attribute__((always_inline)) {
        using DN = std::integral_constant<int, (decltype(D)::value + 1) & 1>;
        const char* sb = smem + (cj & 1) * L::TOTAL;
        const __bf16* Kh = reinterpret_cast<const __bf16*>(sb + L::KH);
        const __bf16* Kl = reinterpret_cast<const __bf16*>(sb + L::KL);
        const __bf16* Vt = reinterpret_cast<const __bf16*>(sb + L::VT);
        const float* gm = reinterpret_cast<const float*>(sb + L::GM);
        const int l = opaque_i(threadIdx.x) & 63, g = l >> 5, cl = l & 31;
        bf16x8 ah[C / 16], al[C / 16], vb[NC][C / 16];
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
          const int ka = ch_at<KT>(mt * 32 + cl, 16 * ks + 8 * g);
          ah[ks] = lds_load8(Kh + ka);
          al[ks] = lds_load8(Kl + ka);
#pragma unroll
          for (int k = 0; k < NC; ++k) vb[k][ks] = lds_load8(Vt + ch_at<KT>(k * 32 + cl, 16 * ks + 8 * g));
        }
        stage_v(DN(), cj + 1);
        load_v(DN(), cj + 3);
#pragma unroll
        for (int bi = 0; bi < TG; ++bi) {
          float f[16];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const float4 x = *reinterpret_cast<const float4*>(gm + bi * DP + mt * 32 + 8 * qq + 4 * g);
            f[4 * qq] = x.x; f[4 * qq + 1] = x.y; f[4 * qq + 2] = x.z; f[4 * qq + 3] = x.w;
          }
#pragma unroll
          for (int k = 0; k < NC; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) S[k][r] *= f[r];
#pragma unroll
          for (int ks = bi * (BT / 16); ks < (bi + 1) * (BT / 16); ++ks)
#pragma unroll
            for (int k = 0; k < NC; ++k) {
              S[k] = mfma32(al[ks], vb[k][ks], S[k]);
              S[k] = mfma32(ah[ks], vb[k][ks], S[k]);
            }
        }
        __syncthreads();
      };
      int cj = 0;
#pragma unroll 1
      for (; cj + 2 <= n; cj += 2) {
        cstep(I0(), cj);
        cstep(I1(), cj + 1);
      }
      if (cj < n) cstep(I0(), cj);
    }
    write_tiles<NC>(S, a.S0 + u.unit * int64_t(dk) * dv, mt, 0, dk, dv);
    __syncthreads();  // lambda table
    __syncthreads();
    return;
  }

  // ---------------- producers (the critical path: they issue ahead of the
  // consumer wave that shares their SIMD)
  __builtin_amdgcn_s_setprio(1);
  const int ptid = int(threadIdx.x) - NC * 64;
  const int pw = __builtin_amdgcn_readfirstlane(ptid >> 6);
  const int part = pw % CP, tb = pw / CP;
  const int sk = H * dk;
  const __bf16* kbase = static_cast<const __bf16*>(a.k) + row0(a, u, dk);
  const float* abase = a.alpha + row0(a, u, dk);
  float lam[4] = {0.f, 0.f, 0.f, 0.f};
  DiagRegs regs[2];

  // lane -> (row r, channels c0 .. c0+3, first token t0 of the lane in the chunk)
  auto lane_map = [&](int& r, int& c0, int& t0) __attribute__((always_inline)) {
    const int lane = opaque_i(threadIdx.x) & 63;
    r = lane / PL;
    c0 = 4 * (PL * part + lane % PL);
    t0 = BT * tb + 8 * r;
  };
  // Tokens past the end of the segment read its last token (a valid
  // address; their weight is 0 and their gate counts as 1); channels past
  // dk / dv read the last channels and only feed rows / columns of S that
  // are not written.  A lane's byte offsets inside a chunk are fixed: its
  // first row's offset is computed once, row q adds q rows (a scalar), and
  // the clamp to the chunk's last token is one unsigned minimum, since the
  // offsets grow with the token.
  int lr, lc0, lt0;
  lane_map(lr, lc0, lt0);
  (void)lr;
  const unsigned rk = unsigned(sk) * 2u, ra = unsigned(sk) * 4u;
  const unsigned ck2 = unsigned(min(lc0, dk - 4)) * 2u;
  const unsigned ok_ = unsigned(lt0) * rk + ck2, oa_ = unsigned(lt0) * ra + 2u * ck2;
  auto load_a = [&](DiagRegs& st, int cq) __attribute__((always_inline)) {
    const int ci = min(cq, last);
    const char* ac = reinterpret_cast<const char*>(abase + int64_t(ci) * C * sk);
    const unsigned lim = unsigned(cq > last ? 0 : chunk_len(u, ci) - 1) * ra + 2u * ck2;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      st.a[q] = nt_f4(ac + min(oa_ + unsigned(q) * ra, lim));
  };
  auto load_k = [&](DiagRegs& st, int cq) __attribute__((always_inline)) {
    const int ci = min(cq, last);
    const char* kc = reinterpret_cast<const char*>(kbase + int64_t(ci) * C * sk);
    const unsigned lim = unsigned(cq > last ? 0 : chunk_len(u, ci) - 1) * rk + ck2;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      st.k[q] = nt_u2(kc + min(ok_ + unsigned(q) * rk, lim));
  };
  auto load_all = [&](auto SET, int ci) __attribute__((always_inline)) {
    DiagRegs& st = regs[decltype(SET)::value];
    load_a(st, ci);
    load_k(st, ci);
  };

  // stage chunk cs from register set SET into buffer cs & 1, reloading the
  // set with chunk cl as each part of it is used up
  auto stage_t = [&](auto TAIL, auto SET, int cs, int cl) __attribute__((always_inline)) {
    constexpr bool tail = decltype(TAIL)::value;
    DiagRegs& st = regs[decltype(SET)::value];
    char* sb = smem + (cs & 1) * L::TOTAL;
    __bf16* Kh = reinterpret_cast<__bf16*>(sb + L::KH);
    __bf16* Kl = reinterpret_cast<__bf16*>(sb + L::KL);
    __bf16* Vt = reinterpret_cast<__bf16*>(sb + L::VT);
    float* gm = reinterpret_cast<float*>(sb + L::GM);
    int r, c0, t0;
    lane_map(r, c0, t0);
    const int lane = opaque_i(threadIdx.x) & 63;
    const int len = chunk_len(u, cs);
    float w[4][8];
    float gv[4], tot[4], pr[4];
    // Gates of tokens past the end count as 1 (such a token keeps the state).
    // A lane's log2 gate sum over its 8 tokens is the log2 of their product,
    // one logarithm instead of eight, as long as the product is a normal
    // float (every partial product is then normal too, the gates being at
    // most 1); otherwise the whole wave takes the gates' logarithms one by one.
    bool tiny = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool ok = !tail || t0 + q < len;
        st.a[q][j] = ok ? st.a[q][j] : 1.f;
      }
      pr[j] = ((st.a[0][j] * st.a[1][j]) * (st.a[2][j] * st.a[3][j])) *
              ((st.a[4][j] * st.a[5][j]) * (st.a[6][j] * st.a[7][j]));
      tiny |= __float_as_int(pr[j]) < 0x00800000;
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(tiny) == 0, 1)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) tot[j] = __builtin_amdgcn_logf(pr[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float l[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) l[q] = log2_gate(st.a[q][j]);
        tot[j] = ((l[0] + l[1]) + (l[2] + l[3])) + ((l[4] + l[5]) + (l[6] + l[7]));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // sum over the rows r' >= r of the block (same lane position)
      float incl = tot[j];
#pragma unroll
      for (int s2 = 1; s2 < RW; s2 <<= 1) {
        const float o = __shfl(incl, lane + s2 * PL, 64);
        incl += (r + s2 < RW) ? o : 0.f;
      }
      w[j][7] = exp2_w(incl - tot[j]);  // product of the gates of later rows
#pragma unroll
      for (int q = 6; q >= 0; --q) w[j][q] = w[j][q + 1] * st.a[q + 1][j];
      lam[j] += incl;  // the block total on rows r == 0, which hold lambda
      gv[j] = exp2_w(incl);
    }
    if (r == 0) *reinterpret_cast<float4*>(gm + tb * DP + c0) = make_float4(gv[0], gv[1], gv[2], gv[3]);
    load_a(st, cl);
    // channel c0 + j: Kw hi / lo of tokens t0 .. t0+7
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      unsigned hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 8; q += 2) {
        const unsigned w0 = (j < 2) ? st.k[q].x : st.k[q].y;
        const unsigned w1 = (j < 2) ? st.k[q + 1].x : st.k[q + 1].y;
        const float x0 = w[j][q] * ((j & 1) ? bf_hi(w0) : bf_lo(w0));
        const float x1 = w[j][q + 1] * ((j & 1) ? bf_hi(w1) : bf_lo(w1));
        split2(x0, x1, hi[q / 2], lo[q / 2]);
      }
      const int at = ch_at<KT>(c0 + j, t0);
      *reinterpret_cast<uint4*>(Kh + at) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<uint4*>(Kl + at) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    load_k(st, cl);
  };
  // One path for full and short chunks (and for the chunk past the last, which
  // the final step stages with every token masked): a branch here makes the
  // compiler merge the register sets at its join, and the register copies
  // there wait for every load in flight, including the ones just issued.
  auto stage = [&](auto SET, int cs, int cl) __attribute__((always_inline)) {
    stage_t(std::true_type(), SET, cs, cl);
  };

  if (n > 0) {
    load_all(I0(), 0);
    load_all(I1(), 1);
    stage(I0(), 0, 2);
    __syncthreads();  // chunk 0 staged
    // step j: stage chunk j+1 (register set (j+1) & 1, buffer (j+1) & 1),
    // reloading the set with chunk j+3; one barrier.  The last step stages
    // the chunk past the end (every token masked: zero weights, no gate) into
    // the buffer nobody reads any more, so every step runs the same code.
    // Reloads for chunks past the last read one row of the last chunk (the
    // loads must be issued, their data is never used; one row stays cached).
    auto step = [&](auto D, int cj) __attribute__((always_inline)) {
      using DN = std::integral_constant<int, (decltype(D)::value + 1) & 1>;
      stage(DN(), cj + 1, cj + 3);
      __syncthreads();
    };
    int cj = 0;
#pragma unroll 1
    for (; cj + 2 <= n; cj += 2) {
      step(I0(), cj);
      step(I1(), cj + 1);
    }
    if (cj < n) step(I0(), cj);
  }
  // lambda: rows r == 0 hold their block's totals; the TG blocks of each
  // channel are summed through LDS (free after the pipeline's last barrier)
  int r, c0, t0;
  lane_map(r, c0, t0);
  (void)t0;
  float* lb = reinterpret_cast<float*>(smem);
  __syncthreads();
  if (r == 0) *reinterpret_cast<float4*>(lb + tb * DP + c0) = make_float4(lam[0], lam[1], lam[2], lam[3]);
  __syncthreads();
  if (r == 0 && tb == 0 && c0 < dk) {
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
