// k_build_sd_pipe.hip -- build of the scalar-decay and diagonal-gate pairs
// (lambda_C, S(C|0)) for bf16 k/v, streaming: the chunk's contraction is on
// split-bf16 MFMA and the inputs of the next chunk(s) are in flight in
// registers while the current chunk is staged and contracted.  Same chunked
// arithmetic as k_build_scalar_diag.hip (which serves fp32 inputs).
// [xix.ai HYPIC article (French), paragraph on linear layers: T_C is the
//  product of the token transitions, S(C|0) the final state from zero; decay
//  (RetNet, Mamba2) and gating (GLA) families.  remio.ai (Japanese), section on
//  state composition: scalar and diagonal transition forms.]
//
// Per chunk of C = 64 tokens, with b_t the in-chunk inclusive prefix of
// log2 alpha (per key channel for the diagonal form):
//   S <- 2^{b_C} (.) S + Kw^T V,   Kw_t = 2^{b_C - b_t} (.) k_t   (factors <= 1)
//
// Staging: thread (token pair tp = lane & 31, channel group of 8) holds
// k, v (and diagonal gates) of tokens 2tp, 2tp+1.  Diagonal prefixes are a
// 32-lane DPP scan over token pairs per channel; the scalar prefix is a
// 64-lane scan every wave does for itself (lanes = tokens).  Kw^T (hi, lo) and
// V^T are written to LDS as (t, t+1) pairs.  Contraction: the DP x DP output
// is cut into 32x32 tiles shared out over the waves, each tile accumulating
// in MFMA registers for the whole segment.
#include "mfma_util.hpp"
#include "pic_internal.hpp"

namespace pic {
namespace {

constexpr int kCs = 64;

template <int DP>
struct SdPipeLds {
  static constexpr int C = kCs;
  static constexpr int KT_LD = C + 8;                 // bf16 row stride (16-byte rows)
  static constexpr int KH = 0;                        // Kw^T hi [DP][KT_LD]
  static constexpr int KL = KH + DP * KT_LD * 2;      // Kw^T lo
  static constexpr int VT = KL + DP * KT_LD * 2;      // V^T
  static constexpr int GM = VT + DP * KT_LD * 2;      // 2^{b_C} per channel [DP]
  static constexpr int TOTAL = GM + DP * 4;
};

__device__ __forceinline__ unsigned pair_w(const uint4& a, const uint4& b, int j) {
  const unsigned wa = (j < 2) ? a.x : (j < 4) ? a.y : (j < 6) ? a.z : a.w;
  const unsigned wb = (j < 2) ? b.x : (j < 4) ? b.y : (j < 6) ? b.z : b.w;
  return __builtin_amdgcn_perm(wb, wa, (j & 1) ? 0x07060302u : 0x05040100u);
}

__device__ __forceinline__ float bf_at(const uint4& a, int j) {
  const unsigned w = (j < 2) ? a.x : (j < 4) ? a.y : (j < 6) ? a.z : a.w;
  return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
}

// element offset of 16-byte chunk `chunk` of row `row` of a transposed
// operand.  With SWZ the chunk index is XOR-swizzled by the row's 8-row group,
// so that transposed writes from rows 8 apart (the scalar form's staging
// mapping) spread over the LDS banks.
template <bool SWZ>
__device__ __forceinline__ int sd_at(int row, int chunk, int ld) {
  return row * ld + 8 * (SWZ ? (chunk ^ ((row >> 3) & 7)) : chunk);
}

__device__ __forceinline__ int opaque_i(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// registers holding one chunk of this thread's staging item
template <bool DIAG>
struct Stage {
  uint4 k0, k1, v0, v1;
  float a0[DIAG ? 8 : 1], a1[DIAG ? 8 : 1];  // diag: gates of tokens t0, t0+1; scalar: lane's gate
};

template <int DP, bool DIAG, int DEPTH>
__global__ __launch_bounds__(4 * DP) void build_sd_pipe_kernel(BuildArgs a) {
  using L = SdPipeLds<DP>;
  constexpr int C = kCs, NTH = 4 * DP, NW = NTH / 64, KT = L::KT_LD;
  constexpr int NTC = DP / 32;                    // 32-wide tiles per side
  constexpr int TILES = NTC * NTC;
  constexpr int TPW = (TILES + NW - 1) / NW;      // tiles per wave
  static_assert((C / 2) * (DP / 8) == NTH, "one staging item per thread");
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  __bf16* Kh = reinterpret_cast<__bf16*>(smem + L::KH);
  __bf16* Kl = reinterpret_cast<__bf16*>(smem + L::KL);
  __bf16* Vt = reinterpret_cast<__bf16*>(smem + L::VT);
  float* gm = reinterpret_cast<float*>(smem + L::GM);

  const int H = a.heads, dk = a.dk, dv = a.dv;
  const int BH = a.batch * H;
  const int seg = a.d_order[blockIdx.x / BH];
  const int bh = blockIdx.x % BH, b = bh / H, h = bh % H;
  const int64_t t_begin = a.d_offsets[seg], t_end = a.d_offsets[seg + 1];
  const int64_t N = a.n_tokens;
  const int n_chunks = int((t_end - t_begin + C - 1) / C);

  f32x16 S[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) S[k] = zero16();
  float lam[DIAG ? 8 : 1];
#pragma unroll
  for (int j = 0; j < (DIAG ? 8 : 1); ++j) lam[j] = 0.f;

  // staging item of a thread: tokens (t0, t0+1) x channels [i0, i0+8).
  // Scalar form: consecutive threads take consecutive channel groups of one
  // token pair, so that a load instruction reads whole 256-byte token rows.
  // Diagonal form: the 32 lanes of a half wave take the 32 token pairs of one
  // channel group (the per-channel prefix is a half-wave scan).
  auto item = [](int tid, int& t0, int& i0) {
    if (DIAG) {
      const int lane = tid & 63;
      t0 = 2 * (lane & 31);
      i0 = 8 * (2 * (tid >> 6) + (lane >> 5));
    } else {
      t0 = 2 * (tid / (DP / 8));
      i0 = 8 * (tid % (DP / 8));
    }
  };
  auto load = [&](Stage<DIAG>& st, int ci) {
    const int tid = opaque_i(threadIdx.x), lane = tid & 63;
    int t0, i0;
    item(tid, t0, i0);
    const int64_t c0 = t_begin + int64_t(ci) * C;
    const int len = (t_end - c0 < C) ? int(t_end - c0) : C;
    const int ta = min(t0, len - 1), tb = min(t0 + 1, len - 1);
    const int ik = min(i0, dk - 8), iv = min(i0, dv - 8);
    const int64_t ra = (int64_t(b) * N + c0 + ta) * H + h;
    const int64_t rb = (int64_t(b) * N + c0 + tb) * H + h;
    const __bf16* kp = static_cast<const __bf16*>(a.k);
    const __bf16* vp = static_cast<const __bf16*>(a.v);
    st.k0 = *reinterpret_cast<const uint4*>(kp + ra * dk + ik);
    st.k1 = *reinterpret_cast<const uint4*>(kp + rb * dk + ik);
    st.v0 = *reinterpret_cast<const uint4*>(vp + ra * dv + iv);
    st.v1 = *reinterpret_cast<const uint4*>(vp + rb * dv + iv);
    if (DIAG) {
      const float4* pa = reinterpret_cast<const float4*>(a.alpha + ra * dk + ik);
      const float4* pb = reinterpret_cast<const float4*>(a.alpha + rb * dk + ik);
      const float4 x0 = pa[0], x1 = pa[1], y0 = pb[0], y1 = pb[1];
      st.a0[0] = x0.x; st.a0[1] = x0.y; st.a0[2] = x0.z; st.a0[3] = x0.w;
      st.a0[4] = x1.x; st.a0[5] = x1.y; st.a0[6] = x1.z; st.a0[7] = x1.w;
      st.a1[0] = y0.x; st.a1[1] = y0.y; st.a1[2] = y0.z; st.a1[3] = y0.w;
      st.a1[4] = y1.x; st.a1[5] = y1.y; st.a1[6] = y1.z; st.a1[7] = y1.w;
    } else {
      st.a0[0] = a.alpha[(int64_t(b) * N + c0 + min(lane, len - 1)) * H + h];
    }
  };

  // stage chunk ci from registers into LDS (Kw^T hi/lo, V^T, channel decays)
  auto stage = [&](const Stage<DIAG>& st, int ci) {
    const int tid = opaque_i(threadIdx.x), lane = tid & 63;
    const int tp = lane & 31;
    int t0, i0;
    item(tid, t0, i0);
    const int64_t c0 = t_begin + int64_t(ci) * C;
    const int len = (t_end - c0 < C) ? int(t_end - c0) : C;
    const bool va = t0 < len, vb = t0 + 1 < len;
    const bool okk = i0 < dk, okv = i0 < dv;
    float w0[8], w1[8];
    if (DIAG) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float l0 = va ? log2f(st.a0[j]) : 0.f, l1 = vb ? log2f(st.a1[j]) : 0.f;
        const float P = half_wave_scan(l0 + l1);  // prefix through token t0+1
        const int Pi = __builtin_bit_cast(int, P);
        const float e0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(Pi, 31));
        const float e1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(Pi, 63));
        const float bend = (lane >> 5) ? e1 : e0;
        w1[j] = exp2f(bend - P);
        w0[j] = exp2f(bend - (P - l1));
        if (tp == 0) {
          lam[j] += bend;
          gm[i0 + j] = exp2f(bend);
        }
      }
    } else {
      const float x = wave_inclusive_scan(lane < len ? log2f(st.a0[0]) : 0.f);
      const float bend =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
      const float wt = exp2f(bend - x);  // weight of token `lane`
      const float wa = __shfl(wt, t0, 64), wb = __shfl(wt, t0 + 1, 64);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        w0[j] = wa;
        w1[j] = wb;
      }
      if (tid == 0) {
        lam[0] += bend;
        gm[0] = exp2f(bend);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      // tokens t0 and t0+1 of channels i0+j and i0+j+1
      const float ka0 = (okk && va) ? w0[j] * bf_at(st.k0, j) : 0.f;
      const float kb0 = (okk && vb) ? w1[j] * bf_at(st.k1, j) : 0.f;
      const float ka1 = (okk && va) ? w0[j + 1] * bf_at(st.k0, j + 1) : 0.f;
      const float kb1 = (okk && vb) ? w1[j + 1] * bf_at(st.k1, j + 1) : 0.f;
      unsigned h0, l0, h1, l1;
      split2(ka0, kb0, h0, l0);
      split2(ka1, kb1, h1, l1);
      const int at0 = sd_at<!DIAG>(i0 + j, t0 >> 3, KT) + (t0 & 7);
      const int at1 = sd_at<!DIAG>(i0 + j + 1, t0 >> 3, KT) + (t0 & 7);
      *reinterpret_cast<unsigned*>(Kh + at0) = h0;
      *reinterpret_cast<unsigned*>(Kl + at0) = l0;
      *reinterpret_cast<unsigned*>(Kh + at1) = h1;
      *reinterpret_cast<unsigned*>(Kl + at1) = l1;
    }
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    const uint4 v0 = (okv && va) ? st.v0 : z, v1 = (okv && vb) ? st.v1 : z;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<unsigned*>(Vt + sd_at<!DIAG>(i0 + j, t0 >> 3, KT) + (t0 & 7)) = pair_w(v0, v1, j);
  };

  // S <- decay (.) S + Kw^T V for this wave's tiles
  auto contract = [&]() {
    const int tid = opaque_i(threadIdx.x), lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, cl = lane & 31;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int tile = wave * TPW + k;
      if (tile < TILES) {
        const int mt = tile / NTC, nt = tile % NTC;
        if (DIAG) {
#pragma unroll
          for (int q = 0; q < 16; ++q) S[k][q] *= gm[mt * 32 + acc_row(q, g)];
        } else {
          S[k] *= gm[0];
        }
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
          const int kch = ks * 2 + g;  // 16-byte chunk of tokens 16 ks + 8 g ..
          const int ka = sd_at<!DIAG>(mt * 32 + cl, kch, KT), va2 = sd_at<!DIAG>(nt * 32 + cl, kch, KT);
          const bf16x8 ah = lds_load8(Kh + ka);
          const bf16x8 al = lds_load8(Kl + ka);
          const bf16x8 vb = lds_load8(Vt + va2);
          S[k] = mfma32(al, vb, S[k]);
          S[k] = mfma32(ah, vb, S[k]);
        }
      }
    }
  };

  Stage<DIAG> buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (d < n_chunks) load(buf[d], d);
#pragma unroll 1
  for (int ci = 0; ci < n_chunks; ci += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int cj = ci + d;
      if (cj < n_chunks) {
        __syncthreads();  // the previous contraction is done with LDS
        stage(buf[d], cj);
        if (cj + DEPTH < n_chunks) load(buf[d], cj + DEPTH);
        __syncthreads();
        contract();
      }
    }
  }

  // ---------------- write the pair
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, cl = lane & 31;
  const int64_t unit = (int64_t(seg) * a.batch + b) * H + h;
  float* out = a.S0 + unit * int64_t(dk) * dv;
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int tile = wave * TPW + k;
    if (tile < TILES) {
      const int mt = tile / NTC, nt = tile % NTC, col = nt * 32 + cl;
      if (col < dv) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = mt * 32 + acc_row(q, g);
          if (row < dk) out[int64_t(row) * dv + col] = S[k][q];
        }
      }
    }
  }
  if (DIAG) {
    const int i0 = 8 * (2 * wave + (lane >> 5));
    if ((lane & 31) == 0 && i0 < dk) {
#pragma unroll
      for (int j = 0; j < 8; ++j) a.log_scale[unit * dk + i0 + j] = lam[j] * kLn2;
    }
  } else if (tid == 0) {
    a.log_scale[unit] = lam[0] * kLn2;
  }
}

template <int DP, bool DIAG>
hipError_t launch_sdp_t(const BuildArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_seg) * a.batch * a.heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  constexpr int DEPTH = DIAG ? 1 : 2;
  hipLaunchKernelGGL((build_sd_pipe_kernel<DP, DIAG, DEPTH>), dim3(unsigned(blocks)),
                     dim3(4 * DP), 0, s, a);
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
