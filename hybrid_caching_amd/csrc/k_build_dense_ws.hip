// k_build_dense_ws.hip -- build of the dense gated-delta pair
// (lambda_C, That_C, S(C|0)) for bf16 k/v with producer and consumer waves.
// Same chunked arithmetic as k_build_dense.hip, which serves fp32 inputs
// (see the derivation there), on sub-chunks of 32 tokens.
// [xix.ai HYPIC article (French), paragraph on linear layers: T_C as the
//  product of the segment's token transitions and S(C|0) from a zero start;
//  dense delta-rule transitions are the heaviest family.]
//
// One workgroup per (segment, layer, head) with DP/32 consumer waves and four
// producer waves (on a 128-wide head: one of each per SIMD).  The segment is
// staged 64 tokens at a time (a "chunk"); the UT transform works on the two
// 32-token halves of a chunk ("sub-chunks" s = 0, 1), which are independent
// of each other, so their triangular systems are solved side by side and
// each is only 32 x 32.
//
// Consumer wave c keeps columns [32c, 32c+32) of BOTH running matrices, S and
// That, in MFMA accumulators for the whole segment, and only runs the chain;
// for sub-chunk s of a chunk:
//   (A_s)  S <- gamma_s S;  N_s = -U_s That,  M_s = W_s - U_s S   (split-bf16 MFMA)
//   (B_s)  That += K_s^T N_s,  S += K_s^T M_s                     (split-bf16 MFMA)
//   (W)    W_s = A'_s V_s of the next chunk, as the seeds of M_s   (MFMA)
// Producer waves prepare chunk ci+1 while the consumers chain chunk ci:
//   stage K (row-major and transposed), V^T and the gates; G_ss = K_s K_s^T;
//   X_s = (I + diag(beta) strictly-lower(G_ss))^{-1} (16x16 blocks by
//   substitution, one 16x16 merge); A_s = X_s diag(beta), A'_s = A_s diag(r)
//   split into bf16 hi/lo; U_s^T = K_s^T A_s^T (MFMA).
// so that S <- gamma S + K^T (W - gamma U S) and That <- That - K^T (U That)
// per sub-chunk.
//
// Hand-over layouts.  The producers compute U_s^T tile by tile; an
// accumulator of a U^T tile holds, in lane (g, token), exactly the A-operand
// fragment the consumer lane (g, token) needs for U . state with the state fed
// from its own accumulators (the permuted K order of mfma_util.hpp), so -U
// goes to LDS as per-lane 16-byte hi/lo fragments and is read back with one
// b128 load each.  Token-indexed K dimensions (K^T, V^T, the columns of A and
// A') are stored with positions 4-7 and 8-11 of every 16 tokens swapped:
// reading positions 8g .. 8g+7 then yields tokens 4g + {0..3} and
// 4g + 8 + {0..3}, the order of an accumulator half used as a B operand.
// In K^T and V^T the eight 16-byte chunks of a row are also XOR-swizzled by
// the row's 8-row group, so that the transposed writes of staging spread
// over the LDS banks; readers apply the same swizzle.
//
// Coalesced loads: a load instruction of a producer wave reads whole 256-byte
// head rows (16 lanes per token row, four token rows), each lane taking
// tokens t and t+1 of one 8-channel group, so that it can write (t, t+1)
// pairs into the transposed layouts.
//
// Both roles run their own loop over chunk cycles with the same sequence of
// seven workgroup barriers per cycle:
//   I0 stage K, V               | S *= gamma_0, (A_0) first half
//   I1 G_00, G_11; gates        | (A_0) second half
//   I2 16x16 diagonal blocks    | (B_0)
//   I3 Y = L X (merge, 1/2)     | S *= gamma_1, (A_1) first half
//   I4 X = -X Y (merge, 2/2)    | (A_1) second half
//   I5 split A, A'              | (B_1)
//   I6 U^T = K^T A^T -> LDS     | W = A' V -> M seeds, N seeds 0
// Cycle ci prepares chunk ci and chains chunk ci-1 (n_chunks + 1 cycles).
#include "mfma_util.hpp"
#include "pic_internal.hpp"
#include "stage_util.hpp"

namespace pic {
namespace {

constexpr int kWsC = 64;
constexpr int kProducers = 4;
constexpr int kPT = kProducers * 64;  // producer threads

template <int DP>
struct WsLds {
  static constexpr int C = kWsC;
  static constexpr int NT = DP / 32;
  static constexpr int KR_LD = DP + 8;  // K row-major, bf16
  static constexpr int KT_LD = C + 8;   // K^T, V^T rows (token positions permuted), bf16
  static constexpr int X_LD = C + 4;    // L, X rows, fp32
  static constexpr int A_LD = C + 8;    // A, A' rows (column positions permuted), bf16
  // region R: K row-major, L and Y while the inverse is formed; then A hi/lo, A' hi/lo
  static constexpr int KR = 0;
  static constexpr int LM = KR + C * KR_LD * 2;
  static constexpr int YM = LM + C * X_LD * 4;
  static constexpr int R_USED = YM + 512 * 4;
  static constexpr int A_BYTES = C * A_LD * 2;
  static constexpr int R_BYTES = (R_USED > 4 * A_BYTES) ? R_USED : 4 * A_BYTES;
  static constexpr int XM = R_BYTES;
  static constexpr int KT = XM + C * X_LD * 4;          // K^T, two buffers (chunk parity)
  static constexpr int VT = KT + 2 * DP * KT_LD * 2;    // V^T
  static constexpr int UF = VT + DP * KT_LD * 2;        // -U fragments
  static constexpr int UF_BYTES = 2 * NT * 2 * 2 * 64 * 16;  // [s][t][h][hi,lo][lane] x 16 B
  static constexpr int GB = UF + UF_BYTES;              // beta of the chunk's tokens
  static constexpr int GR = GB + C * 4;                 // r = gate ratio per token
  static constexpr int GG = GR + C * 4;                 // gamma [chunk parity][sub-chunk]
  static constexpr int GA = GG + 16;                    // alpha, beta of the staged chunk
  static constexpr int GBT = GA + C * 4;
  static constexpr int TOTAL = GBT + C * 4;
  static_assert(KT % 16 == 0 && VT % 16 == 0 && UF % 16 == 0 && XM % 16 == 0, "alignment");
  static_assert(A_BYTES % 16 == 0 && LM % 16 == 0 && GB % 16 == 0, "alignment");
};

// byte offset of a -U fragment: sub-chunk s, channel tile t, half h, part (0 hi, 1 lo), lane
template <int NT>
__device__ __forceinline__ int uf_off(int s, int t, int h, int part, int lane) {
  return ((((s * NT + t) * 2 + h) * 2 + part) * 64 + lane) * 16;
}

template <int DP>
__global__ __launch_bounds__((DP / 32 + kProducers) * 64) void build_dense_ws_kernel(BuildArgs a) {
  using L = WsLds<DP>;
  constexpr int C = kWsC, NT = L::NT;
  constexpr int KR = L::KR_LD, KT = L::KT_LD, XL = L::X_LD, AL = L::A_LD;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  __bf16* Kr = reinterpret_cast<__bf16*>(smem + L::KR);
  __bf16* Kt0 = reinterpret_cast<__bf16*>(smem + L::KT);
  __bf16* Vt = reinterpret_cast<__bf16*>(smem + L::VT);
  char* Uf = smem + L::UF;
  float* Lm = reinterpret_cast<float*>(smem + L::LM);
  float* Xm = reinterpret_cast<float*>(smem + L::XM);
  float* Ym = reinterpret_cast<float*>(smem + L::YM);
  __bf16* Ah = reinterpret_cast<__bf16*>(smem + L::KR);  // X diag(beta), hi / lo
  __bf16* Al = Ah + C * AL;
  __bf16* Bh = Al + C * AL;                              // X diag(beta r), hi / lo
  __bf16* Bl = Bh + C * AL;
  float* gb = reinterpret_cast<float*>(smem + L::GB);
  float* gr = reinterpret_cast<float*>(smem + L::GR);
  float* gg = reinterpret_cast<float*>(smem + L::GG);
  float* ga = reinterpret_cast<float*>(smem + L::GA);
  float* gbt = reinterpret_cast<float*>(smem + L::GBT);

  const int H = a.heads, dk = a.dk, dv = a.dv;
  const int BH = a.batch * H;
  const int seg = seg_in_order(a, int(build_unit(a, blockIdx.x) / BH));
  const int bh = int(build_unit(a, blockIdx.x) % BH), b = bh / H, h = bh % H;
  const int64_t t_begin = seg_offset(a, seg), t_end = seg_offset(a, seg + 1);
  const int64_t N = a.n_tokens;
  const int n_chunks = int((t_end - t_begin + C - 1) / C);
  const int64_t unit = (int64_t(seg) * a.batch + b) * H + h;
  const int lane = threadIdx.x & 63, g = lane >> 5, cl = lane & 31;
  // wave index in a scalar register: the role branch below is uniform
  const int wid = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));

  if (wid < NT) {
    // ===================================================================
    // consumer wave: columns [32 wid, 32 wid + 32) of S and That
    // ===================================================================
    const int c = wid;
    f32x16 XS[NT], XT[NT], PM[2], PN[2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      XS[t] = zero16();
#pragma unroll
      for (int q = 0; q < 16; ++q) XT[t][q] = (t * 32 + acc_row(q, g) == c * 32 + cl) ? 1.f : 0.f;
    }
    PM[0] = PM[1] = PN[0] = PN[1] = zero16();
    constexpr int NK = 2 * NT;  // channel k-steps of 16

    // (A_s) over channel k-steps [k0, k1): N_s += (-U_s) That, M_s += (-U_s) S
    auto chain_a = [&](int s, int k0, int k1) {
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        if (ks < k0 || ks >= k1) continue;
        const int t = ks >> 1, hh = ks & 1;
        bf16x8 th, tl, sh, sl;
        split_acc_half(XT[t], hh, th, tl);
        split_acc_half(XS[t], hh, sh, sl);
        const bf16x8 uh = *reinterpret_cast<const bf16x8*>(Uf + uf_off<NT>(s, t, hh, 0, lane));
        const bf16x8 ul = *reinterpret_cast<const bf16x8*>(Uf + uf_off<NT>(s, t, hh, 1, lane));
        PN[s] = mfma32(ul, th, PN[s]);
        PM[s] = mfma32(ul, sh, PM[s]);
        PN[s] = mfma32(uh, tl, PN[s]);
        PM[s] = mfma32(uh, sl, PM[s]);
        PN[s] = mfma32(uh, th, PN[s]);
        PM[s] = mfma32(uh, sh, PM[s]);
      }
    };
    // (B_s): That += K_s^T N_s, S += K_s^T M_s over the sub-chunk's 32 tokens
    auto chain_b = [&](int s, const __bf16* Ktp) {
      const int ln = opaque(lane);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int kb = kt_lane_base<KT>(ln & 31, ln >> 5, hh);
        bf16x8 nh, nl, mh, ml;
        split_acc_half(PN[s], hh, nh, nl);
        split_acc_half(PM[s], hh, mh, ml);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 kf = lds_load8(Ktp + kb + kt_tile<KT>(t, s));
          XT[t] = mfma32(kf, nl, XT[t]);
          XS[t] = mfma32(kf, ml, XS[t]);
          XT[t] = mfma32(kf, nh, XT[t]);
          XS[t] = mfma32(kf, mh, XS[t]);
        }
      }
    };
    auto scale_s = [&](float gam) {
#pragma unroll
      for (int t = 0; t < NT; ++t) XS[t] *= gam;
    };

#pragma unroll 1
    for (int ci = 0; ci <= n_chunks; ++ci) {
      const bool chain = ci > 0, prep = ci < n_chunks;
      const __bf16* Ktp = Kt0 + ((ci - 1) & 1) * (DP * KT);
      const float* gamma = gg + 2 * ((ci - 1) & 1);
      __syncthreads();  // I0: -U and gamma of chunk ci-1 are in LDS
      if (chain) {
        scale_s(gamma[0]);
        chain_a(0, 0, NK / 2);
      }
      __syncthreads();  // I1
      if (chain) chain_a(0, NK / 2, NK);
      __syncthreads();  // I2
      if (chain) chain_b(0, Ktp);
      __syncthreads();  // I3
      if (chain) {
        scale_s(gamma[1]);
        chain_a(1, 0, NK / 2);
      }
      __syncthreads();  // I4
      if (chain) chain_a(1, NK / 2, NK);
      __syncthreads();  // I5
      if (chain) chain_b(1, Ktp);
      __syncthreads();  // I6: A' and V^T of chunk ci are in LDS
      if (prep) {
        const int ln = opaque(lane);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          f32x16 acc = zero16();
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int kc = 32 * s + 16 * kk + 8 * g;
            const bf16x8 ph = lds_load8(Bh + (s * 32 + cl) * AL + kc);
            const bf16x8 pl = lds_load8(Bl + (s * 32 + cl) * AL + kc);
            const bf16x8 vf = lds_load8(Vt + kt_lane_base<KT>(ln & 31, ln >> 5, kk) +
                                        kt_tile<KT>(c, s));
            acc = mfma32(pl, vf, acc);
            acc = mfma32(ph, vf, acc);
          }
          PM[s] = acc;
          PN[s] = zero16();
        }
      }
    }

    // write this wave's columns of S(C|0) and That_C
    const int ncol = c * 32 + cl;
    if (ncol < dv) {
      float* out = a.S0 + unit * int64_t(dk) * dv;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = t * 32 + acc_row(q, g);
          if (row < dk) out[int64_t(row) * dv + ncol] = XS[t][q];
        }
    }
    if (ncol < dk) {
      float* out = a.T_hat + unit * int64_t(dk) * dk;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = t * 32 + acc_row(q, g);
          if (row < dk) out[int64_t(row) * dk + ncol] = XT[t][q];
        }
    }
  } else {
    // ===================================================================
    // producer waves
    // ===================================================================
    const int pw = wid - NT;                 // producer wave 0..3
    const int p = pw * 64 + lane;            // producer thread 0..255
    constexpr int NCG = DP / 8;              // 8-channel groups
    constexpr int NIT = (32 * NCG + kPT - 1) / kPT;  // staging items per thread
    constexpr int PPI = kPT / NCG;                   // token pairs per item round
    float lam = 0.f;

    // strictly upper 16x16 blocks of each sub-chunk's X stay zero for the
    // whole segment (the blocks coupling the two sub-chunks are never read)
    for (int e = p; e < 2 * 256; e += kPT) {
      const int s = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      Xm[(32 * s + r) * XL + 32 * s + 16 + cc] = 0.f;
    }

    // register prefetch of one chunk: item i of this thread is tokens
    // (t0, t0+1) x channels [8 cg, 8 cg + 8) with cg = p % 16 and
    // t0 = 2 (p / 16 + 16 i): each load instruction of a wave covers four
    // whole 256-byte token rows.
    uint4 pk[NIT][2], pv[NIT][2];
    // alpha, beta of token lane, prefetched by every producer wave with the
    // k/v items: loads without a select on the loaded value, so that no wait
    // for them is needed before they are staged (beta = 1 is applied at use)
    float pa = 1.f, pb = 0.f;
    const float* bsrc = a.beta ? a.beta : a.alpha;
    auto prefetch = [&](int ci) {
      const int64_t c0 = t_begin + int64_t(ci) * C;
      const int len = (t_end - c0 < C) ? int(t_end - c0) : C;
      const __bf16* kp = static_cast<const __bf16*>(a.k);
      const __bf16* vp = static_cast<const __bf16*>(a.v);
      const int cg = p % NCG;
      const int ik = min(8 * cg, dk - 8), iv = min(8 * cg, dv - 8);
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int t0 = 2 * (p / NCG + PPI * i);
        // clamped (in-segment, in-head) addresses; zeroing happens at staging
        const int ta = min(t0, len - 1), tb = min(t0 + 1, len - 1);
        const int64_t ra = (int64_t(b) * N + c0 + ta) * H + h;
        const int64_t rb = (int64_t(b) * N + c0 + tb) * H + h;
        pk[i][0] = *reinterpret_cast<const uint4*>(kp + ra * dk + ik);
        pk[i][1] = *reinterpret_cast<const uint4*>(kp + rb * dk + ik);
        pv[i][0] = *reinterpret_cast<const uint4*>(vp + ra * dv + iv);
        pv[i][1] = *reinterpret_cast<const uint4*>(vp + rb * dv + iv);
      }
      const int64_t gi = (int64_t(b) * N + c0 + min(lane, len - 1)) * H + h;
      pa = a.alpha[gi];
      pb = bsrc[gi];
    };

    if (n_chunks > 0) prefetch(0);
#pragma unroll 1
    for (int ci = 0; ci <= n_chunks; ++ci) {
      const bool prep = ci < n_chunks;
      __bf16* Kt = Kt0 + (ci & 1) * (DP * KT);
      const int64_t c0 = t_begin + int64_t(ci) * C;
      const int len = prep ? ((t_end - c0 < C) ? int(t_end - c0) : C) : 0;

      // ---------------- I0: stage chunk ci; prefetch chunk ci+1
      __syncthreads();
      if (prep) {
        const int cg = p % NCG, i0 = 8 * cg;
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
          const int t0 = 2 * (p / NCG + PPI * i);
          if (t0 < C) {
            const int pos = tpos(t0);
            const uint4 k0 = ws_pick(i0 < dk && t0 < len, pk[i][0]);
            const uint4 k1 = ws_pick(i0 < dk && t0 + 1 < len, pk[i][1]);
            const uint4 v0 = ws_pick(i0 < dv && t0 < len, pv[i][0]);
            const uint4 v1 = ws_pick(i0 < dv && t0 + 1 < len, pv[i][1]);
            *reinterpret_cast<uint4*>(Kr + t0 * KR + i0) = k0;
            *reinterpret_cast<uint4*>(Kr + (t0 + 1) * KR + i0) = k1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int at = kt_at<KT>(i0 + j, pos >> 3) + (pos & 7);
              *reinterpret_cast<unsigned*>(Kt + at) = ws_pair(k0, k1, j);
              *reinterpret_cast<unsigned*>(Vt + at) = ws_pair(v0, v1, j);
            }
          }
        }
        if (pw == kProducers - 1) {
          ga[lane] = pa;
          gbt[lane] = pb;
        }
        if (ci + 1 < n_chunks) prefetch(ci + 1);
      }

      // ---------------- I1: G_ss = strictly-lower(K_s K_s^T) (waves 0, 1; row
      // r of L is beta_r times row r of G, applied where L is read); gates of
      // both sub-chunks (wave 3, one sub-chunk per half wave)
      __syncthreads();
      if (prep && pw < 2) {
        const int s = pw;
        f32x16 acc0 = zero16(), acc1 = zero16();  // two chains of dependent MFMAs
#pragma unroll
        for (int ks = 0; ks < DP / 16; ++ks) {
          const int kc = ks * 16 + 8 * g;
          const bf16x8 ak = lds_load8(Kr + (s * 32 + cl) * KR + kc);
          if (ks & 1)
            acc1 = mfma32(ak, ak, acc1);
          else
            acc0 = mfma32(ak, ak, acc0);
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = acc_row(q, g);
          Lm[(s * 32 + r) * XL + s * 32 + cl] = (cl < r) ? acc0[q] + acc1[q] : 0.f;
        }
      }
      if (prep && pw == kProducers - 1) {
        const float x = half_wave_scan(lane < len ? log2f(ga[lane]) : 0.f);
        const int xi = __builtin_bit_cast(int, x);
        const float e0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 31));
        const float e1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 63));
        const float bend = g ? e1 : e0;
        gb[lane] = lane < len ? (a.beta ? gbt[lane] : 1.f) : 0.f;
        gr[lane] = exp2f(bend - x);
        if (lane == 0) {
          gg[2 * (ci & 1)] = exp2f(e0);
          gg[2 * (ci & 1) + 1] = exp2f(e1);
        }
        lam += e0 + e1;
      }

      // ---------------- I2: 16x16 diagonal blocks of X by substitution
      // (four lanes per column, lane pp owning entries 4pp .. 4pp+3; partial
      // sums combined on DPP)
      __syncthreads();
      if (prep) {
        const int col = p >> 2, pp = p & 3;
        const int o = 16 * (col >> 4), cc = col & 15;
        float xo[4], lv[16][4], br[16];
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const float4 b4 = *reinterpret_cast<const float4*>(gb + o + r);
          br[r] = b4.x; br[r + 1] = b4.y; br[r + 2] = b4.z; br[r + 3] = b4.w;
        }
#pragma unroll
        for (int r = 1; r < 16; ++r) {
          const float4 v4 = *reinterpret_cast<const float4*>(Lm + (o + r) * XL + o + 4 * pp);
          const float v[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) lv[r][j] = (4 * pp + j < r) ? br[r] * v[j] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) xo[j] = (4 * pp + j == cc) ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
          float sm = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) sm = fmaf(lv[r][j], xo[j], sm);
          sm = group_sum<4>(sm);
          if (r > cc && pp == (r >> 2)) xo[r & 3] = -sm;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) Xm[(o + 4 * pp + j) * XL + o + cc] = xo[j];
      }

      // ---------------- I3: 16x16 merges, Y = L_10 X_00 of each sub-chunk
      // (each thread: one row, two adjacent columns; vector LDS loads)
      __syncthreads();
      if (prep) {
        const int s = p >> 7, r = (p >> 3) & 15, c2 = 2 * (p & 7);
        const int orow = 32 * s + 16, ocol = 32 * s;
        float lrow[16];
#pragma unroll
        for (int q = 0; q < 16; q += 4) {
          const float4 v = *reinterpret_cast<const float4*>(Lm + (orow + r) * XL + ocol + q);
          lrow[q] = v.x; lrow[q + 1] = v.y; lrow[q + 2] = v.z; lrow[q + 3] = v.w;
        }
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const float2 x = *reinterpret_cast<const float2*>(Xm + (ocol + q) * XL + ocol + c2);
          s0 = fmaf(lrow[q], x.x, s0);
          s1 = fmaf(lrow[q], x.y, s1);
        }
        const float bw = gb[orow + r];
        *reinterpret_cast<float2*>(Ym + s * 256 + r * 16 + c2) = make_float2(bw * s0, bw * s1);
      }

      // ---------------- I4: X_10 = -X_11 Y of each sub-chunk
      __syncthreads();
      if (prep) {
        const int s = p >> 7, r = (p >> 3) & 15, c2 = 2 * (p & 7);
        const int orow = 32 * s + 16, ocol = 32 * s;
        float xrow[16];
#pragma unroll
        for (int q = 0; q < 16; q += 4) {
          const float4 v = *reinterpret_cast<const float4*>(Xm + (orow + r) * XL + orow + q);
          xrow[q] = v.x; xrow[q + 1] = v.y; xrow[q + 2] = v.z; xrow[q + 3] = v.w;
        }
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const float2 y = *reinterpret_cast<const float2*>(Ym + s * 256 + q * 16 + c2);
          s0 = fmaf(xrow[q], y.x, s0);
          s1 = fmaf(xrow[q], y.y, s1);
        }
        *reinterpret_cast<float2*>(Xm + (orow + r) * XL + ocol + c2) = make_float2(-s0, -s1);
      }

      // ---------------- I5: A_s = X_s diag(beta), A'_s = A_s diag(r), split
      // hi/lo, columns stored at permuted positions (region of K, L, Y is dead)
      __syncthreads();
      if (prep) {
        const int s = p >> 7, row = 32 * s + ((p >> 2) & 31), c0 = 32 * s + 8 * (p & 3);
        // positions c0 .. c0+7 hold tokens t4 + {0..3} and t4 + 8 + {0..3}
        const int t4 = (c0 & ~15) + ((c0 & 8) ? 4 : 0);
        float av[8], bv[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int tk = t4 + 8 * hf;
          const float4 x = *reinterpret_cast<const float4*>(Xm + row * XL + tk);
          const float4 bb = *reinterpret_cast<const float4*>(gb + tk);
          const float4 rr = *reinterpret_cast<const float4*>(gr + tk);
          av[4 * hf] = x.x * bb.x; av[4 * hf + 1] = x.y * bb.y;
          av[4 * hf + 2] = x.z * bb.z; av[4 * hf + 3] = x.w * bb.w;
          bv[4 * hf] = av[4 * hf] * rr.x; bv[4 * hf + 1] = av[4 * hf + 1] * rr.y;
          bv[4 * hf + 2] = av[4 * hf + 2] * rr.z; bv[4 * hf + 3] = av[4 * hf + 3] * rr.w;
        }
        bf16x8 h8, l8;
        split8(av, h8, l8);
        *reinterpret_cast<bf16x8*>(Ah + row * AL + c0) = h8;
        *reinterpret_cast<bf16x8*>(Al + row * AL + c0) = l8;
        split8(bv, h8, l8);
        *reinterpret_cast<bf16x8*>(Bh + row * AL + c0) = h8;
        *reinterpret_cast<bf16x8*>(Bl + row * AL + c0) = l8;
      }

      // ---------------- I6: U_s^T = K_s^T A_s^T tile by tile; -U fragments to
      // LDS (the consumers finished reading the previous -U in I4)
      __syncthreads();
      if (prep) {
#pragma unroll
        for (int i = 0; i < (2 * NT + kProducers - 1) / kProducers; ++i) {
          const int tile = pw + i * kProducers;
          if (tile >= 2 * NT) break;
          const int t = tile % NT, s = tile / NT;
          f32x16 acc = zero16();
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int kc = 32 * s + 16 * kk + 8 * g;
            const bf16x8 kf = lds_load8(Kt + kt_lane_base<KT>(cl, g, kk) + kt_tile<KT>(t, s));
            const bf16x8 ah = lds_load8(Ah + (s * 32 + cl) * AL + kc);
            const bf16x8 al = lds_load8(Al + (s * 32 + cl) * AL + kc);
            acc = mfma32(kf, al, acc);
            acc = mfma32(kf, ah, acc);
          }
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = -acc[8 * hh + j];
            bf16x8 h8, l8;
            split8(x, h8, l8);
            *reinterpret_cast<bf16x8*>(Uf + uf_off<NT>(s, t, hh, 0, lane)) = h8;
            *reinterpret_cast<bf16x8*>(Uf + uf_off<NT>(s, t, hh, 1, lane)) = l8;
          }
        }
      }
    }
    if (pw == kProducers - 1 && lane == 0) a.log_scale[unit] = lam * kLn2;
  }
}

template <int DP>
hipError_t launch_ws_t(const BuildArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_seg) * a.batch * a.heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(build_dense_ws_kernel<DP>, dim3(unsigned(blocks)),
                     dim3((DP / 32 + kProducers) * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_dense_ws(const BuildArgs& a, hipStream_t s) {
  const int d = a.dk > a.dv ? a.dk : a.dv;
  if (d <= 32) return launch_ws_t<32>(a, s);
  if (d <= 64) return launch_ws_t<64>(a, s);
  return launch_ws_t<128>(a, s);
}

}  // namespace pic
