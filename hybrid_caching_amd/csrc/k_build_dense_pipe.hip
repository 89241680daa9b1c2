// k_build_dense_pipe.hip -- build of the dense gated-delta pair
// (lambda_C, That_C, S(C|0)) for bf16 k/v, with the next chunk's inputs
// prefetched into registers.  Same chunked arithmetic as k_build_dense.hip
// (which serves fp32 inputs); see the derivation there.
// [xix.ai HYPIC article (French), paragraph on linear layers: T_C as the
//  product of the segment's token transitions and S(C|0) from a zero start;
//  dense delta-rule transitions are the heaviest family.]
//
// One workgroup per (segment, layer, head); 2*DP/32 waves: waves [0, DP/32)
// hold 32-column strips of S, waves [DP/32, 2*DP/32) strips of That, in MFMA
// accumulators for the whole segment.  Per chunk of 64 tokens:
//   1  stage K (row-major and transposed) and V^T into LDS from registers,
//      gates (DPP prefix scan of log2 alpha, one wave); prefetch the next chunk
//   2  L = diag(beta) strictly-lower(K K^T)              (MFMA, exact in bf16)
//   3  X = (I + L)^{-1}, 16x16 diagonal blocks: lanes share a column and
//      combine partial sums with DPP lane exchanges
//   4  16x16 merges  X_10 = -X_11 L_10 X_00,  X_32 = -X_33 L_32 X_22  (2 steps)
//   5  32x32 merge   X_[2:4][0:2] = -X_22 L_21 X_11       (split-bf16 MFMA)
//   6  A = X diag(beta) and A' = X diag(beta r) split into bf16 hi/lo once;
//      U = A K into LDS; the accumulator M of each wave is seeded with
//      W = A' V (S strips) or 0 (That strips)
//   7  M += U (sigma X) with sigma = -gamma (S) or -1 (That); S *= gamma;
//      X += K^T M                                          (split-bf16 MFMA)
// so that S <- gamma S + K^T (W - gamma U S) and That <- That - K^T (U That).
//
// Software pipeline.  Steps 1-6 of a chunk do not depend on the running
// pair, so step 7 of chunk ci-1 is cut into four slices that run in the
// phases of steps 1-4 of chunk ci (K^T is double-buffered by chunk parity);
// the matrix-core work of one chunk fills the latency of the next one's
// preparation.  The last chunk's step 7 runs after the loop.
#include "mfma_util.hpp"
#include "pic_internal.hpp"

namespace pic {
namespace {

constexpr int kC = 64;

template <int DP>
struct PipeLds {
  static constexpr int C = kC;
  static constexpr int KR_LD = DP + 8;  // K row-major (16-byte rows for b128 reads)
  static constexpr int U_LD = DP + 4;   // U rows (b64 reads; stride spreads banks)
  static constexpr int KT_LD = C + 8;   // K^T, V^T rows
  static constexpr int X_LD = C + 4;    // L, X rows (fp32)
  static constexpr int A_LD = C + 8;    // split X diag(beta), X diag(beta r) rows
  // region R: K row-major, L and Y while the chunk's inverse is formed; then
  // the four split operand matrices of U = A K and W = A' V
  static constexpr int KR = 0;
  static constexpr int LM = KR + C * KR_LD * 2;
  static constexpr int YM = LM + C * X_LD * 4;
  static constexpr int R_USED = YM + 512 * 4;
  static constexpr int A_BYTES = C * A_LD * 2;  // one split part
  static constexpr int R_BYTES = (R_USED > 4 * A_BYTES) ? R_USED : 4 * A_BYTES;
  static constexpr int KT = R_BYTES;                  // K^T, two buffers (chunk parity)
  static constexpr int VT = KT + 2 * DP * KT_LD * 2;
  static constexpr int UH = VT + DP * KT_LD * 2;
  static constexpr int UL = UH + C * U_LD * 2;
  static constexpr int XM = UL + C * U_LD * 2;
  static constexpr int GB = XM + C * X_LD * 4;
  static constexpr int GR = GB + C * 4;
  static constexpr int GG = GR + C * 4;  // gamma per chunk parity
  static constexpr int TOTAL = GG + 16;
  static_assert(KT % 16 == 0 && VT % 16 == 0 && UH % 16 == 0 && XM % 16 == 0, "alignment");
  static_assert(A_BYTES % 16 == 0 && LM % 16 == 0, "alignment");
};

// (element j of token a, element j of token b) as one packed pair: one
// byte permute of the 32-bit words holding them
__device__ __forceinline__ unsigned pair_of(const uint4& a, const uint4& b, int j) {
  const unsigned wa = (j < 2) ? a.x : (j < 4) ? a.y : (j < 6) ? a.z : a.w;
  const unsigned wb = (j < 2) ? b.x : (j < 4) ? b.y : (j < 6) ? b.z : b.w;
  return __builtin_amdgcn_perm(wb, wa, (j & 1) ? 0x07060302u : 0x05040100u);
}

// a copy of v the compiler cannot see through: keeps per-lane address
// arithmetic inside the chunk loop instead of hoisting it (and spilling it)
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int DP>
__global__ __launch_bounds__(4 * DP) void build_dense_pipe_kernel(BuildArgs a) {
  using L = PipeLds<DP>;
  constexpr int C = kC, NT = DP / 32, NW = 2 * NT, NTH = NW * 64;
  constexpr int KR = L::KR_LD, ULD = L::U_LD, KT = L::KT_LD, XL = L::X_LD, AL = L::A_LD;
  constexpr int TPC = NTH / 64;  // lanes per column in the diagonal solve
  constexpr int JPT = 16 / TPC;  // column entries owned per lane
  static_assert((C / 2) * (DP / 8) == NTH, "one staging item per thread");
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  __bf16* Kr = reinterpret_cast<__bf16*>(smem + L::KR);
  __bf16* Kt0 = reinterpret_cast<__bf16*>(smem + L::KT);
  __bf16* Vt = reinterpret_cast<__bf16*>(smem + L::VT);
  __bf16* Uh = reinterpret_cast<__bf16*>(smem + L::UH);
  __bf16* Ul = reinterpret_cast<__bf16*>(smem + L::UL);
  float* Lm = reinterpret_cast<float*>(smem + L::LM);
  float* Xm = reinterpret_cast<float*>(smem + L::XM);
  float* Ym = reinterpret_cast<float*>(smem + L::YM);
  __bf16* Ah = reinterpret_cast<__bf16*>(smem + L::KR);  // X diag(beta), hi / lo
  __bf16* Al = Ah + C * L::A_LD;
  __bf16* Bh = Al + C * L::A_LD;                          // X diag(beta r), hi / lo
  __bf16* Bl = Bh + C * L::A_LD;
  float* gb = reinterpret_cast<float*>(smem + L::GB);
  float* gr = reinterpret_cast<float*>(smem + L::GR);
  float* gg = reinterpret_cast<float*>(smem + L::GG);

  const int H = a.heads, dk = a.dk, dv = a.dv;
  const int BH = a.batch * H;
  const int seg = a.d_order[blockIdx.x / BH];
  const int bh = blockIdx.x % BH, b = bh / H, h = bh % H;
  const int64_t t_begin = a.d_offsets[seg], t_end = a.d_offsets[seg + 1];
  const int64_t N = a.n_tokens;
  const int n_chunks = int((t_end - t_begin + C - 1) / C);
  const bool s_wave = int(threadIdx.x >> 6) < NT;  // wave-uniform

  f32x16 X[NT];  // this wave's strip of S (s_wave) or That
  {
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
    const int ncol = ((tid >> 6) % NT) * 32 + (lane & 31);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        X[t][q] = (!s_wave && t * 32 + acc_row(q, g) == ncol) ? 1.f : 0.f;
    // strictly upper 16x16 blocks of X stay zero for the whole segment
    for (int e = tid; e < 6 * 256; e += NTH) {
      const int blk = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      const int bi = (blk < 3) ? 0 : ((blk < 5) ? 1 : 2);
      const int bj = (blk < 3) ? blk + 1 : ((blk < 5) ? blk - 1 : 3);
      Xm[(16 * bi + r) * XL + 16 * bj + cc] = 0.f;
    }
  }
  float lam = 0.f;

  // register prefetch of one chunk: this thread's staging item is tokens
  // (t0, t0+1) x dims [i0, i0+8) with t0 = 2 (lane & 31) and
  // i0 = 8 (2 wave + lane / 32), so that the transposed LDS writes of a wave
  // fall on consecutive banks; wave 0 also takes alpha/beta of token lane
  uint4 pk0, pk1, pv0, pv1;
  float pa = 1.f, pb = 0.f;
  auto prefetch = [&](int ci) {
    const int tid = opaque(threadIdx.x), lane = tid & 63;
    const int t0 = 2 * (lane & 31), i0 = 8 * (2 * (tid >> 6) + (lane >> 5));
    const int64_t c0 = t_begin + int64_t(ci) * C;
    const int len = (t_end - c0 < C) ? int(t_end - c0) : C;
    // unconditional 16-byte loads from clamped (in-segment) addresses; lanes
    // past the segment end or the head size keep zeros
    const int ta = min(t0, len - 1), tb = min(t0 + 1, len - 1);
    const int ik = min(i0, dk - 8), iv = min(i0, dv - 8);
    const int64_t ra = (int64_t(b) * N + c0 + ta) * H + h;
    const int64_t rb = (int64_t(b) * N + c0 + tb) * H + h;
    const __bf16* kp = static_cast<const __bf16*>(a.k);
    const __bf16* vp = static_cast<const __bf16*>(a.v);
    const uint4 k0 = *reinterpret_cast<const uint4*>(kp + ra * dk + ik);
    const uint4 k1 = *reinterpret_cast<const uint4*>(kp + rb * dk + ik);
    const uint4 v0 = *reinterpret_cast<const uint4*>(vp + ra * dv + iv);
    const uint4 v1 = *reinterpret_cast<const uint4*>(vp + rb * dv + iv);
    pk0 = k0;
    pk1 = k1;
    pv0 = v0;
    pv1 = v1;
    if ((tid >> 6) == 0) {
      const int64_t gi = (int64_t(b) * N + c0 + min(lane, len - 1)) * H + h;
      pa = a.alpha[gi];
      pb = a.beta ? a.beta[gi] : 1.f;
    }
  };
  // zero what lies past the segment end or the head size (applied when the
  // prefetched registers are consumed, so the loads stay in flight until then)
  auto pick = [](bool ok, uint4 x) {
    return make_uint4(ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u, ok ? x.w : 0u);
  };

  f32x16 P[2];  // M of the chunk in flight (seeded with W or 0)

  // step 7 slices for chunk pc (its U in LDS, its K^T in buffer pc & 1)
  auto chain_um = [&](int half, int pc) {  // P += U (sigma X) over K rows of one half
    const int lane = opaque(threadIdx.x) & 63, g = lane >> 5, cl = lane & 31;
    const float sigma = s_wave ? -gg[pc & 1] : -1.f;
#pragma unroll
    for (int kk = 0; kk < NT; ++kk) {
      const int ks = half * NT + kk, t = ks >> 1, hh = ks & 1;
      float xv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xv[j] = sigma * X[t][8 * hh + j];
      bf16x8 bhi, blo;
      split8(xv, bhi, blo);
      const int kc = 32 * t + 16 * hh + 4 * g;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 ah = lds_perm8(Uh + (mt * 32 + cl) * ULD, kc);
        const bf16x8 al = lds_perm8(Ul + (mt * 32 + cl) * ULD, kc);
        P[mt] = mfma32(al, bhi, P[mt]);
        P[mt] = mfma32(ah, blo, P[mt]);
        P[mt] = mfma32(ah, bhi, P[mt]);
      }
    }
  };
  auto chain_ktm = [&](int mt, int pc) {  // X += K^T M_mt  (S first scaled by gamma)
    const int lane = opaque(threadIdx.x) & 63, g = lane >> 5, cl = lane & 31;
    const __bf16* Ktp = Kt0 + (pc & 1) * (DP * KT);
    if (mt == 0 && s_wave) {
      const float gam = gg[pc & 1];
#pragma unroll
      for (int t = 0; t < NT; ++t) X[t] *= gam;
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x8 bhi, blo;
      split_acc_half(P[mt], hh, bhi, blo);
      const int kc = 32 * mt + 16 * hh + 4 * g;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 kh = lds_perm8(Ktp + (t * 32 + cl) * KT, kc);
        X[t] = mfma32(kh, blo, X[t]);
        X[t] = mfma32(kh, bhi, X[t]);
      }
    }
  };

  if (n_chunks > 0) prefetch(0);
#pragma unroll 1
  for (int ci = 0; ci < n_chunks; ++ci) {
    const int tid = opaque(threadIdx.x), lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, cl = lane & 31;
    const int strip = wave % NT;
    const bool chain = ci > 0;  // step 7 of chunk ci-1 rides along
    __bf16* Kt = Kt0 + (ci & 1) * (DP * KT);

    // ---------------- 1: stage chunk ci, gates; prefetch chunk ci+1
    __syncthreads();  // the previous chunk is done with every LDS buffer
    // The S wave and the That wave sharing a SIMD take their phase work in
    // opposite orders (matrix slice first / preparation first), so that one's
    // MFMAs overlap the other's VALU and LDS work.
    if (chain && s_wave) chain_um(0, ci - 1);
    {
      const int t0 = 2 * (lane & 31), i0 = 8 * (2 * wave + (lane >> 5));
      const int64_t c0 = t_begin + int64_t(ci) * C;
      const int len = (t_end - c0 < C) ? int(t_end - c0) : C;
      const uint4 k0 = pick(i0 < dk && t0 < len, pk0), k1 = pick(i0 < dk && t0 + 1 < len, pk1);
      const uint4 v0 = pick(i0 < dv && t0 < len, pv0), v1 = pick(i0 < dv && t0 + 1 < len, pv1);
      *reinterpret_cast<uint4*>(Kr + t0 * KR + i0) = k0;
      *reinterpret_cast<uint4*>(Kr + (t0 + 1) * KR + i0) = k1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        *reinterpret_cast<unsigned*>(Kt + (i0 + j) * KT + t0) = pair_of(k0, k1, j);
        *reinterpret_cast<unsigned*>(Vt + (i0 + j) * KT + t0) = pair_of(v0, v1, j);
      }
    }
    if (wave == 0) {
      const int64_t c0 = t_begin + int64_t(ci) * C;
      const int len = (t_end - c0 < C) ? int(t_end - c0) : C;
      const float x = wave_inclusive_scan(lane < len ? log2f(pa) : 0.f);
      const float bend =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
      gb[lane] = lane < len ? pb : 0.f;
      gr[lane] = exp2f(bend - x);
      if (lane == 0) gg[ci & 1] = exp2f(bend);
      lam += bend;
    }
    if (ci + 1 < n_chunks) prefetch(ci + 1);
    if (chain && !s_wave) chain_um(0, ci - 1);

    // ---------------- 2: L = diag(beta) strictly-lower(K K^T)  (That waves)
    __syncthreads();
    if (chain && s_wave) chain_um(1, ci - 1);
    for (int tile = (wave + NT) % NW; tile < 3; tile += NW) {
      const int mt = (tile == 0) ? 0 : 1, nt = (tile == 2) ? 1 : 0;
      f32x16 acc = zero16();
#pragma unroll
      for (int ks = 0; ks < DP / 16; ++ks) {
        const int kc = ks * 16 + 8 * g;
        const bf16x8 ah = lds_load8(Kr + (mt * 32 + cl) * KR + kc);
        const bf16x8 bk = lds_load8(Kr + (nt * 32 + cl) * KR + kc);
        acc = mfma32(ah, bk, acc);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = mt * 32 + acc_row(q, g), c = nt * 32 + cl;
        const float bv = gb[r];
        Lm[r * XL + c] = (c < r) ? bv * acc[q] : 0.f;
      }
    }
    if (chain && !s_wave) chain_um(1, ci - 1);

    // ---------------- 3: 16x16 diagonal blocks of X by substitution
    __syncthreads();
    if (chain && s_wave) chain_ktm(0, ci - 1);
    {
      const int col = tid / TPC, p = tid % TPC;
      const int o = 16 * (col >> 4), cc = col & 15;
      float xo[JPT], lv[16][JPT];  // L entries this lane needs, zero above the diagonal
#pragma unroll
      for (int r = 1; r < 16; ++r)
#pragma unroll
        for (int j = 0; j < JPT; ++j) {
          const float v = Lm[(o + r) * XL + o + p + TPC * j];
          lv[r][j] = (p + TPC * j < r) ? v : 0.f;
        }
#pragma unroll
      for (int j = 0; j < JPT; ++j) xo[j] = (p + TPC * j == cc) ? 1.f : 0.f;
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < JPT; ++j) s = fmaf(lv[r][j], xo[j], s);
        s = group_sum<TPC>(s);
        if (r > cc && p == (r % TPC)) xo[r / TPC] = -s;
      }
#pragma unroll
      for (int j = 0; j < JPT; ++j) Xm[(o + p + TPC * j) * XL + o + cc] = xo[j];
    }
    if (chain && !s_wave) chain_ktm(0, ci - 1);

    // ---------------- 4: 16x16 merges (Y = L X, then X = -X Y)
    __syncthreads();
    if (chain && s_wave) chain_ktm(1, ci - 1);
    for (int e = tid; e < 512; e += NTH) {
      const int inst = e >> 8, r = (e >> 4) & 15, c = e & 15;
      const int orow = inst ? 48 : 16, ocol = inst ? 32 : 0;
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        s = fmaf(Lm[(orow + r) * XL + ocol + q], Xm[(ocol + q) * XL + ocol + c], s);
      Ym[e] = s;
    }
    if (chain && !s_wave) chain_ktm(1, ci - 1);
    __syncthreads();
    for (int e = tid; e < 512; e += NTH) {
      const int inst = e >> 8, r = (e >> 4) & 15, c = e & 15;
      const int orow = inst ? 48 : 16, ocol = inst ? 32 : 0;
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        s = fmaf(Xm[(orow + r) * XL + orow + q], Ym[inst * 256 + q * 16 + c], s);
      Xm[(orow + r) * XL + ocol + c] = -s;
    }

    // ---------------- 5: 32x32 merge on split-bf16 MFMA (wave 0)
    __syncthreads();
    if (wave == 0) {
      f32x16 y = zero16();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float av[8], bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          av[j] = Lm[(32 + cl) * XL + 16 * ks + 8 * g + j];
          bv[j] = Xm[(16 * ks + 8 * g + j) * XL + cl];
        }
        bf16x8 ah, al, bh, bl;
        split8(av, ah, al);
        split8(bv, bh, bl);
        y = mfma32(al, bh, y);
        y = mfma32(ah, bl, y);
        y = mfma32(ah, bh, y);
      }
      f32x16 z = zero16();
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 bh, bl;
        split_acc_half(y, hh, bh, bl);
        float av[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) av[j] = Xm[(32 + cl) * XL + 32 + kperm(hh, g, j)];
        bf16x8 ah, al;
        split8(av, ah, al);
        z = mfma32(al, bh, z);
        z = mfma32(ah, bl, z);
        z = mfma32(ah, bh, z);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) Xm[(32 + acc_row(q, g)) * XL + cl] = -z[q];
    }

    // ---------------- 6a: split X diag(beta) and X diag(beta r) once (the
    // region of K row-major, L and Y is dead now)
    __syncthreads();
    for (int e = tid; e < C * C / 8; e += NTH) {
      const int row = e / (C / 8), c0 = (e % (C / 8)) * 8;
      float av[8], bv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        av[j] = Xm[row * XL + c0 + j] * gb[c0 + j];
        bv[j] = av[j] * gr[c0 + j];
      }
      bf16x8 h8, l8;
      split8(av, h8, l8);
      *reinterpret_cast<bf16x8*>(Ah + row * AL + c0) = h8;
      *reinterpret_cast<bf16x8*>(Al + row * AL + c0) = l8;
      split8(bv, h8, l8);
      *reinterpret_cast<bf16x8*>(Bh + row * AL + c0) = h8;
      *reinterpret_cast<bf16x8*>(Bl + row * AL + c0) = l8;
    }

    // ---------------- 6b: U = A K -> LDS; seed M with W = A' V (S) or 0
    __syncthreads();
    {
      const int mt = wave / NT, nt = wave % NT;
      f32x16 acc = zero16();
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) {
        const int kc = ks * 16 + 8 * g;
        const bf16x8 ah = lds_load8(Ah + (mt * 32 + cl) * AL + kc);
        const bf16x8 al = lds_load8(Al + (mt * 32 + cl) * AL + kc);
        const bf16x8 kh = lds_load8(Kt + (nt * 32 + cl) * KT + kc);
        acc = mfma32(al, kh, acc);
        acc = mfma32(ah, kh, acc);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = mt * 32 + acc_row(q, g), c = nt * 32 + cl;
        const __bf16 hi = to_bf16(acc[q]);
        Uh[r * ULD + c] = hi;
        Ul[r * ULD + c] = to_bf16(acc[q] - from_bf16(hi));
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 acc = zero16();
      if (s_wave) {
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
          const int kc = ks * 16 + 8 * g;
          const bf16x8 ah = lds_load8(Bh + (mt * 32 + cl) * AL + kc);
          const bf16x8 al = lds_load8(Bl + (mt * 32 + cl) * AL + kc);
          const bf16x8 vh = lds_load8(Vt + (strip * 32 + cl) * KT + kc);
          acc = mfma32(al, vh, acc);
          acc = mfma32(ah, vh, acc);
        }
      }
      P[mt] = acc;
    }

  }

  // ---------------- step 7 of the last chunk
  if (n_chunks > 0) {
    __syncthreads();  // U and K^T of the last chunk complete
    chain_um(0, n_chunks - 1);
    chain_um(1, n_chunks - 1);
    chain_ktm(0, n_chunks - 1);
    chain_ktm(1, n_chunks - 1);
  }

  // ---------------- write the pair
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
  const int ncol = ((tid >> 6) % NT) * 32 + (lane & 31);
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

template <int DP>
hipError_t launch_pipe_t(const BuildArgs& a, hipStream_t s) {
  const int64_t blocks = int64_t(a.n_seg) * a.batch * a.heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(build_dense_pipe_kernel<DP>, dim3(unsigned(blocks)), dim3(4 * DP), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_dense_pipe(const BuildArgs& a, hipStream_t s) {
  const int d = a.dk > a.dv ? a.dk : a.dv;
  if (d <= 32) return launch_pipe_t<32>(a, s);
  if (d <= 64) return launch_pipe_t<64>(a, s);
  return launch_pipe_t<128>(a, s);
}

}  // namespace pic
