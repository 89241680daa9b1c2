// k_compose_seam.hip -- reuse with seam windows.  Along a chain of cached
// pairs, each entry first advances the running state through its seam tokens
// one token at a time, writing o_t = S_t^T q_t after each, and then applies the
// entry's pair:  S <- e^lambda That S + S0  (dense and KDA: split-bf16
// matrix-core products, as in the dense compose; scalar / diagonal: one scale
// per head or per key row).
// [xix.ai HYPIC article (French), paragraph on full-attention layers: the
//  first w tokens (8 by default) of every inner segment are kept out of the
//  cache and recomputed on reuse under the full prefix; the linear layers run
//  the running state through them and pass each token's output to the
//  attention layer above.  Paragraph on linear layers: applying a cached pair
//  left-multiplies the state by T_C and adds S(C|0).]
//
// One workgroup of four waves per (request, layer, head).  Wave w owns columns
// [32w, 32w+32) of the state in 32x32 accumulator layout: lane (g, c) holds
// column 32w + c, rows 32t + 8i + 4g + {0..3} of tile t.  A seam token is a
// rank-one update in fp32 on the vector units:
//   dense     u = S^T k,  S <- a S + k (b (v - a u))^T
//   KDA       u = S^T (a (.) k),  S <- Diag(a) S + k (b (v - u))^T
//   scalar    S <- a S + k v^T
//   diagonal  S <- Diag(a) S + k v^T
// Dense and scalar forms with bf16 inputs take a window of up to eight tokens
// at once (chunked form, products on the matrix cores).  With S0 the state
// before the window, g_t the product of the window's gates up to token t and
// r(t,s) = a_{s+1} ... a_t:
//   S_t = g_t S0 + sum_{s<=t} r(t,s) k_s c_s^T
//   c_t = b_t (v_t - g_t S0^T k_t - sum_{s<t} r(t,s) (k_s . k_t) c_s)   (dense;
//         scalar: c_t = v_t)
//   o_t = g_t S0^T q_t + sum_{s<=t} r(t,s) (k_s . q_t) c_s
// so one product [K; Q] S0 (16 rows, split-bf16 B from the accumulators; k and
// q are exact in bf16) gives every column sum, one product on wave 0 gives the
// 8x8 products k_s . k_t and k_s . q_t, each lane runs the short recurrence for
// its column in fp32, and S <- g S0 + K^T C~ is one more product per tile.
// The diagonal and KDA forms and fp32 inputs update token by token on the
// vector units: a lane holds half of each of its column's rows, so the column sums
// S^T k and S^T q take a partial sum over its 64 rows and one exchange with
// lane l ^ 32.  Seam tokens are staged in LDS eight at a time, zero padded to
// 128 channels.  The
// first eight tokens of the next entry's window are loaded into registers as
// soon as the current window is staged (one 8- or 16-byte piece of k, q and v
// per thread, token indices clamped into the call's range so that no load is
// conditional), so they arrive while the current tokens and pair are applied.
#include <type_traits>

#include "mfma_util.hpp"
#include "pic_internal.hpp"

namespace pic {
namespace {

constexpr int SP = 128;        // padded head size (state rows and columns)
constexpr int SNT = SP / 32;   // 32-row tiles of a column strip
constexpr int STW = 8;         // seam tokens staged per round
constexpr int SLDR = SP + 8;   // row stride of the staged operator (bf16)

// FULL: dk = dv = 128, so every operator, S0 and state access is an
// unconditional load at a loop-invariant offset from the step's base address
// INL: the chain and seam tables travel in the kernel arguments
// a workgroup barrier that no instruction is scheduled across (the
// compiler otherwise moves register-only products into the next phase)
__device__ __forceinline__ void seam_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

template <int FORM, bool BF16, bool FULL, bool INL>
__global__ __launch_bounds__(256) void compose_seam_kernel(SeamArgs sa) {
  constexpr bool TH = FORM == kDense || FORM == kKda;   // pairs carry That
  constexpr bool PCG = FORM == kDiag || FORM == kKda;   // a gate per key channel
  constexpr bool ERASE = FORM == kDense || FORM == kKda;  // beta and the erase
  __shared__ __attribute__((aligned(16))) __bf16 th_hi[TH ? SP * SLDR : 8];
  __shared__ __attribute__((aligned(16))) __bf16 th_lo[TH ? SP * SLDR : 8];
  // window path: dense / scalar forms with bf16 inputs
  constexpr bool WIN = BF16 && (FORM == kDense || FORM == kScalar);
  __shared__ __attribute__((aligned(16))) float sk[WIN ? 1 : STW][SP];
  __shared__ __attribute__((aligned(16))) float sq[WIN ? 1 : STW][SP];
  __shared__ __attribute__((aligned(16))) __bf16 skb[WIN ? STW : 1][SP];   // k rows
  __shared__ __attribute__((aligned(16))) __bf16 sqb[WIN ? STW : 1][SP];   // q rows
  __shared__ __attribute__((aligned(16))) __bf16 skT[WIN ? SP : 1][STW];   // k columns
  __shared__ __attribute__((aligned(16))) float skk[WIN ? 2 * STW : 1][STW];  // k.k, q.k
  __shared__ __attribute__((aligned(16))) float sv[STW][SP];
  __shared__ __attribute__((aligned(16))) float sg[STW][PCG ? SP : 4];  // gates
  __shared__ float sb[STW];                                                       // beta

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int dk = FULL ? SP : sa.c.dk, dv = FULL ? SP : sa.c.dv, H = sa.c.heads;
  const int64_t BH = int64_t(sa.c.batch) * H;
  const int64_t unit = blockIdx.x;
  const int64_t r = unit / BH, bh = unit % BH;
  const int b = int(bh / H), h = int(bh % H);
  const int n = wave * 32 + (lane & 31);  // state column of this lane
  const bool ncol = FULL || n < dv;
  const int64_t sdd = int64_t(dk) * dv;
  const int64_t NS = sa.n_seam;

  f32x16 S[SNT];
#pragma unroll
  for (int t = 0; t < SNT; ++t)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = t * 32 + acc_row(q, g);
      S[t][q] = (sa.c.S_in && (FULL || (ncol && row < dk))) ? sa.c.S_in[unit * sdd + int64_t(row) * dv + n] : 0.f;
    }

  // operator of one chain step (dense), this thread's float4 items, zero padded
  float4 pre[16];
  auto load_op = [&](int64_t pu) {
    const float* Tp = sa.c.pool_T_hat + pu * int64_t(dk) * dk;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int e = threadIdx.x + it * 256;
      const int row = (e * 4) / SP, col = (e * 4) % SP;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (FULL || (row < dk && col < dk)) x = *reinterpret_cast<const float4*>(Tp + row * dk + col);
      pre[it] = x;
    }
  };

  // One round of up to STW seam tokens in registers: thread e holds channels
  // 4 (e % 32) .. +3 of token e / 32 of k, q and v (and of the diagonal gates);
  // threads 0 .. STW-1 hold the scalar gate and beta of token e.
  const int rt = threadIdx.x >> 5, rc = 4 * (threadIdx.x & 31);
  typedef typename std::conditional<BF16, uint2, float4>::type Piece;
  Piece pk, pq, pv;
  float4 pa = make_float4(1.f, 1.f, 1.f, 1.f);
  float pa1 = 1.f, pb1 = 1.f;
  auto piece = [&](const void* base, int64_t off) -> Piece {
    if constexpr (BF16)
      return *reinterpret_cast<const uint2*>(static_cast<const __bf16*>(base) + off);
    else
      return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
  };
  // load the round starting at seam token t0 (tokens past the call's end are
  // clamped to its last one; they are loaded but never used)
  auto load_round = [&](int64_t t0) {
    const int64_t tl = t0 + rt < NS ? t0 + rt : NS - 1;
    const int64_t tok = (int64_t(b) * NS + tl) * H + h;
    const int ck = rc < dk ? rc : 0, cv = rc < dv ? rc : 0;
    pk = piece(sa.k, tok * dk + ck);
    pq = piece(sa.q, tok * dk + ck);
    pv = piece(sa.v, tok * dv + cv);
    if (PCG) pa = *reinterpret_cast<const float4*>(sa.alpha + tok * dk + ck);
    if (FORM != kDiag) {
      const int64_t ts = t0 + (threadIdx.x & (STW - 1)) < NS ? t0 + (threadIdx.x & (STW - 1)) : NS - 1;
      const int64_t tk = (int64_t(b) * NS + ts) * H + h;
      if (!PCG) pa1 = sa.alpha[tk];
      if (ERASE && sa.beta) pb1 = sa.beta[tk];
    }
  };
  auto as4 = [&](const Piece& x) -> float4 {
    if constexpr (BF16)
      return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                         __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
    else
      return x;
  };
  // write the round held in registers to LDS (zero padded past dk / dv)
  auto store_round = [&]() {
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (WIN) {
      const uint2 kz = rc < dk ? pk : make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(&skb[rt][rc]) = kz;
      *reinterpret_cast<uint2*>(&sqb[rt][rc]) = rc < dk ? pq : make_uint2(0u, 0u);
      const unsigned short* kh = reinterpret_cast<const unsigned short*>(&kz);
#pragma unroll
      for (int j = 0; j < 4; ++j) reinterpret_cast<unsigned short*>(&skT[rc + j][0])[rt] = kh[j];
    } else {
      *reinterpret_cast<float4*>(&sk[rt][rc]) = rc < dk ? as4(pk) : z;
      *reinterpret_cast<float4*>(&sq[rt][rc]) = rc < dk ? as4(pq) : z;
    }
    *reinterpret_cast<float4*>(&sv[rt][rc]) = rc < dv ? as4(pv) : z;
    if (PCG)
      *reinterpret_cast<float4*>(&sg[rt][rc]) = rc < dk ? pa : make_float4(1.f, 1.f, 1.f, 1.f);
    if (FORM != kDiag && threadIdx.x < STW) {
      if (!PCG) sg[threadIdx.x][0] = pa1;
      sb[threadIdx.x] = pb1;
    }
  };

  // one seam token (staged slot tt, seam token index t): update, then readout
  auto token = [&](int tt, int64_t t) {
    if constexpr (FORM == kKda) {
      // the rows decay by their own gates before the erase reads them; the
      // key is read from LDS on both passes (no register copy of it)
      const float vn = sv[tt][n];
      float up[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 k4 = *reinterpret_cast<const float4*>(&sk[tt][32 * t4 + 8 * i + 4 * g]);
          const float4 a4 = *reinterpret_cast<const float4*>(&sg[tt][32 * t4 + 8 * i + 4 * g]);
          const float kv[4] = {k4.x, k4.y, k4.z, k4.w}, av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            S[t4][4 * i + e] *= av[e];
            up[e] = fmaf(kv[e], S[t4][4 * i + e], up[e]);
          }
        }
      float u = (up[0] + up[1]) + (up[2] + up[3]);
      u += __shfl_xor(u, 32);
      const float cc = sb[tt] * (vn - u);
#pragma unroll
      for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 k4 = *reinterpret_cast<const float4*>(&sk[tt][32 * t4 + 8 * i + 4 * g]);
          S[t4][4 * i + 0] = fmaf(k4.x, cc, S[t4][4 * i + 0]);
          S[t4][4 * i + 1] = fmaf(k4.y, cc, S[t4][4 * i + 1]);
          S[t4][4 * i + 2] = fmaf(k4.z, cc, S[t4][4 * i + 2]);
          S[t4][4 * i + 3] = fmaf(k4.w, cc, S[t4][4 * i + 3]);
        }
    } else {
    float kr[SNT][16];
#pragma unroll
    for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(&sk[tt][32 * t4 + 8 * i + 4 * g]);
        kr[t4][4 * i] = x.x; kr[t4][4 * i + 1] = x.y; kr[t4][4 * i + 2] = x.z; kr[t4][4 * i + 3] = x.w;
      }
    const float vn = sv[tt][n];
    if (FORM == kDense) {
      float up[4] = {0.f, 0.f, 0.f, 0.f};  // independent partial sums
#pragma unroll
      for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
        for (int q = 0; q < 16; ++q) up[q & 3] = fmaf(kr[t4][q], S[t4][q], up[q & 3]);
      float u = (up[0] + up[1]) + (up[2] + up[3]);
      u += __shfl_xor(u, 32);
      const float a = sg[tt][0];
      const float cc = sb[tt] * (vn - a * u);
#pragma unroll
      for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
        for (int q = 0; q < 16; ++q) S[t4][q] = fmaf(kr[t4][q], cc, a * S[t4][q]);
    } else if (FORM == kScalar) {
      const float a = sg[tt][0];
#pragma unroll
      for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
        for (int q = 0; q < 16; ++q) S[t4][q] = fmaf(kr[t4][q], vn, a * S[t4][q]);
    } else {
#pragma unroll
      for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 ga = *reinterpret_cast<const float4*>(&sg[tt][32 * t4 + 8 * i + 4 * g]);
          const float gv[4] = {ga.x, ga.y, ga.z, ga.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            S[t4][4 * i + e] = fmaf(kr[t4][4 * i + e], vn, gv[e] * S[t4][4 * i + e]);
        }
    }
    }
    float op[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(&sq[tt][32 * t4 + 8 * i + 4 * g]);
        op[0] = fmaf(x.x, S[t4][4 * i], op[0]);
        op[1] = fmaf(x.y, S[t4][4 * i + 1], op[1]);
        op[2] = fmaf(x.z, S[t4][4 * i + 2], op[2]);
        op[3] = fmaf(x.w, S[t4][4 * i + 3], op[3]);
      }
    float o = (op[0] + op[1]) + (op[2] + op[3]);
    o += __shfl_xor(o, 32);
    if (g == 0 && ncol) sa.O[((int64_t(b) * NS + t) * H + h) * dv + n] = o;
  };

  // the m (<= STW) tokens staged in LDS, from seam token t_lo, in chunked form
  auto window = [&](int m, int64_t t_lo) {
    const int cl = lane & 31;
    // A rows: k_0..k_7, q_0..q_7, then copies of k rows (finite, unused)
    const __bf16* arow = cl < STW ? skb[cl] : (cl < 2 * STW ? sqb[cl - STW] : skb[cl & (STW - 1)]);
    if (wave == 0) {  // k_s . k_t (rows 0..7) and q_t . k_s (rows 8..15), column s or t
      const __bf16* brow = skb[cl & (STW - 1)];
      f32x16 gacc = zero16();
#pragma unroll
      for (int ks = 0; ks < SP / 16; ++ks)
        gacc = mfma32(lds_load8(arow + 16 * ks + 8 * g), lds_load8(brow + 16 * ks + 8 * g), gacc);
      if (cl < STW) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          skk[4 * g + e][cl] = gacc[e];
          skk[STW + 4 * g + e][cl] = gacc[4 + e];
        }
      }
    }
    // column sums S0^T k_t (rows 0..7) and S0^T q_t (rows 8..15) of this
    // lane's column; the B operand comes from the accumulators (permuted K)
    f32x16 racc = zero16();
#pragma unroll
    for (int t4 = 0; t4 < SNT; ++t4)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 bhi, blo;
        split_acc_half(S[t4], hh, bhi, blo);
        const bf16x8 af = lds_perm8(arow, 32 * t4 + 16 * hh + 4 * g);
        racc = mfma32(af, bhi, racc);
        racc = mfma32(af, blo, racc);
      }
    // lane half g holds tokens 4g .. 4g+3; take the other half's from l ^ 32
    float a[STW], bq[STW];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float xa = __shfl_xor(racc[e], 32), xb = __shfl_xor(racc[4 + e], 32);
      a[e] = g ? xa : racc[e];
      a[4 + e] = g ? racc[e] : xa;
      bq[e] = g ? xb : racc[4 + e];
      bq[4 + e] = g ? racc[4 + e] : xb;
    }
    seam_barrier();  // the 8x8 products are in LDS
    float al[STW], cc[STW];
#pragma unroll
    for (int t = 0; t < STW; ++t) al[t] = sg[t][0];
    float gt = 1.f;
#pragma unroll
    for (int t = 0; t < STW; ++t) {
      cc[t] = 0.f;
      if (t < m) {
        gt *= al[t];
        float kk[STW], qk[STW];
#pragma unroll
        for (int s4 = 0; s4 < STW / 4; ++s4) {
          const float4 x = *reinterpret_cast<const float4*>(&skk[t][4 * s4]);
          const float4 y = *reinterpret_cast<const float4*>(&skk[STW + t][4 * s4]);
          kk[4 * s4] = x.x; kk[4 * s4 + 1] = x.y; kk[4 * s4 + 2] = x.z; kk[4 * s4 + 3] = x.w;
          qk[4 * s4] = y.x; qk[4 * s4 + 1] = y.y; qk[4 * s4 + 2] = y.z; qk[4 * s4 + 3] = y.w;
        }
        const float vt = sv[t][n];
        if (FORM == kDense) {
          float acc = 0.f, rr = 1.f;
#pragma unroll
          for (int s = t - 1; s >= 0; --s) {
            rr *= al[s + 1];
            acc = fmaf(rr * kk[s], cc[s], acc);
          }
          cc[t] = sb[t] * (vt - gt * a[t] - acc);
        } else {
          cc[t] = vt;
        }
        float o = fmaf(qk[t], cc[t], gt * bq[t]);
        float rr = 1.f;
#pragma unroll
        for (int s = t - 1; s >= 0; --s) {
          rr *= al[s + 1];
          o = fmaf(rr * qk[s], cc[s], o);
        }
        if (g == 0 && ncol) sa.O[((int64_t(b) * NS + t_lo + t) * H + h) * dv + n] = o;
      }
    }
    // S <- g S0 + sum_s r(m-1, s) k_s c_s^T: scale, then K^T C~ per row tile
    float ct[STW];
    float rr = 1.f;
#pragma unroll
    for (int s = STW - 1; s >= 0; --s) {
      ct[s] = 0.f;
      if (s < m) {
        ct[s] = rr * cc[s];
        rr *= al[s];
      }
    }
#pragma unroll
    for (int t4 = 0; t4 < SNT; ++t4) S[t4] *= gt;
    bf16x8 chi, clo;
    split8(ct, chi, clo);
    if (g) {  // tokens 8..15 of the K step are zero
#pragma unroll
      for (int j = 0; j < 8; ++j) { chi[j] = __bf16(0.f); clo[j] = __bf16(0.f); }
    }
#pragma unroll
    for (int t4 = 0; t4 < SNT; ++t4) {
      bf16x8 kt = lds_load8(&skT[32 * t4 + cl][0]);
      if (g) {
#pragma unroll
        for (int j = 0; j < 8; ++j) kt[j] = __bf16(0.f);
      }
      S[t4] = mfma32(kt, chi, S[t4]);
      S[t4] = mfma32(kt, clo, S[t4]);
    }
  };

  const int64_t c0 = chain_offset_t<INL>(sa.c, r), c1 = chain_offset_t<INL>(sa.c, r + 1);
  // The chain's pool indices, log scales (scalar / dense) and window bounds,
  // 64 entries at a time, one per lane (vector loads); a step takes its own
  // with readlane, so no step issues a scalar or table load (those share the
  // LDS wait counter and would hold up the next barrier for a memory round
  // trip).
  int64_t cb = c0;
  int ent_l = 0;
  float lam_l = 0.f;
  int64_t so0_l = 0, so1_l = 0;
  auto fetch = [&](int64_t base) {
    cb = base;
    const int64_t cc = base + lane;
    int e = 0;
    float l = 0.f;
    int64_t x0 = 0, x1 = 0;
    if (cc < c1) {
      e = chain_entry_t<INL>(sa.c, cc);
      if (FORM != kDiag) l = table_at(sa.c.pool_log_scale, int64_t(e) * BH + bh);
      x0 = seam_offset_t<INL>(sa, cc);
      x1 = seam_offset_t<INL>(sa, cc + 1);
    }
    ent_l = e;
    lam_l = l;
    so0_l = x0;
    so1_l = x1;
  };
  auto rl64 = [&](int64_t x, int64_t c) {
    const int i = int(c - cb);
    const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(x)), i));
    const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint64_t(x) >> 32), i));
    return int64_t((uint64_t(hi) << 32) | lo);
  };
  auto entry_at = [&](int64_t c) { return __builtin_amdgcn_readlane(ent_l, int(c - cb)); };
  const bool seams = NS > 0;
  if (c0 < c1) {
    fetch(c0);
    if (TH) load_op(int64_t(entry_at(c0)) * BH + bh);
    if (seams) load_round(rl64(so0_l, c0));
  }
  // One chain step: after a barrier the entry's operator (dense) and the first
  // round of its window go to LDS and the next operator and window are
  // loaded (they arrive while this step's window and product run); after a
  // second barrier the window, then the pair.
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t pu = int64_t(entry_at(c)) * BH + bh;
    const float lam = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam_l), int(c - cb)));
    const int64_t t_lo = rl64(so0_l, c), t_hi = rl64(so1_l, c);
    const bool next = seams && c + 1 < c1;
    if (c + 1 < c1 && c + 1 - cb >= 64) fetch(c + 1);  // entries c+1 .. c+64
    const bool win = t_hi > t_lo, one_round = t_hi - t_lo <= STW;
    seam_barrier();  // the previous step's operator and tokens are no longer read
    if (TH) {
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int e = threadIdx.x + it * 256;
        const int row = (e * 4) / SP, col = (e * 4) % SP;
        unsigned h0, l0, h1, l1;
        split2(pre[it].x, pre[it].y, h0, l0);
        split2(pre[it].z, pre[it].w, h1, l1);
        // columns permuted within each 16 (bits 2 and 3 swapped) so that the
        // 8 columns of a permuted K-step are contiguous
        const int pcol = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
        *reinterpret_cast<uint2*>(th_hi + row * SLDR + pcol) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(th_lo + row * SLDR + pcol) = make_uint2(l0, l1);
      }
      if (c + 1 < c1) load_op(int64_t(entry_at(c + 1)) * BH + bh);
    }
    if (win) store_round();  // the window's first round was loaded ahead
    if (next && (!win || one_round)) load_round(t_hi);
    seam_barrier();
    if (win) {
      const int m0 = int(one_round ? t_hi - t_lo : STW);
      if constexpr (WIN) {
        window(m0, t_lo);
      } else if constexpr (FORM == kKda) {
#pragma unroll 1
        for (int tt = 0; tt < m0; ++tt) token(tt, t_lo + tt);
      } else {
#pragma unroll
        for (int tt = 0; tt < STW; ++tt)  // unrolled, so that reads run ahead
          if (tt < m0) token(tt, t_lo + tt);
      }
      for (int64_t t0 = t_lo + STW; t0 < t_hi; t0 += STW) {  // windows longer than a round
        const int m = int(t_hi - t0 < STW ? t_hi - t0 : STW);
        load_round(t0);
        seam_barrier();
        store_round();
        seam_barrier();
        if constexpr (WIN)
          window(m, t0);
        else
          for (int tt = 0; tt < m; ++tt) token(tt, t0 + tt);
      }
      if (!one_round && next) load_round(t_hi);
    }
    // then the entry's pair (its operator is in LDS)
    const float* S0p = sa.c.pool_S0 + pu * sdd;
    if (TH) {
      f32x16 s0[SNT];
#pragma unroll
      for (int t = 0; t < SNT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = t * 32 + acc_row(q, g);
          s0[t][q] = (FULL || (ncol && row < dk)) ? S0p[int64_t(row) * dv + n] : 0.f;
        }
      const float scale = expf(lam);
      f32x16 acc[SNT];
#pragma unroll
      for (int t = 0; t < SNT; ++t) acc[t] = zero16();
#pragma unroll
      for (int ks = 0; ks < 2 * SNT; ++ks) {
        const int t = ks >> 1, hh = ks & 1;
        bf16x8 bhi, blo;
        split_acc_half(S[t], hh, bhi, blo);
        const int kc = 32 * t + 16 * hh + 8 * g;
#pragma unroll
        for (int mt = 0; mt < SNT; ++mt) {
          const int arow = mt * 32 + (lane & 31);
          const bf16x8 ahi = lds_load8(th_hi + arow * SLDR + kc);
          const bf16x8 alo = lds_load8(th_lo + arow * SLDR + kc);
          acc[mt] = mfma32(alo, bhi, acc[mt]);
          acc[mt] = mfma32(ahi, blo, acc[mt]);
          acc[mt] = mfma32(ahi, bhi, acc[mt]);
        }
      }
#pragma unroll
      for (int t = 0; t < SNT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) S[t][q] = fmaf(scale, acc[t][q], s0[t][q]);
    } else {
      const float sc = (FORM == kScalar) ? expf(lam) : 1.f;
      // S0 one row tile at a time, the next tile's loads issued before this
      // tile's products (left to itself the compiler waited for each load)
      auto s0_tile = [&](int t) __attribute__((always_inline)) {
        f32x16 x;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = t * 32 + acc_row(q, g);
          x[q] = (FULL || (ncol && row < dk)) ? S0p[int64_t(row) * dv + n] : 0.f;
        }
        return x;
      };
      f32x16 nxt = s0_tile(0);
#pragma unroll
      for (int t = 0; t < SNT; ++t) {
        const f32x16 cur = nxt;
        if (t + 1 < SNT) nxt = s0_tile(t + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = t * 32 + acc_row(q, g);
          const float rs = (FORM == kDiag) ? (row < dk ? expf(sa.c.pool_log_scale[pu * dk + row]) : 1.f) : sc;
          S[t][q] = fmaf(rs, S[t][q], cur[q]);
        }
      }
    }
  }

  if (ncol) {
#pragma unroll
    for (int t = 0; t < SNT; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = t * 32 + acc_row(q, g);
        if (FULL || row < dk) sa.c.S_out[unit * sdd + int64_t(row) * dv + n] = S[t][q];
      }
  }
}

template <int FORM, bool BF16, bool INL>
void launch_seam_i(const SeamArgs& a, dim3 grid, hipStream_t s) {
  if (a.c.dk == SP && a.c.dv == SP)
    hipLaunchKernelGGL((compose_seam_kernel<FORM, BF16, true, INL>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((compose_seam_kernel<FORM, BF16, false, INL>), grid, dim3(256), 0, s, a);
}
template <int FORM, bool BF16>
void launch_seam_f(const SeamArgs& a, dim3 grid, hipStream_t s) {
  if (a.c.inl)
    launch_seam_i<FORM, BF16, true>(a, grid, s);
  else
    launch_seam_i<FORM, BF16, false>(a, grid, s);
}

template <int FORM>
void launch_seam_t(const SeamArgs& a, dim3 grid, hipStream_t s) {
  if (a.qkv_bf16)
    launch_seam_f<FORM, true>(a, grid, s);
  else
    launch_seam_f<FORM, false>(a, grid, s);
}

}  // namespace

hipError_t launch_compose_seams(const SeamArgs& a, hipStream_t s) {
  const int64_t units = int64_t(a.c.n_req) * a.c.batch * a.c.heads;
  if (units <= 0) return hipSuccess;
  if (units > 0x7fffffffLL || a.c.dk > SP || a.c.dv > SP) return hipErrorInvalidConfiguration;
  const dim3 grid{unsigned(units), 1, 1};
  switch (a.c.form) {
    case kScalar: launch_seam_t<kScalar>(a, grid, s); break;
    case kDiag: launch_seam_t<kDiag>(a, grid, s); break;
    case kDense: launch_seam_t<kDense>(a, grid, s); break;
    case kKda: launch_seam_t<kKda>(a, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pic
