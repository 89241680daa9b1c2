// k_compose.hip -- reuse-time kernels of the segment transform:
//   * dense compose      S <- e^lambda_p * That_p * S + S0_p along a chain,
//                        one 128x128x128 split-bf16 MFMA product per step;
//   * elementwise compose (scalar / diagonal forms)  S <- e^lambda_p (.) S + S0_p;
//   * naive add          S <- S + S0_p (the ablation);
//   * materialize        plain fp32 T_C = e^lambda That.
// [xix.ai HYPIC article (French), paragraph on linear layers: reuse of a cached
//  segment left-multiplies the running state by T_C and adds S(C|0), in time
//  independent of the segment's length; plain addition omits T.]
#include <algorithm>
#include "mfma_util.hpp"
#include "pic_internal.hpp"

namespace pic {
namespace {

// ---------------------------------------------------------------------------
// elementwise compose / naive add
// ---------------------------------------------------------------------------
// One thread owns 4 consecutive state elements (a float4 inside one row) of
// one chain unit (request, layer, head) and walks the chain; 256 threads per
// block, blocks_per_unit blocks per unit.  All loads are 16-byte coalesced.
constexpr int kElemThreads = 256;

template <bool NAIVE, bool DIAG>
__global__ __launch_bounds__(kElemThreads) void compose_elem_kernel(ComposeArgs a,
                                                                    int blocks_per_unit) {
  const int64_t BH = int64_t(a.batch) * a.heads;
  const int nelem4 = a.dk * a.dv / 4;
  const int64_t unit = blockIdx.x / blocks_per_unit;
  const int e4 = (blockIdx.x % blocks_per_unit) * kElemThreads + threadIdx.x;
  if (e4 >= nelem4) return;
  const int64_t r = unit / BH, bh = unit % BH;
  const int row = (e4 * 4) / a.dv;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (a.S_in) s = reinterpret_cast<const float4*>(a.S_in)[unit * nelem4 + e4];
  const float4* S0 = reinterpret_cast<const float4*>(a.pool_S0);
  const int64_t c0 = chain_offset(a, r), c1 = chain_offset(a, r + 1);
  int64_t c = c0;
  // four steps at a time: issue the loads together, then fold in order
  for (; c + 4 <= c1; c += 4) {
    float4 x[4];
    float sc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t pu = int64_t(chain_entry(a, c + u)) * BH + bh;
      x[u] = S0[pu * nelem4 + e4];
      if (!NAIVE) sc[u] = DIAG ? a.pool_log_scale[pu * a.dk + row] : a.pool_log_scale[pu];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (NAIVE) {
        s.x += x[u].x; s.y += x[u].y; s.z += x[u].z; s.w += x[u].w;
      } else {
        const float t = expf(sc[u]);
        s.x = fmaf(t, s.x, x[u].x); s.y = fmaf(t, s.y, x[u].y);
        s.z = fmaf(t, s.z, x[u].z); s.w = fmaf(t, s.w, x[u].w);
      }
    }
  }
  for (; c < c1; ++c) {
    const int64_t pu = int64_t(chain_entry(a, c)) * BH + bh;
    const float4 x = S0[pu * nelem4 + e4];
    if (NAIVE) {
      s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
    } else {
      const float t = expf(DIAG ? a.pool_log_scale[pu * a.dk + row] : a.pool_log_scale[pu]);
      s.x = fmaf(t, s.x, x.x); s.y = fmaf(t, s.y, x.y);
      s.z = fmaf(t, s.z, x.z); s.w = fmaf(t, s.w, x.w);
    }
  }
  reinterpret_cast<float4*>(a.S_out)[unit * nelem4 + e4] = s;
}

// ---------------------------------------------------------------------------
// dense compose
// ---------------------------------------------------------------------------
// One workgroup per chain unit (request, layer, head).  Wave w owns columns
// [32w, 32w+32) of the running state S (dk x dv) in MFMA accumulators, as
// DKP/32 row tiles.  Each chain step stages That_p in LDS as hi/lo bf16 rows
// (padded stride to spread LDS banks; columns stored in the permuted K order
// of the products) and forms That_p * S with split-bf16
// MFMAs (3 per 32x32x16 block), taking the B operand straight from the
// accumulators of the old S (K order permuted to match, see mfma_util.hpp).
// Then S <- e^lambda * (That S) + S0_p.  The next step's operator is loaded
// into registers while the current step's MFMAs run, and S0_p is loaded
// before them.  Sizes not a multiple of 32 are zero-padded, which leaves the
// result unchanged.
// PROD = true forms the chain's operator instead: the "state" is dk x dk,
// starts at I, and each step is X <- That_p X (no scale, no additive term);
// the launcher passes dv = dk and S_out = the That output.
// FULL = true when dk = dv = DKP: no padding, so every operator and S0
// access is an unconditional load at a loop-invariant offset from the step's
// (uniform) base address.
// INL: the chain tables travel in the kernel arguments
template <int DKP, bool PROD, bool FULL, bool INL>
__global__ __launch_bounds__(256) void compose_dense_kernel(ComposeArgs a) {
  constexpr int NT = DKP / 32;
  // row stride of the staged operator (bf16): 16-byte aligned rows whose
  // 16-byte reads from 32 consecutive rows spread evenly over the banks
  constexpr int LDR = DKP + 8;
  constexpr int F4 = DKP * DKP / 4;   // float4 items of one operator
  __shared__ __attribute__((aligned(16))) __bf16 th_hi[DKP * LDR];
  __shared__ __attribute__((aligned(16))) __bf16 th_lo[DKP * LDR];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, cl = lane & 31;
  // with FULL the block is 64 * DKP / 32 threads (one wave per 32 columns)
  const int nthr = FULL ? 64 * NT : int(blockDim.x);
  const int dk = a.dk, dv = a.dv;
  const int64_t BH = int64_t(a.batch) * a.heads;
  const int64_t unit = blockIdx.x;
  const int64_t r = unit / BH, bh = unit % BH;
  const int n = wave * 32 + cl;  // state column of this lane
  const bool ncol = FULL || n < dv;
  const int64_t sdd = int64_t(dk) * dv;
  const int per_thr = (F4 + nthr - 1) / nthr;  // <= 16: the launcher gives >= F4 / 16 threads

  f32x16 S[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = t * 32 + acc_row(q, g);
      if (PROD)
        S[t][q] = (row == n && row < dk) ? 1.f : 0.f;
      else
        S[t][q] = (a.S_in && ncol && (FULL || row < dk)) ? a.S_in[unit * sdd + int64_t(row) * dv + n] : 0.f;
    }
  }

  // operator of one chain step, as this thread's float4 items (zero padded)
  float4 pre[16];
  auto load_op = [&](int64_t pu) {
    const float* Tp = a.pool_T_hat + pu * int64_t(dk) * dk;
    if (FULL) {
      // item e is float4 e of the row-major operator
#pragma unroll
      for (int it = 0; it < 16; ++it)
        if (it < per_thr) pre[it] = reinterpret_cast<const float4*>(Tp)[threadIdx.x + it * nthr];
      return;
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int e = threadIdx.x + it * nthr;
      const int row = (e * 4) / DKP, col = (e * 4) % DKP;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (it < per_thr && e < F4 && row < dk && col < dk)
        x = *reinterpret_cast<const float4*>(Tp + row * dk + col);
      pre[it] = x;
    }
  };

  const int64_t c0 = chain_offset_t<INL>(a, r), c1 = chain_offset_t<INL>(a, r + 1);
  // The chain's pool indices and log scales, 64 entries at a time, one per
  // lane (one vector load each); a step takes its own with readlane, so no
  // step issues a scalar or table load (those share the LDS wait counter and
  // would hold up the next barrier for a memory round trip).
  int64_t cb = c0;
  int ent_l = 0;
  float lam_l = 0.f;
  auto fetch = [&](int64_t base) {
    cb = base;
    const int64_t cc = base + lane;
    int e = 0;
    float l = 0.f;
    if (cc < c1) {
      e = chain_entry_t<INL>(a, cc);
      if (!PROD) l = table_at(a.pool_log_scale, int64_t(e) * BH + bh);
    }
    ent_l = e;
    lam_l = l;
  };
  auto entry_at = [&](int64_t c) { return __builtin_amdgcn_readlane(ent_l, int(c - cb)); };
  if (c0 < c1) {
    fetch(c0);
    load_op(int64_t(entry_at(c0)) * BH + bh);
  }
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t pu = int64_t(entry_at(c)) * BH + bh;
    const float lam = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam_l), int(c - cb)));
    __syncthreads();  // every wave is done reading the previous operator
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int e = threadIdx.x + it * nthr;
      if (it < per_thr && (FULL || e < F4)) {
        const int row = (e * 4) / DKP, col = (e * 4) % DKP;
        unsigned h0, l0, h1, l1;
        split2(pre[it].x, pre[it].y, h0, l0);
        split2(pre[it].z, pre[it].w, h1, l1);
        // column positions permuted within each 16 (bits 2 and 3 swapped), so
        // that the 8 columns of a permuted K-step are contiguous
        const int pcol = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
        *reinterpret_cast<uint2*>(th_hi + row * LDR + pcol) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(th_lo + row * LDR + pcol) = make_uint2(l0, l1);
      }
    }
    if (c + 1 < c1) {
      if (c + 1 - cb >= 64) fetch(c + 1);
      load_op(int64_t(entry_at(c + 1)) * BH + bh);
    }
    // this step's S0 strip, loaded ahead of the products
    f32x16 s0[NT];
    float scale = 1.f;
    if (!PROD) {
      const float* S0p = a.pool_S0 + pu * sdd;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = t * 32 + acc_row(q, g);
          if (FULL)
            s0[t][q] = S0p[row * DKP + n];
          else
            s0[t][q] = (ncol && row < dk) ? S0p[int64_t(row) * dv + n] : 0.f;
        }
      scale = expf(lam);
    }
    __syncthreads();

    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = zero16();
#pragma unroll
    for (int ks = 0; ks < 2 * NT; ++ks) {
      const int t = ks >> 1, h = ks & 1;
      bf16x8 bhi, blo;
      split_acc_half(S[t], h, bhi, blo);
      // K indices kperm(h, g, 0..7) sit at positions 16h + 8g .. +7
      const int kc = 32 * t + 16 * h + 8 * g;
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const int arow = mt * 32 + cl;
        const bf16x8 ahi = lds_load8(th_hi + arow * LDR + kc);
        const bf16x8 alo = lds_load8(th_lo + arow * LDR + kc);
        acc[mt] = mfma32(alo, bhi, acc[mt]);
        acc[mt] = mfma32(ahi, blo, acc[mt]);
        acc[mt] = mfma32(ahi, bhi, acc[mt]);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) S[t][q] = PROD ? acc[t][q] : fmaf(scale, acc[t][q], s0[t][q]);
  }

  if (ncol) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = t * 32 + acc_row(q, g);
        if (FULL || row < dk) a.S_out[unit * sdd + int64_t(row) * dv + n] = S[t][q];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// chain pair: log scale of the chain = sum of the entries' log scales
// ---------------------------------------------------------------------------
// One thread per (request, layer, head[, key channel]); consecutive threads
// read consecutive entries of each pool row.
__global__ void chain_log_scale_kernel(ComposeArgs a, int per) {
  const int64_t BH = int64_t(a.batch) * a.heads;
  const int64_t total = int64_t(a.n_req) * BH * per;
  const int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (e >= total) return;
  const int64_t r = e / (BH * per), rest = e % (BH * per);
  float acc = 0.f;
  for (int64_t c = chain_offset(a, r); c < chain_offset(a, r + 1); ++c)
    acc += a.pool_log_scale[int64_t(chain_entry(a, c)) * BH * per + rest];
  a.log_scale_out[e] = acc;
}

// ---------------------------------------------------------------------------
// plain operator
// ---------------------------------------------------------------------------
__global__ void materialize_kernel(int form, int64_t n_units, int dk, const float* log_scale,
                                   const float* T_hat, float* T_out) {
  const int64_t total = n_units * dk * dk;
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < total;
       e += int64_t(gridDim.x) * blockDim.x) {
    const int64_t u = e / (int64_t(dk) * dk);
    const int i = int((e / dk) % dk), j = int(e % dk);
    float v;
    if (form == kDense || form == kKda) {
      v = expf(log_scale[u]) * T_hat[e];
    } else if (form == kScalar) {
      v = (i == j) ? expf(log_scale[u]) : 0.f;
    } else {
      v = (i == j) ? expf(log_scale[u * dk + i]) : 0.f;
    }
    T_out[e] = v;
  }
}

}  // namespace

hipError_t launch_compose_elementwise(const ComposeArgs& a, bool naive, hipStream_t s) {
  const int nelem4 = a.dk * a.dv / 4;
  const int bpu = (nelem4 + kElemThreads - 1) / kElemThreads;
  const int64_t units = int64_t(a.n_req) * a.batch * a.heads;
  const int64_t blocks = units * bpu;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (naive)
    hipLaunchKernelGGL((compose_elem_kernel<true, false>), dim3(unsigned(blocks)),
                       dim3(kElemThreads), 0, s, a, bpu);
  else if (a.form == kDiag)
    hipLaunchKernelGGL((compose_elem_kernel<false, true>), dim3(unsigned(blocks)),
                       dim3(kElemThreads), 0, s, a, bpu);
  else
    hipLaunchKernelGGL((compose_elem_kernel<false, false>), dim3(unsigned(blocks)),
                       dim3(kElemThreads), 0, s, a, bpu);
  return hipGetLastError();
}

template <int DKP, bool PROD, bool INL>
void launch_dense_i(const ComposeArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.dk == DKP && a.dv == DKP)
    hipLaunchKernelGGL((compose_dense_kernel<DKP, PROD, true, INL>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((compose_dense_kernel<DKP, PROD, false, INL>), grid, block, 0, s, a);
}
template <int DKP, bool PROD>
void launch_dense_t(const ComposeArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.inl)
    launch_dense_i<DKP, PROD, true>(a, grid, block, s);
  else
    launch_dense_i<DKP, PROD, false>(a, grid, block, s);
}

template <bool PROD>
hipError_t launch_dense_chain(const ComposeArgs& a, hipStream_t s) {
  const int64_t units = int64_t(a.n_req) * a.batch * a.heads;
  if (units <= 0) return hipSuccess;
  if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int dkp = (a.dk + 31) / 32 * 32;
  // one wave per 32 state columns, and enough threads to stage a whole
  // operator at 16 float4 items per thread (waves past dv hold zero columns)
  const int op_waves = (dkp * dkp / 4 + 16 * 64 - 1) / (16 * 64);
  const int waves = std::max((a.dv + 31) / 32, op_waves);
  const dim3 grid{unsigned(units), 1, 1};
  const dim3 block{unsigned(64 * waves), 1, 1};
  switch (dkp) {
    case 32: launch_dense_t<32, PROD>(a, grid, block, s); break;
    case 64: launch_dense_t<64, PROD>(a, grid, block, s); break;
    case 96: launch_dense_t<96, PROD>(a, grid, block, s); break;
    case 128: launch_dense_t<128, PROD>(a, grid, block, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_compose_dense(const ComposeArgs& a, hipStream_t s) {
  return launch_dense_chain<false>(a, s);
}

hipError_t launch_chain_T_hat(const ComposeArgs& a, hipStream_t s) {
  ComposeArgs t = a;
  t.dv = a.dk;
  t.S_in = nullptr;
  t.pool_S0 = nullptr;
  t.S_out = a.T_hat_out;
  return launch_dense_chain<true>(t, s);
}

hipError_t launch_chain_log_scale(const ComposeArgs& a, hipStream_t s) {
  const int per = (a.form == kDiag) ? a.dk : 1;
  const int64_t total = int64_t(a.n_req) * a.batch * a.heads * per;
  if (total <= 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(chain_log_scale_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, a, per);
  return hipGetLastError();
}

hipError_t launch_materialize_T(int form, int64_t n_units, int dk, const float* log_scale,
                                const float* T_hat, float* T_out, hipStream_t s) {
  const int64_t total = n_units * dk * dk;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(materialize_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, form, n_units,
                     dk, log_scale, T_hat, T_out);
  return hipGetLastError();
}

}  // namespace pic
