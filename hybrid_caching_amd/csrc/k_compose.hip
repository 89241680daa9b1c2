// k_compose.hip -- reuse-time kernels of the segment transform:
//   * dense compose      S <- e^lambda_p * That_p * S + S0_p along a chain,
//                        one 128x128x128 split-bf16 MFMA product per step
//                        (two workgroups per compute unit at full size, one's
//                        products under the other's loads);
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

// 16-byte load with the nontemporal hint: pool data is streamed once per
// chain step, so it should not displace other lines from the caches
// (measured: +7% on the naive add of 32 x 30 x 32 states)
__device__ __forceinline__ float4 load_nt(const float4* p) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const f32x4v t = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
  return make_float4(t[0], t[1], t[2], t[3]);
}

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
      x[u] = load_nt(S0 + pu * nelem4 + e4);
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
    const float4 x = load_nt(S0 + pu * nelem4 + e4);
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
// result unchanged.  This kernel serves the padded sizes (dk or dv below
// DKP); dk = dv = DKP runs compose_dense_full_kernel below.
// PROD = true forms the chain's operator instead: the "state" is dk x dk,
// starts at I, and each step is X <- That_p X (no scale, no additive term);
// the launcher passes dv = dk and S_out = the That output.
// INL: the chain tables travel in the kernel arguments
template <int DKP, bool PROD, bool INL>
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
  const int nthr = int(blockDim.x);
  const int dk = a.dk, dv = a.dv;
  const int64_t BH = int64_t(a.batch) * a.heads;
  const int64_t unit = blockIdx.x;
  const int64_t r = unit / BH, bh = unit % BH;
  const int n = wave * 32 + cl;  // state column of this lane
  const bool ncol = n < dv;
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
        S[t][q] = (a.S_in && ncol && row < dk) ? a.S_in[unit * sdd + int64_t(row) * dv + n] : 0.f;
    }
  }

  // operator of one chain step, as this thread's float4 items (zero padded)
  float4 pre[16];
  auto load_op = [&](int64_t pu) {
    const float* Tp = a.pool_T_hat + pu * int64_t(dk) * dk;
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
      if (it < per_thr && e < F4) {
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
        if (row < dk) a.S_out[unit * sdd + int64_t(row) * dv + n] = S[t][q];
      }
    }
  }
}

// Full-size dense compose (dk = dv = DKP), laid out so that two workgroups
// share a compute unit and one's products run under the other's loads.
// That_p lands in LDS as plain fp32 straight from memory (16-byte
// global-to-LDS loads, no registers on the way), its float4 columns XOR
// swizzled by row so the A-fragment reads are bank-conflict free; each wave
// splits its A fragments into hi/lo bf16 as it reads them.  S0_p is loaded
// straight into the accumulators, and e^lambda scales S before the product:
// S <- That_p (e^lambda S) + S0_p.
// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds + 16 i (lds is the same for the whole wave); nontemporal (the last
// argument is the cache policy: 2 = nt on gfx950), the operator is read once
__device__ __forceinline__ void load_lds16(const float4* src, float4* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 2);
}

template <int DKP>
struct FullTile {
  static constexpr int NT = DKP / 32;
  static constexpr int NTHR = 64 * NT;
  static constexpr int R4 = DKP / 4;                          // float4 per row
  static constexpr int SWZ = (DKP == 96) ? 7 : (R4 >= 16 ? 15 : R4 - 1);
  static constexpr int PER = DKP * DKP / 4 / NTHR;            // float4 per thread
};

template <int DKP, bool PROD, bool INL>
__global__ __launch_bounds__(64 * (DKP / 32)) __attribute__((amdgpu_waves_per_eu(2)))
void compose_dense_full_kernel(ComposeArgs a) {
  using F = FullTile<DKP>;
  constexpr int NT = F::NT, R4 = F::R4, SWZ = F::SWZ, PER = F::PER;
  __shared__ __attribute__((aligned(16))) float4 tl[DKP * R4];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, cl = lane & 31;
  const int64_t BH = int64_t(a.batch) * a.heads;
  const int64_t unit = blockIdx.x;
  const int64_t r = unit / BH, bh = unit % BH;
  const int n = wave * 32 + cl;  // state column of this lane
  constexpr int64_t sdd = int64_t(DKP) * DKP;

  f32x16 S[NT], acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = t * 32 + acc_row(q, g);
      if (PROD)
        S[t][q] = (row == n) ? 1.f : 0.f;
      else
        S[t][q] = a.S_in ? a.S_in[unit * sdd + int64_t(row) * DKP + n] : 0.f;
    }
  }

  const int64_t c0 = chain_offset_t<INL>(a, r), c1 = chain_offset_t<INL>(a, r + 1);
  // chain entries and log scales, 64 at a time, one per lane (see above)
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
  // That_p into LDS: instruction it of wave w fills slots [(it * NT + w) * 64, +64),
  // slot s holding row s / R4, float4 column (s % R4) ^ (row & SWZ)
  auto load_op = [&](int64_t pu) {
    const float4* Tp = reinterpret_cast<const float4*>(a.pool_T_hat + pu * sdd);
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int s0 = (it * NT + wave) * 64;
      const int s = s0 + lane;
      const int row = s / R4, c4 = (s % R4) ^ (row & SWZ);
      load_lds16(Tp + row * R4 + c4, tl + s0);
    }
  };
  // S0_p straight into the accumulators (nontemporal, read once)
  auto load_s0 = [&](int64_t pu) {
    const float* S0p = a.pool_S0 + pu * sdd;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (PROD)
          acc[t][q] = 0.f;
        else
          acc[t][q] = __builtin_nontemporal_load(S0p + (t * 32 + acc_row(q, g)) * DKP + n);
      }
  };
  if (c0 < c1) {
    fetch(c0);
    const int64_t pu = int64_t(entry_at(c0)) * BH + bh;
    load_op(pu);
    load_s0(pu);
  }
  for (int64_t c = c0; c < c1; ++c) {
    const float lam = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam_l), int(c - cb)));
    // this wave's global-to-LDS loads have landed; after the barrier, everyone's
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (!PROD) {
      const float scale = expf(lam);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) S[t][q] *= scale;
    }
#pragma unroll
    for (int ks = 0; ks < 2 * NT; ++ks) {
      const int t = ks >> 1, h = ks & 1;
      bf16x8 bhi, blo;
      split_acc_half(S[t], h, bhi, blo);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        // K index j of lane group g is column 16 ks + 8 (j >> 2) + 4 g + (j & 3),
        // the state row that split_acc_half put at the same place
        const int row = mt * 32 + cl;
        const float4 x0 = tl[row * R4 + ((4 * ks + g) ^ (row & SWZ))];
        const float4 x1 = tl[row * R4 + ((4 * ks + 2 + g) ^ (row & SWZ))];
        const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        bf16x8 ahi, alo;
        split8(x, ahi, alo);
        acc[mt] = mfma32(alo, bhi, acc[mt]);
        acc[mt] = mfma32(ahi, blo, acc[mt]);
        acc[mt] = mfma32(ahi, bhi, acc[mt]);
      }
    }
    __syncthreads();  // every wave is done reading That_p
#pragma unroll
    for (int t = 0; t < NT; ++t) S[t] = acc[t];
    if (c + 1 < c1) {
      if (c + 1 - cb >= 64) fetch(c + 1);
      const int64_t pu = int64_t(entry_at(c + 1)) * BH + bh;
      load_op(pu);
      load_s0(pu);
    }
  }

#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int q = 0; q < 16; ++q)
      a.S_out[unit * sdd + int64_t(t * 32 + acc_row(q, g)) * DKP + n] = S[t][q];
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
    hipLaunchKernelGGL((compose_dense_full_kernel<DKP, PROD, INL>), grid,
                       dim3(FullTile<DKP>::NTHR), 0, s, a);
  else
    hipLaunchKernelGGL((compose_dense_kernel<DKP, PROD, INL>), grid, block, 0, s, a);
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
