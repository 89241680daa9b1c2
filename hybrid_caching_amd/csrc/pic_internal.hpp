// pic_internal.hpp -- launcher interface between the C-ABI host layer and the
// HIP kernels of the segment transform.  Internal: not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace pic {

enum Form : int { kScalar = 0, kDiag = 1, kDense = 2, kKda = 3 };

// Small plans travel inside the kernel arguments, so a call needs no
// host-to-device copy before its kernel: up to kInlineSeg segments for a
// build, up to kInlineReq requests with kInlineIdx chain entries for a
// compose.  Larger plans go through the caller's workspace.
constexpr int kInlineSeg = 32;
constexpr int kInlineReq = 16;
constexpr int kInlineIdx = 64;

// Sizes of one build call, after validation.
struct BuildArgs {
  int form;
  bool qkv_bf16;
  int batch, heads, dk, dv;
  int64_t n_tokens;
  int32_t n_seg;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;          // dense only, may be null (= 1)
  const int64_t* d_offsets;   // device copy of the segment offsets [n_seg+1]
  const int32_t* d_order;     // device: segment visiting order [n_seg]
  float* log_scale;
  float* T_hat;
  float* S0;
  int64_t inl_off[kInlineSeg + 1];  // the offsets and order when n_seg <= kInlineSeg
  int32_t inl_order[kInlineSeg];
  const void* q = nullptr;    // prefill with outputs only: queries
  void* O = nullptr;          // prefill with outputs only: outputs [batch][n_tokens][heads][dv]
  unsigned* nonfinite = nullptr;  // fp16 kernels: set to 1 when an output is not finite
};

// The fp16-operand kernels' overflow report: a lane that stored a value that
// is not finite (an fp16 operand overflowed somewhere upstream: inf or NaN
// propagate to the outputs) sets the flag word with a vector atomic.
__device__ __forceinline__ bool not_finite(float x) { return !__builtin_isfinite(x); }
__device__ __forceinline__ void report_nonfinite(unsigned* flag, bool bad) {
  if (bad && flag) atomicOr(flag, 1u);
}

// a plan table entry in device memory, read as global memory: a pointer that
// may point either into the kernel arguments or into device memory would be
// read with a flat load, which also counts on the LDS wait counter, so every
// later LDS wait (e.g. before a barrier) would wait for the memory round trip
template <class T>
__device__ __forceinline__ T table_at(const T* p, int64_t i) {
  return ((const __attribute__((address_space(1))) T*)(p))[i];
}

// segment offset i and the i-th segment of the visiting order
__device__ __forceinline__ int64_t seg_offset(const BuildArgs& a, int i) {
  if (a.n_seg <= kInlineSeg) return a.inl_off[i];
  return table_at(a.d_offsets, i);
}
__device__ __forceinline__ int seg_in_order(const BuildArgs& a, int i) {
  if (a.n_seg <= kInlineSeg) return a.inl_order[i];
  return table_at(a.d_order, i);
}

// The build unit a workgroup takes: rank * (batch * heads) + layer * heads +
// head, with rank the segment's place in the visiting order.  Workgroups are
// dispatched round-robin over the 8 XCDs, each with its own L2, and the heads
// of one (segment, layer) read the same 128-byte lines of the per-head gates
// and erase strengths; so a group of `heads` units goes to one XCD, one
// workgroup after another: XCD x's k-th workgroup takes head k % heads of
// group 8 (k / heads) + x.  Workgroups past the last whole round of 8 groups
// keep their own index.  A bijection on the units, in about the visiting
// order.
__device__ __forceinline__ int64_t build_unit(const BuildArgs& a, int64_t blk) {
  constexpr int kXcd = 8;
  const int64_t groups = int64_t(a.n_seg) * a.batch;
  const int64_t full = (groups / kXcd) * kXcd * a.heads;
  if (blk >= full) return blk;
  const int64_t x = blk % kXcd, k = blk / kXcd;
  return ((k / a.heads) * kXcd + x) * a.heads + k % a.heads;
}

// One compose / naive-add call, after validation.
struct ComposeArgs {
  int form;
  int batch, heads, dk, dv;
  int64_t pool_size;
  const float* pool_log_scale;
  const float* pool_T_hat;
  const float* pool_S0;
  int32_t n_req;
  const int64_t* d_chain_off;  // device [n_req+1]
  const int32_t* d_chain_idx;  // device [chain_total]
  int64_t chain_total;
  const float* S_in;           // may be null
  float* S_out;
  float* log_scale_out;        // chain pair: sum of log scales, may be null
  float* T_hat_out;            // chain pair: product of That (dense), may be null
  bool inl;                    // chain tables inline (the fields below)
  int64_t inl_off[kInlineReq + 1];
  int32_t inl_idx[kInlineIdx];
};

// chain offset r and chain entry c
__device__ __forceinline__ int64_t chain_offset(const ComposeArgs& a, int64_t r) {
  if (a.inl) return a.inl_off[r];
  return table_at(a.d_chain_off, r);
}
__device__ __forceinline__ int chain_entry(const ComposeArgs& a, int64_t c) {
  if (a.inl) return a.inl_idx[c];
  return table_at(a.d_chain_idx, c);
}
// the same with the table's place known at compile time (a runtime choice is
// turned into a select between the two addresses, i.e. a flat load)
template <bool INL>
__device__ __forceinline__ int64_t chain_offset_t(const ComposeArgs& a, int64_t r) {
  if constexpr (INL) return a.inl_off[r];
  else return table_at(a.d_chain_off, r);
}
template <bool INL>
__device__ __forceinline__ int chain_entry_t(const ComposeArgs& a, int64_t c) {
  if constexpr (INL) return a.inl_idx[c];
  else return table_at(a.d_chain_idx, c);
}

// One reuse-with-seams call, after validation: a compose whose chain entries
// each first run a window of seam tokens through the state.
constexpr int kMaxSeam = 64;  // tokens in one seam window
struct SeamArgs {
  ComposeArgs c;               // pool, chains, states (the chain-pair outputs are unused)
  bool qkv_bf16;
  int64_t n_seam;              // seam tokens of the call (the token axis of q, k, v, ...)
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;           // dense only, may be null (= 1)
  float* O;                    // outputs [batch][n_seam][heads][dv]
  const int64_t* d_seam_off;   // device [chain_total + 1]
  int64_t inl_seam_off[kInlineIdx + 1];  // when c.inl
};

// first seam token of chain entry c (c = chain_total gives the end)
template <bool INL>
__device__ __forceinline__ int64_t seam_offset_t(const SeamArgs& a, int64_t c) {
  if constexpr (INL) return a.inl_seam_off[c];
  else return table_at(a.d_seam_off, c);
}

// Re-rotation of cached pairs (rotary embeddings on the keys): entry j of the
// output is pool entry d_idx[j] moved by d_shift[j] positions.
struct RotateArgs {
  int form;
  int batch, heads, dk, dv;
  const float* pool_log_scale;
  const float* pool_T_hat;  // null for the scalar and diagonal forms
  const float* pool_S0;
  int32_t n;
  const int32_t* d_idx;     // device [n]
  const int64_t* d_shift;   // device [n]
  int rot_dim;              // rotated channels, a multiple of 8 in [8, dk]
  double base;              // angle of pair i: shift * base^(-2i/rot_dim)
  bool half;                // pairs (i, i + rot/2); else (2i, 2i+1)
  float* log_scale_out;
  float* T_hat_out;
  float* S0_out;
};

hipError_t launch_rerotate(const RotateArgs& a, hipStream_t s);

// Convolution warm-up: conv outputs of the first n_warm tokens of each entry's
// segment, with the previous segment's raw tail as history.
struct ConvArgs {
  bool bf16;                   // x and y are bf16 (else fp32)
  int batch, heads, dc, width;
  int64_t n_tokens;
  const float* weight;         // [heads][dc][width]
  const void* x;               // [batch][n_tokens][heads][dc]
  int32_t n, n_warm;
  const int64_t* d_hist_end;   // device [n]
  const int32_t* d_hist_len;   // device [n]
  const int64_t* d_head_start; // device [n]
  void* y;                     // [batch][n * n_warm][heads][dc]
};

hipError_t launch_conv_warmup(const ConvArgs& a, hipStream_t s);
hipError_t launch_build_scalar_diag(const BuildArgs& a, hipStream_t s);
hipError_t launch_build_sd_pipe(const BuildArgs& a, hipStream_t s);
hipError_t launch_build_dense(const BuildArgs& a, hipStream_t s);
hipError_t launch_build_dense_ws(const BuildArgs& a, hipStream_t s);
// fp16 operand precision (bf16 inputs, any dk, dv <= 128)
hipError_t launch_build_dense_h16(const BuildArgs& a, hipStream_t s);
// prefill with per-token outputs (dense form, bf16 q/k/v, fp16 operands),
// That tracked when track_T
hipError_t launch_dense_prefill(const BuildArgs& a, bool track_T, hipStream_t s);
// KDA form: token by token in fp32 on the vector units
hipError_t launch_build_kda(const BuildArgs& a, hipStream_t s);
// KDA form in chunks of 32 tokens on the matrix cores (bf16 k/v, fp16
// operands, dk = dv = 128)
hipError_t launch_build_kda_chunk(const BuildArgs& a, hipStream_t s);
hipError_t launch_compose_dense(const ComposeArgs& a, hipStream_t s);
hipError_t launch_compose_elementwise(const ComposeArgs& a, bool naive, hipStream_t s);
hipError_t launch_compose_seams(const SeamArgs& a, hipStream_t s);
// chain pair: log_scale_out (all forms) and That_out = That_pn ... That_p1 (dense)
hipError_t launch_chain_log_scale(const ComposeArgs& a, hipStream_t s);
hipError_t launch_chain_T_hat(const ComposeArgs& a, hipStream_t s);
hipError_t launch_materialize_T(int form, int64_t n_units, int dk, const float* log_scale,
                                const float* T_hat, float* T_out, hipStream_t s);

}  // namespace pic
