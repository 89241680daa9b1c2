// pic_host.cpp -- the C ABI declared in include/pic.h: argument validation,
// host-side planning (segment order, chain tables), workspace layout and
// kernel launches.  Validation touches no HIP API, so it can be exercised on
// a machine without a GPU.
#include "pic.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <mutex>
#include <numeric>
#include <vector>

#include "pic_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return PIC_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool dim_ok(int d) { return d >= 16 && d <= 128 && d % 16 == 0; }

// forms whose pair carries an operator That (a per-head lambda and a dk x dk matrix)
bool has_T_hat(int form) { return form == PIC_FORM_DENSE || form == PIC_FORM_KDA; }

// ---------------------------------------------------------------- staging
// Tables too large for the kernel arguments (segment offsets and order,
// chain tables, ...) reach the caller's workspace by hipMemcpyAsync.  By
// default they are copied straight from host memory that is gone (or may be
// reused) once the call returns, so the call then waits for its stream; the
// library holds no memory between calls.  pic_staging_reserve() opts into a
// pool of pinned host slots on the current device: the tables are first
// copied into a slot, and the slot's copy to the device is asynchronous, so
// back-to-back calls queue on the stream without waiting for the device.  A
// slot is reused after the copy that last read it has completed (one event
// per slot; with 64 slots that wait is normally already over).  The pool is
// held until pic_staging_release().  A mutex guards the pools.  Neither way
// is usable under stream capture.
struct Piece {
  void* dst;
  const void* src;
  size_t bytes;
};

class Staging {
 public:
  static constexpr int kSlots = 64;
  static constexpr size_t kSlotBytes = 64 * 1024;
  static constexpr int kMaxDevices = 64;

  hipError_t copy(std::initializer_list<Piece> pieces, hipStream_t s) {
    size_t total = 0;
    for (const Piece& p : pieces) total += p.bytes + kSlack;
    if (total == 0) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu_);
    if (total > kSlotBytes || dev < 0 || dev >= kMaxDevices || !pools_[dev].host)
      return copy_pageable(pieces, s);
    Pool& pool = pools_[dev];
    const int i = pool.next;
    pool.next = (pool.next + 1) % kSlots;
    if (pool.pending[i]) {
      e = hipEventSynchronize(pool.ev[i]);
      if (e != hipSuccess) return e;
      pool.pending[i] = false;
    }
    // The pieces go to ascending places of one workspace: lay them out in
    // the slot as they lie there and move the whole span with one copy.
    char* slot = pool.host + size_t(i) * kSlotBytes;
    char* base = nullptr;
    size_t span = 0;
    for (const Piece& p : pieces) {
      if (p.bytes == 0) continue;
      char* d = static_cast<char*>(p.dst);
      if (!base) base = d;
      if (d < base + span || size_t(d - base) + p.bytes > kSlotBytes) {
        base = nullptr;  // not laid out as expected: one copy per piece
        break;
      }
      span = size_t(d - base) + p.bytes;
    }
    if (base) {
      for (const Piece& p : pieces)
        if (p.bytes) std::memcpy(slot + (static_cast<char*>(p.dst) - base), p.src, p.bytes);
      e = hipMemcpyAsync(base, slot, span, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return e;
    } else {
      size_t at = 0;
      for (const Piece& p : pieces) {
        if (p.bytes == 0) continue;
        std::memcpy(slot + at, p.src, p.bytes);
        e = hipMemcpyAsync(p.dst, slot + at, p.bytes, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return e;
        at += p.bytes;
      }
    }
    e = hipEventRecord(pool.ev[i], s);
    pool.pending[i] = e == hipSuccess;
    return e;
  }

  // pinned pool of the current device (no-op if it exists)
  hipError_t reserve() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu_);
    Pool& pool = pools_[dev];
    if (pool.host) return hipSuccess;
    e = hipHostMalloc(reinterpret_cast<void**>(&pool.host), kSlots * kSlotBytes,
                      hipHostMallocDefault);
    if (e != hipSuccess) {
      pool.host = nullptr;
      return e;
    }
    for (int i = 0; i < kSlots; ++i) {
      e = hipEventCreateWithFlags(&pool.ev[i], hipEventDisableTiming);
      if (e != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(pool.ev[j]);
        (void)hipHostFree(pool.host);
        pool.host = nullptr;
        return e;
      }
      pool.pending[i] = false;
    }
    pool.next = 0;
    held_ += kSlots * kSlotBytes;
    return hipSuccess;
  }

  // every pool: wait for the copies that read it, then free it
  hipError_t release() {
    std::lock_guard<std::mutex> lock(mu_);
    hipError_t first = hipSuccess;
    int cur = 0;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (int dev = 0; dev < kMaxDevices; ++dev) {
      Pool& pool = pools_[dev];
      if (!pool.host) continue;
      (void)hipSetDevice(dev);
      for (int i = 0; i < kSlots; ++i) {
        hipError_t e = pool.pending[i] ? hipEventSynchronize(pool.ev[i]) : hipSuccess;
        if (e == hipSuccess) e = hipEventDestroy(pool.ev[i]);
        if (e != hipSuccess && first == hipSuccess) first = e;
        pool.pending[i] = false;
      }
      const hipError_t e = hipHostFree(pool.host);
      if (e != hipSuccess && first == hipSuccess) first = e;
      pool.host = nullptr;
      held_ -= kSlots * kSlotBytes;
    }
    if (have_cur) (void)hipSetDevice(cur);
    return first;
  }

  size_t held() {
    std::lock_guard<std::mutex> lock(mu_);
    return held_;
  }

 private:
  static constexpr size_t kSlack = 256;  // alignment gaps between the pieces
  struct Pool {
    char* host = nullptr;
    hipEvent_t ev[kSlots];
    bool pending[kSlots];
    int next = 0;
  };
  static hipError_t copy_pageable(std::initializer_list<Piece> pieces, hipStream_t s) {
    for (const Piece& p : pieces) {
      if (p.bytes == 0) continue;
      const hipError_t e = hipMemcpyAsync(p.dst, p.src, p.bytes, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return e;
    }
    return hipStreamSynchronize(s);
  }
  std::mutex mu_;
  Pool pools_[kMaxDevices];
  size_t held_ = 0;
};

Staging& staging() {
  // the object itself is never destroyed (calls may come from other static
  // destructors); the pinned memory it holds is freed by pic_staging_release
  static Staging* st = new Staging();
  return *st;
}

// product of non-negative sizes, or -1 on int64 overflow
int64_t mul_sizes(std::initializer_list<int64_t> xs) {
  int64_t p = 1;
  for (int64_t x : xs) {
    if (x < 0) return -1;
    if (x != 0 && p > std::numeric_limits<int64_t>::max() / x) return -1;
    p *= x;
  }
  return p;
}

int check_common_dims(int batch, int heads, int dk, int dv) {
  if (batch < 1 || heads < 1)
    return fail(PIC_ERR_DIMS, "batch (%d) and heads (%d) must be >= 1", batch, heads);
  if (!dim_ok(dk) || !dim_ok(dv))
    return fail(PIC_ERR_DIMS, "dk (%d) and dv (%d) must be multiples of 16 in [16, 128]", dk,
                dv);
  return PIC_OK;
}

// Build workspace: offsets (n_seg+1 int64) then order (n_seg int32).
size_t build_ws_bytes(int32_t n_seg) {
  if (n_seg < 0) return 0;
  return align_up(sizeof(int64_t) * (size_t(n_seg) + 1)) + align_up(sizeof(int32_t) * size_t(n_seg));
}

size_t compose_ws_bytes(int32_t n_req, int64_t total) {
  if (n_req < 0 || total < 0) return 0;
  return align_up(sizeof(int64_t) * (size_t(n_req) + 1)) +
         align_up(sizeof(int32_t) * size_t(std::max<int64_t>(total, 1)));
}

// Reuse with seams: the compose tables, then the seam offsets (int64 each).
static_assert(pic::kMaxSeam == PIC_MAX_SEAM, "seam window limit of the header");

size_t compose_seams_ws_bytes(int32_t n_req, int64_t total) {
  if (n_req < 0 || total < 0) return 0;
  return compose_ws_bytes(n_req, total) + align_up(sizeof(int64_t) * (size_t(total) + 1));
}

int check_chains(int64_t pool_size, int32_t n_req, const int64_t* off, const int32_t* idx) {
  if (n_req < 0) return fail(PIC_ERR_DIMS, "n_req (%d) must be >= 0", n_req);
  if (pool_size < 0) return fail(PIC_ERR_DIMS, "pool_size must be >= 0");
  if (!off) return fail(PIC_ERR_NULL, "chain_offsets is NULL");
  if (off[0] != 0) return fail(PIC_ERR_CHAIN, "chain_offsets[0] = %lld, must be 0", (long long)off[0]);
  for (int32_t r = 0; r < n_req; ++r)
    if (off[r + 1] < off[r])
      return fail(PIC_ERR_CHAIN, "chain_offsets decrease at request %d", r);
  const int64_t total = off[n_req];
  if (total > 0 && !idx) return fail(PIC_ERR_NULL, "chain_idx is NULL");
  if (total > std::numeric_limits<int32_t>::max())
    return fail(PIC_ERR_CHAIN, "chain too long");
  for (int64_t s = 0; s < total; ++s)
    if (idx[s] < 0 || int64_t(idx[s]) >= pool_size)
      return fail(PIC_ERR_CHAIN, "chain_idx[%lld] = %d outside [0, %lld)", (long long)s, idx[s],
                  (long long)pool_size);
  return PIC_OK;
}

bool overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  if (!a || !b || a_bytes <= 0 || b_bytes <= 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + uintptr_t(b_bytes) && y < x + uintptr_t(a_bytes);
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// every non-null device pointer must be 16-byte aligned
int check_align(std::initializer_list<const void*> ptrs) {
  int i = 0;
  for (const void* p : ptrs) {
    if (p && misaligned(p)) return fail(PIC_ERR_ALIGN, "device pointer argument %d is not 16-byte aligned", i);
    ++i;
  }
  return PIC_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PIC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Visiting order of a build: longest segment first, ties by index, so that
// long units start early and short ones fill the tail of the launch.
std::vector<int32_t> build_order(const int64_t* off, int32_t n_seg) {
  std::vector<int32_t> order(n_seg);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return off[a + 1] - off[a] > off[b + 1] - off[b];
  });
  return order;
}

int check_seg_offsets(const int64_t* seg_offsets, int32_t n_seg, int64_t n_tokens) {
  if (!seg_offsets) return fail(PIC_ERR_NULL, "seg_offsets is NULL");
  if (seg_offsets[0] != 0)
    return fail(PIC_ERR_OFFSETS, "seg_offsets[0] = %lld, must be 0", (long long)seg_offsets[0]);
  for (int32_t s = 0; s < n_seg; ++s)
    if (seg_offsets[s + 1] < seg_offsets[s])
      return fail(PIC_ERR_OFFSETS, "seg_offsets decrease at segment %d", s);
  if (seg_offsets[n_seg] != n_tokens)
    return fail(PIC_ERR_OFFSETS, "seg_offsets[n_seg] = %lld, must equal n_tokens = %lld",
                (long long)seg_offsets[n_seg], (long long)n_tokens);
  return PIC_OK;
}

// ------------------------------------------------------- static scratch
// Device memory for pic_compose_noalloc: its chain tables live in this
// file-scope array (one copy per device, held until the process ends), so
// that entry point needs neither a workspace nor an allocation.  In host code
// the array's name is only a stand-in: the device address of each device's
// copy is looked up once per device (with that device current) and kept.
constexpr size_t kScratchBytes = PIC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_symbol_mu;
void* g_scratch_ptr[Staging::kMaxDevices] = {};

// Device address of a file-scope __device__ variable on the current device,
// looked up once per device (each device holds its own copy) and kept.
hipError_t symbol_address(const void* symbol, void** cache, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= Staging::kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_symbol_mu);
  if (!cache[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, symbol);
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    cache[dev] = p;
  }
  *out = cache[dev];
  return hipSuccess;
}

hipError_t scratch_address(void** out) {
  return symbol_address(HIP_SYMBOL(scratch), g_scratch_ptr, out);
}

// ------------------------------------------------------- fp16 overflow flag
// One word per device, set by the fp16-operand kernels (a vector atomic OR)
// when a value they store is not finite; read and cleared by
// pic_nonfinite_check.  Zero-initialised with the code object.
static __device__ __align__(4) unsigned int nonfinite_flag[1];
void* g_flag_ptr[Staging::kMaxDevices] = {};

hipError_t flag_address(unsigned** out) {
  void* p = nullptr;
  const hipError_t e = symbol_address(HIP_SYMBOL(nonfinite_flag), g_flag_ptr, &p);
  *out = static_cast<unsigned*>(p);
  return e;
}

}  // namespace

extern "C" {

int pic_abi_version(void) { return PIC_ABI_VERSION; }

const char* pic_status_string(int status) {
  switch (status) {
    case PIC_OK: return "ok";
    case PIC_ERR_NULL: return "required pointer is NULL";
    case PIC_ERR_DIMS: return "unsupported or inconsistent sizes";
    case PIC_ERR_OFFSETS: return "bad segment offsets";
    case PIC_ERR_CHAIN: return "bad chain offsets or pool index";
    case PIC_ERR_WORKSPACE: return "workspace missing or too small";
    case PIC_ERR_UNSUPPORTED: return "unsupported form, dtype or argument combination";
    case PIC_ERR_HIP: return "HIP runtime error";
    case PIC_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case PIC_ERR_NONFINITE: return "an fp16-operand call stored a value that is not finite";
    default: return "unknown status";
  }
}

const char* pic_last_error(void) { return g_last_error; }

int pic_staging_reserve(void) {
  const hipError_t e = staging().reserve();
  if (e != hipSuccess) return hip_fail(e, "allocating the pinned staging pool");
  return ok();
}

int pic_staging_release(void) {
  const hipError_t e = staging().release();
  if (e != hipSuccess) return hip_fail(e, "releasing the pinned staging pools");
  return ok();
}

size_t pic_staging_bytes(void) { return staging().held(); }

/* ------------------------------------------------------------------ build */

// the segment plan (offsets and longest-first order) into the arguments
// (small) or the workspace (copied)
static int enqueue_build_plan(const int64_t* seg_offsets, int32_t n_seg, void* workspace,
                              hipStream_t s, pic::BuildArgs& a) {
  const std::vector<int32_t> order = build_order(seg_offsets, n_seg);
  if (n_seg <= pic::kInlineSeg) {
    std::copy(seg_offsets, seg_offsets + n_seg + 1, a.inl_off);
    std::copy(order.begin(), order.end(), a.inl_order);
    return PIC_OK;
  }
  char* ws = static_cast<char*>(workspace);
  int64_t* d_off = reinterpret_cast<int64_t*>(ws);
  int32_t* d_order =
      reinterpret_cast<int32_t*>(ws + align_up(sizeof(int64_t) * (size_t(n_seg) + 1)));
  const hipError_t e = staging().copy({{d_off, seg_offsets, sizeof(int64_t) * (size_t(n_seg) + 1)},
                                       {d_order, order.data(), sizeof(int32_t) * size_t(n_seg)}},
                                      s);
  if (e != hipSuccess) return hip_fail(e, "copying the segment plan");
  a.d_offsets = d_off;
  a.d_order = d_order;
  return PIC_OK;
}

size_t pic_segment_build_workspace(int form, int batch, int heads, int dk, int dv,
                                   int64_t n_tokens, int32_t n_seg) {
  (void)form; (void)batch; (void)heads; (void)dk; (void)dv; (void)n_tokens;
  return build_ws_bytes(n_seg);
}

}  // extern "C"

// checks of a build's arguments; the workspace must hold `need` bytes
// (need = SIZE_MAX: not checked here)
static int validate_build_args(int form, int qkv_dtype, int precision, int batch, int heads,
                               int dk, int dv, int64_t n_tokens, const void* q, const void* k,
                               const void* v, const float* alpha, const float* beta,
                               const int64_t* seg_offsets, int32_t n_seg, const float* log_scale,
                               const float* T_hat, const float* S0, const void* workspace,
                               size_t workspace_bytes, size_t need) {
  (void)q;  // never read: the pair does not depend on queries
  (void)beta;
  if (form < PIC_FORM_SCALAR || form > PIC_FORM_KDA)
    return fail(PIC_ERR_UNSUPPORTED, "unknown form %d", form);
  if (qkv_dtype != PIC_DT_F32 && qkv_dtype != PIC_DT_BF16)
    return fail(PIC_ERR_UNSUPPORTED, "unknown qkv dtype %d", qkv_dtype);
  if (precision != PIC_PREC_FP32 && precision != PIC_PREC_FP16)
    return fail(PIC_ERR_UNSUPPORTED, "unknown precision %d", precision);
  if (precision == PIC_PREC_FP16 &&
      ((form != PIC_FORM_DENSE && form != PIC_FORM_KDA) || qkv_dtype != PIC_DT_BF16))
    return fail(PIC_ERR_UNSUPPORTED, "PIC_PREC_FP16 needs the dense or KDA form with bf16 k/v");
  if (precision == PIC_PREC_FP16 && form == PIC_FORM_KDA && (dk != 128 || dv != 128))
    return fail(PIC_ERR_UNSUPPORTED, "the KDA form at PIC_PREC_FP16 needs dk = dv = 128 (%d, %d)",
                dk, dv);
  if (int rc = check_common_dims(batch, heads, dk, dv)) return rc;
  if (n_seg < 1) return fail(PIC_ERR_DIMS, "n_seg (%d) must be >= 1", n_seg);
  if (n_tokens < 0) return fail(PIC_ERR_DIMS, "n_tokens must be >= 0");
  const int64_t per_gate = (form == PIC_FORM_DIAG || form == PIC_FORM_KDA) ? dk : 1;
  if (mul_sizes({batch, n_tokens, heads, std::max(dk, dv)}) < 0 ||
      mul_sizes({n_seg, batch, heads, dk, std::max(dk, dv)}) < 0 ||
      mul_sizes({batch, n_tokens, heads, per_gate}) < 0)
    return fail(PIC_ERR_DIMS, "sizes overflow 64-bit indexing");
  if (!seg_offsets) return fail(PIC_ERR_NULL, "seg_offsets is NULL");
  if (n_tokens > 0 && (!k || !v || !alpha))
    return fail(PIC_ERR_NULL, "k, v and alpha are required");
  if (!log_scale || !S0) return fail(PIC_ERR_NULL, "log_scale and S0 outputs are required");
  if (has_T_hat(form) && !T_hat)
    return fail(PIC_ERR_NULL, "T_hat output is required for the dense and KDA forms");
  if (!has_T_hat(form) && T_hat)
    return fail(PIC_ERR_UNSUPPORTED, "T_hat must be NULL for scalar and diagonal forms");
  if (int rc = check_seg_offsets(seg_offsets, n_seg, n_tokens)) return rc;
  if (int rc = check_align({k, v, alpha, beta, log_scale, T_hat, S0, workspace})) return rc;
  if (need == SIZE_MAX) return ok();
  if (!workspace || workspace_bytes < need)
    return fail(PIC_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  return ok();
}

// the build of validated arguments: plan, then the kernel of the form and
// precision
static int enqueue_build(int form, int qkv_dtype, int precision, int batch, int heads, int dk,
                         int dv, int64_t n_tokens, const void* k, const void* v,
                         const float* alpha, const float* beta, const int64_t* seg_offsets,
                         int32_t n_seg, float* log_scale, float* T_hat, float* S0,
                         void* workspace, hipStream_t s) {
  pic::BuildArgs a{form, qkv_dtype == PIC_DT_BF16, batch, heads, dk, dv, n_tokens, n_seg,
                   k, v, alpha, beta, nullptr, nullptr, log_scale, T_hat, S0, {}, {}};
  if (precision == PIC_PREC_FP16) {
    const hipError_t fe = flag_address(&a.nonfinite);
    if (fe != hipSuccess) return hip_fail(fe, "looking up the overflow flag");
  }
  if (int rc = enqueue_build_plan(seg_offsets, n_seg, workspace, s, a)) return rc;
  hipError_t e = hipSuccess;
  if (form == PIC_FORM_DENSE)
    e = (precision == PIC_PREC_FP16) ? pic::launch_build_dense_h16(a, s)
                                     : pic::launch_build_dense(a, s);
  else if (form == PIC_FORM_KDA)
    e = (precision == PIC_PREC_FP16) ? pic::launch_build_kda_chunk(a, s)
                                     : pic::launch_build_kda(a, s);
  else
    e = pic::launch_build_scalar_diag(a, s);
  if (e != hipSuccess) return hip_fail(e, "launching the build kernel");
  return PIC_OK;
}

// pieces of every segment for the split build: whole 64-token chunks, as
// equal as they allow; chain_off[s] .. chain_off[s+1] are segment s's pieces
static std::vector<int64_t> split_pieces(const int64_t* off, int32_t n_seg, int32_t n_split,
                                         std::vector<int64_t>& chain_off) {
  constexpr int64_t kChunk = 64;
  std::vector<int64_t> sub(1, 0);
  chain_off.assign(1, 0);
  for (int32_t i = 0; i < n_seg; ++i) {
    const int64_t len = off[i + 1] - off[i];
    const int64_t chunks = (len + kChunk - 1) / kChunk;
    const int64_t p = std::min<int64_t>(n_split, std::max<int64_t>(chunks, 1));
    const int64_t q = chunks / p, r = chunks % p;
    int64_t at = off[i];
    for (int64_t j = 0; j < p; ++j) {
      at = (j == p - 1) ? off[i + 1] : at + (q + (j < r ? 1 : 0)) * kChunk;
      sub.push_back(at);
    }
    chain_off.push_back(chain_off.back() + p);
  }
  return sub;
}

// workspace of the split build for P pieces: their pairs, then the build plan,
// then the merge's chain tables
struct SplitLayout {
  size_t lam = 0, T = 0, S = 0, plan = 0, chains = 0, total = 0;
};
static SplitLayout split_layout(int form, int batch, int heads, int dk, int dv, int64_t P,
                                int32_t n_seg) {
  SplitLayout L;
  const size_t units = size_t(P) * size_t(batch) * size_t(heads);
  const size_t per_lam = (form == PIC_FORM_DIAG) ? size_t(dk) : 1;
  size_t at = 0;
  L.lam = at;
  at += align_up(units * per_lam * sizeof(float));
  L.T = at;
  if (has_T_hat(form)) at += align_up(units * size_t(dk) * size_t(dk) * sizeof(float));
  L.S = at;
  at += align_up(units * size_t(dk) * size_t(dv) * sizeof(float));
  L.plan = at;
  at += build_ws_bytes(int32_t(P));
  L.chains = at;
  at += compose_ws_bytes(n_seg, P);
  L.total = at;
  return L;
}

extern "C" {

int pic_validate_build(int form, int qkv_dtype, int precision, int batch, int heads, int dk, int dv,
                       int64_t n_tokens, const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, const int64_t* seg_offsets,
                       int32_t n_seg, const float* log_scale, const float* T_hat,
                       const float* S0, const void* workspace, size_t workspace_bytes) {
  return validate_build_args(form, qkv_dtype, precision, batch, heads, dk, dv, n_tokens, q, k, v,
                             alpha, beta, seg_offsets, n_seg, log_scale, T_hat, S0, workspace,
                             workspace_bytes, n_seg >= 0 ? build_ws_bytes(n_seg) : SIZE_MAX);
}

int pic_segment_build(int form, int qkv_dtype, int precision, int batch, int heads, int dk, int dv,
                      int64_t n_tokens, const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, const int64_t* seg_offsets,
                      int32_t n_seg, float* log_scale, float* T_hat, float* S0,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = pic_validate_build(form, qkv_dtype, precision, batch, heads, dk, dv, n_tokens, q, k, v,
                                  alpha, beta, seg_offsets, n_seg, log_scale, T_hat, S0,
                                  workspace, workspace_bytes))
    return rc;
  if (int rc = enqueue_build(form, qkv_dtype, precision, batch, heads, dk, dv, n_tokens, k, v,
                             alpha, beta, seg_offsets, n_seg, log_scale, T_hat, S0, workspace,
                             static_cast<hipStream_t>(stream)))
    return rc;
  return ok();
}

/* ---------------------------------------------------------------- prefill */

int pic_validate_prefill(int batch, int heads, int dk, int dv, int64_t n_tokens, const void* q,
                         const void* k, const void* v, const float* alpha, const float* beta,
                         const int64_t* seg_offsets, int32_t n_seg, const float* log_scale,
                         const float* T_hat, const float* S0, const void* O_out,
                         const void* workspace, size_t workspace_bytes) {
  if (int rc = check_common_dims(batch, heads, dk, dv)) return rc;
  if (n_seg < 1) return fail(PIC_ERR_DIMS, "n_seg (%d) must be >= 1", n_seg);
  if (n_tokens < 0) return fail(PIC_ERR_DIMS, "n_tokens must be >= 0");
  if (mul_sizes({batch, n_tokens, heads, std::max(dk, dv)}) < 0 ||
      mul_sizes({n_seg, batch, heads, dk, std::max(dk, dv)}) < 0)
    return fail(PIC_ERR_DIMS, "sizes overflow 64-bit indexing");
  if (!seg_offsets) return fail(PIC_ERR_NULL, "seg_offsets is NULL");
  if (n_tokens > 0 && (!q || !k || !v || !alpha))
    return fail(PIC_ERR_NULL, "q, k, v and alpha are required");
  if (n_tokens > 0 && !O_out) return fail(PIC_ERR_NULL, "O_out is required");
  if (!log_scale || !S0) return fail(PIC_ERR_NULL, "log_scale and S0 outputs are required");
  if (int rc = check_seg_offsets(seg_offsets, n_seg, n_tokens)) return rc;
  if (int rc = check_align({q, k, v, alpha, beta, log_scale, T_hat, S0, O_out, workspace}))
    return rc;
  const int64_t o_b = int64_t(batch) * n_tokens * heads * dv * 2;
  const int64_t qk_b = int64_t(batch) * n_tokens * heads * dk * 2;
  const int64_t g_b = int64_t(batch) * n_tokens * heads * 4;
  if (overlap(O_out, o_b, q, qk_b) || overlap(O_out, o_b, k, qk_b) || overlap(O_out, o_b, v, o_b) ||
      overlap(O_out, o_b, alpha, g_b) || overlap(O_out, o_b, beta, g_b))
    return fail(PIC_ERR_UNSUPPORTED, "O_out overlaps an input");
  const size_t need = build_ws_bytes(n_seg);
  if (!workspace || workspace_bytes < need)
    return fail(PIC_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  return ok();
}

int pic_segment_prefill(int batch, int heads, int dk, int dv, int64_t n_tokens, const void* q,
                        const void* k, const void* v, const float* alpha, const float* beta,
                        const int64_t* seg_offsets, int32_t n_seg, float* log_scale,
                        float* T_hat, float* S0, void* O_out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (int rc = pic_validate_prefill(batch, heads, dk, dv, n_tokens, q, k, v, alpha, beta,
                                    seg_offsets, n_seg, log_scale, T_hat, S0, O_out, workspace,
                                    workspace_bytes))
    return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  pic::BuildArgs a{PIC_FORM_DENSE, true, batch, heads, dk, dv, n_tokens, n_seg,
                   k, v, alpha, beta, nullptr, nullptr, log_scale, T_hat, S0, {}, {}};
  a.q = q;
  a.O = O_out;
  const hipError_t fe = flag_address(&a.nonfinite);
  if (fe != hipSuccess) return hip_fail(fe, "looking up the overflow flag");
  if (int rc = enqueue_build_plan(seg_offsets, n_seg, workspace, s, a)) return rc;
  const hipError_t e = pic::launch_dense_prefill(a, T_hat != nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "launching the prefill kernel");
  return ok();
}

int pic_nonfinite_check(void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned* flag = nullptr;
  hipError_t e = flag_address(&flag);
  if (e != hipSuccess) return hip_fail(e, "looking up the overflow flag");
  unsigned h = 0;
  e = hipMemcpyAsync(&h, flag, sizeof h, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the overflow flag");
  if (h == 0) return ok();
  const unsigned zero = 0;
  e = hipMemcpyAsync(flag, &zero, sizeof zero, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "clearing the overflow flag");
  return fail(PIC_ERR_NONFINITE,
              "an fp16-operand build or prefill stored a value that is not finite (an fp16 "
              "operand overflowed: inputs outside the PIC_PREC_FP16 preconditions)");
}

/* ---------------------------------------------------------------- compose */

size_t pic_compose_workspace(int32_t n_req, int64_t chain_total) {
  return compose_ws_bytes(n_req, chain_total);
}

int pic_validate_compose(int form, int batch, int heads, int dk, int dv, int64_t pool_size,
                         const float* pool_log_scale, const float* pool_T_hat,
                         const float* pool_S0, int32_t n_req, const int64_t* chain_offsets,
                         const int32_t* chain_idx, const float* S_in, const float* S_out,
                         const float* log_scale_out, const float* T_hat_out,
                         const void* workspace, size_t workspace_bytes) {
  (void)S_in;
  if (form < PIC_FORM_SCALAR || form > PIC_FORM_KDA)
    return fail(PIC_ERR_UNSUPPORTED, "unknown form %d", form);
  if (int rc = check_common_dims(batch, heads, dk, dv)) return rc;
  if (mul_sizes({pool_size, batch, heads, dk, std::max(dk, dv)}) < 0 ||
      mul_sizes({n_req, batch, heads, dk, dv}) < 0)
    return fail(PIC_ERR_DIMS, "sizes overflow 64-bit indexing");
  if (int rc = check_chains(pool_size, n_req, chain_offsets, chain_idx)) return rc;
  const int64_t total = chain_offsets[n_req];
  if (n_req > 0 && !S_out) return fail(PIC_ERR_NULL, "S_out is required");
  if (total > 0 && (!pool_S0 || !pool_log_scale))
    return fail(PIC_ERR_NULL, "pool_S0 and pool_log_scale are required");
  if (total > 0 && has_T_hat(form) && !pool_T_hat)
    return fail(PIC_ERR_NULL, "pool_T_hat is required for the dense and KDA forms");
  if (!has_T_hat(form) && pool_T_hat)
    return fail(PIC_ERR_UNSUPPORTED, "pool_T_hat must be NULL for scalar and diagonal forms");
  if (!has_T_hat(form) && T_hat_out)
    return fail(PIC_ERR_UNSUPPORTED, "T_hat_out must be NULL for scalar and diagonal forms");
  if (has_T_hat(form) && (!log_scale_out) != (!T_hat_out))
    return fail(PIC_ERR_NULL, "the chain pair needs both log_scale_out and T_hat_out");
  if (mul_sizes({n_req, batch, heads, dk, dk}) < 0)
    return fail(PIC_ERR_DIMS, "sizes overflow 64-bit indexing");
  if (int rc = check_align({pool_log_scale, pool_T_hat, pool_S0, S_in, S_out, log_scale_out,
                            T_hat_out, workspace}))
    return rc;
  const size_t need = compose_ws_bytes(n_req, total);
  if (!workspace || workspace_bytes < need)
    return fail(PIC_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  return ok();
}

int pic_validate_naive_add(int batch, int heads, int dk, int dv, int64_t pool_size,
                           const float* pool_S0, int32_t n_req, const int64_t* chain_offsets,
                           const int32_t* chain_idx, const float* S_in, const float* S_out,
                           const void* workspace, size_t workspace_bytes) {
  (void)S_in;
  if (int rc = check_common_dims(batch, heads, dk, dv)) return rc;
  if (mul_sizes({pool_size, batch, heads, dk, dv}) < 0 ||
      mul_sizes({n_req, batch, heads, dk, dv}) < 0)
    return fail(PIC_ERR_DIMS, "sizes overflow 64-bit indexing");
  if (int rc = check_chains(pool_size, n_req, chain_offsets, chain_idx)) return rc;
  const int64_t total = chain_offsets[n_req];
  if (n_req > 0 && !S_out) return fail(PIC_ERR_NULL, "S_out is required");
  if (total > 0 && !pool_S0) return fail(PIC_ERR_NULL, "pool_S0 is required");
  if (int rc = check_align({pool_S0, S_in, S_out, workspace})) return rc;
  const size_t need = compose_ws_bytes(n_req, total);
  if (!workspace || workspace_bytes < need)
    return fail(PIC_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  return ok();
}

// chain tables into the arguments (small) or the workspace (copied)
static int enqueue_chains(int32_t n_req, const int64_t* off, const int32_t* idx, void* workspace,
                          hipStream_t s, pic::ComposeArgs& a, bool force_table = false) {
  const int64_t total = off[n_req];
  a.inl = !force_table && n_req <= pic::kInlineReq && total <= pic::kInlineIdx;
  if (a.inl) {
    std::copy(off, off + n_req + 1, a.inl_off);
    if (total > 0) std::copy(idx, idx + total, a.inl_idx);
    return PIC_OK;
  }
  char* ws = static_cast<char*>(workspace);
  int64_t* o = reinterpret_cast<int64_t*>(ws);
  int32_t* i = reinterpret_cast<int32_t*>(ws + align_up(sizeof(int64_t) * (size_t(n_req) + 1)));
  const hipError_t e = staging().copy(
      {{o, off, sizeof(int64_t) * (size_t(n_req) + 1)},
       {i, idx, total > 0 ? sizeof(int32_t) * size_t(total) : size_t(0)}},
      s);
  if (e != hipSuccess) return hip_fail(e, "copying the chain tables");
  a.d_chain_off = o;
  a.d_chain_idx = i;
  return PIC_OK;
}

int pic_compose(int form, int batch, int heads, int dk, int dv, int64_t pool_size,
                const float* pool_log_scale, const float* pool_T_hat, const float* pool_S0,
                int32_t n_req, const int64_t* chain_offsets, const int32_t* chain_idx,
                const float* S_in, float* S_out, float* log_scale_out, float* T_hat_out,
                void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = pic_validate_compose(form, batch, heads, dk, dv, pool_size, pool_log_scale,
                                    pool_T_hat, pool_S0, n_req, chain_offsets, chain_idx, S_in,
                                    S_out, log_scale_out, T_hat_out, workspace, workspace_bytes))
    return rc;
  if (n_req == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  pic::ComposeArgs a{form,    batch,    heads,    dk,     dv,       pool_size,
                     pool_log_scale, pool_T_hat, pool_S0, n_req, nullptr, nullptr,
                     chain_offsets[n_req], S_in, S_out, log_scale_out, T_hat_out, false, {}, {}};
  if (int rc = enqueue_chains(n_req, chain_offsets, chain_idx, workspace, s, a)) return rc;
  hipError_t e = has_T_hat(form) ? pic::launch_compose_dense(a, s)
                                          : pic::launch_compose_elementwise(a, false, s);
  if (e != hipSuccess) return hip_fail(e, "launching the compose kernel");
  if (log_scale_out) {
    e = pic::launch_chain_log_scale(a, s);
    if (e != hipSuccess) return hip_fail(e, "launching the chain log-scale kernel");
  }
  if (T_hat_out) {
    e = pic::launch_chain_T_hat(a, s);
    if (e != hipSuccess) return hip_fail(e, "launching the chain operator kernel");
  }
  return ok();
}

/* ------------------------------------------------------ split build */

int pic_split_plan(int32_t n_seg, const int64_t* seg_offsets, int64_t n_tokens, int32_t n_split,
                   int64_t* piece_offsets, int64_t piece_capacity, int64_t* seg_pieces,
                   int64_t* n_pieces) {
  if (n_seg < 1) return fail(PIC_ERR_DIMS, "n_seg (%d) must be >= 1", n_seg);
  if (n_split < 1) return fail(PIC_ERR_DIMS, "n_split (%d) must be >= 1", n_split);
  if (n_tokens < 0) return fail(PIC_ERR_DIMS, "n_tokens must be >= 0");
  if (!n_pieces || !seg_pieces) return fail(PIC_ERR_NULL, "n_pieces and seg_pieces are required");
  if (int rc = check_seg_offsets(seg_offsets, n_seg, n_tokens)) return rc;
  std::vector<int64_t> chain_off;
  const std::vector<int64_t> sub = split_pieces(seg_offsets, n_seg, n_split, chain_off);
  *n_pieces = int64_t(sub.size()) - 1;
  if (piece_capacity < int64_t(sub.size()))
    return fail(PIC_ERR_WORKSPACE, "%lld piece offsets needed, room for %lld",
                (long long)sub.size(), (long long)piece_capacity);
  if (!piece_offsets) return fail(PIC_ERR_NULL, "piece_offsets is NULL");
  std::copy(sub.begin(), sub.end(), piece_offsets);
  std::copy(chain_off.begin(), chain_off.end(), seg_pieces);
  return ok();
}

size_t pic_segment_build_split_workspace(int form, int batch, int heads, int dk, int dv,
                                         int64_t n_tokens, int32_t n_seg, int32_t n_split) {
  if (n_seg < 0 || n_split < 1 || n_tokens < 0 || batch < 1 || heads < 1 || dk < 1 || dv < 1)
    return 0;
  // a segment of c chunks gives at most min(n_split, max(c, 1)) pieces, and
  // sum over segments of max(c, 1) <= n_tokens / 64 + 2 n_seg
  const int64_t P = std::min<int64_t>(int64_t(n_seg) * n_split, n_tokens / 64 + 2 * int64_t(n_seg));
  return std::max(split_layout(form, batch, heads, dk, dv, P, n_seg).total,
                  build_ws_bytes(n_seg));
}

int pic_segment_build_split(int form, int qkv_dtype, int precision, int batch, int heads, int dk,
                            int dv, int64_t n_tokens, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, const int64_t* seg_offsets,
                            int32_t n_seg, int32_t n_split, float* log_scale, float* T_hat,
                            float* S0, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_split < 1) return fail(PIC_ERR_DIMS, "n_split (%d) must be >= 1", n_split);
  if (n_split == 1)
    return pic_segment_build(form, qkv_dtype, precision, batch, heads, dk, dv, n_tokens, q, k, v,
                             alpha, beta, seg_offsets, n_seg, log_scale, T_hat, S0, workspace,
                             workspace_bytes, stream);
  if (int rc = validate_build_args(form, qkv_dtype, precision, batch, heads, dk, dv, n_tokens, q,
                                   k, v, alpha, beta, seg_offsets, n_seg, log_scale, T_hat, S0,
                                   workspace, workspace_bytes, SIZE_MAX))
    return rc;
  std::vector<int64_t> chain_off;
  const std::vector<int64_t> sub = split_pieces(seg_offsets, n_seg, n_split, chain_off);
  const int64_t P = int64_t(sub.size()) - 1;
  if (P > 0x7fffffffLL || mul_sizes({P, batch, heads, dk, std::max(dk, dv)}) < 0)
    return fail(PIC_ERR_DIMS, "the pieces' sizes overflow 64-bit indexing");
  const SplitLayout L = split_layout(form, batch, heads, dk, dv, P, n_seg);
  if (!workspace || workspace_bytes < L.total)
    return fail(PIC_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                workspace ? workspace_bytes : size_t(0));
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* p_lam = reinterpret_cast<float*>(ws + L.lam);
  float* p_T = has_T_hat(form) ? reinterpret_cast<float*>(ws + L.T) : nullptr;
  float* p_S = reinterpret_cast<float*>(ws + L.S);
  if (int rc = enqueue_build(form, qkv_dtype, precision, batch, heads, dk, dv, n_tokens, k, v,
                             alpha, beta, sub.data(), int32_t(P), p_lam, p_T, p_S, ws + L.plan, s))
    return rc;
  // merge: segment i's pair is the chain pair of pieces chain_off[i] .. in order
  std::vector<int32_t> idx(static_cast<size_t>(P));
  for (int64_t j = 0; j < P; ++j) idx[size_t(j)] = int32_t(j);
  pic::ComposeArgs a{form,  batch,    heads,   dk,      dv,     P,      p_lam,     p_T,
                     p_S,   n_seg,    nullptr, nullptr, P,      nullptr, S0,       log_scale,
                     T_hat, false,    {},      {}};
  if (int rc = enqueue_chains(n_seg, chain_off.data(), idx.data(), ws + L.chains, s, a)) return rc;
  hipError_t e = has_T_hat(form) ? pic::launch_compose_dense(a, s)
                                 : pic::launch_compose_elementwise(a, false, s);
  if (e != hipSuccess) return hip_fail(e, "launching the merge of the pieces");
  e = pic::launch_chain_log_scale(a, s);
  if (e != hipSuccess) return hip_fail(e, "launching the merge of the pieces' log-scales");
  if (T_hat) {
    e = pic::launch_chain_T_hat(a, s);
    if (e != hipSuccess) return hip_fail(e, "launching the merge of the pieces' operators");
  }
  return ok();
}

int pic_compose_noalloc(int form, int batch, int heads, int dk, int dv, int64_t pool_size,
                        const float* pool_log_scale, const float* pool_T_hat,
                        const float* pool_S0, int32_t n_req, const int64_t* chain_offsets,
                        const int32_t* chain_idx, const float* S_in, float* S_out,
                        float* log_scale_out, float* T_hat_out, void* stream) {
  // validation as for pic_compose, with the static scratch as the workspace
  // (a stand-in address: validation never dereferences it)
  if (n_req >= 0 && chain_offsets && chain_offsets[0] == 0) {
    bool mono = true;
    for (int32_t r = 0; r < n_req && mono; ++r) mono = chain_offsets[r + 1] >= chain_offsets[r];
    if (mono) {
      const size_t need = compose_ws_bytes(n_req, chain_offsets[n_req]);
      if (need > kScratchBytes)
        return fail(PIC_ERR_WORKSPACE,
                    "chain tables of %zu bytes exceed the static scratch of %zu bytes", need,
                    kScratchBytes);
    }
  }
  if (int rc = pic_validate_compose(form, batch, heads, dk, dv, pool_size, pool_log_scale,
                                    pool_T_hat, pool_S0, n_req, chain_offsets, chain_idx, S_in,
                                    S_out, log_scale_out, T_hat_out,
                                    reinterpret_cast<void*>(uintptr_t(kAlign)), kScratchBytes))
    return rc;
  if (n_req == 0) return ok();
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e, "looking up the static scratch");
  hipStream_t s = static_cast<hipStream_t>(stream);
  pic::ComposeArgs a{form,    batch,    heads,    dk,     dv,       pool_size,
                     pool_log_scale, pool_T_hat, pool_S0, n_req, nullptr, nullptr,
                     chain_offsets[n_req], S_in, S_out, log_scale_out, T_hat_out, false, {}, {}};
  // the tables always go through the scratch (never the kernel arguments)
  if (int rc = enqueue_chains(n_req, chain_offsets, chain_idx, ws, s, a, true)) return rc;
  e = has_T_hat(form) ? pic::launch_compose_dense(a, s) : pic::launch_compose_elementwise(a, false, s);
  if (e != hipSuccess) return hip_fail(e, "launching the compose kernel");
  if (log_scale_out) {
    e = pic::launch_chain_log_scale(a, s);
    if (e != hipSuccess) return hip_fail(e, "launching the chain log-scale kernel");
  }
  if (T_hat_out) {
    e = pic::launch_chain_T_hat(a, s);
    if (e != hipSuccess) return hip_fail(e, "launching the chain operator kernel");
  }
  return ok();
}

int pic_naive_add(int batch, int heads, int dk, int dv, int64_t pool_size, const float* pool_S0,
                  int32_t n_req, const int64_t* chain_offsets, const int32_t* chain_idx,
                  const float* S_in, float* S_out, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (int rc = pic_validate_naive_add(batch, heads, dk, dv, pool_size, pool_S0, n_req,
                                      chain_offsets, chain_idx, S_in, S_out, workspace,
                                      workspace_bytes))
    return rc;
  if (n_req == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  pic::ComposeArgs a{PIC_FORM_SCALAR, batch,   heads,   dk,    dv,      pool_size,
                     nullptr,         nullptr, pool_S0, n_req, nullptr, nullptr,
                     chain_offsets[n_req], S_in, S_out, nullptr, nullptr, false, {}, {}};
  if (int rc = enqueue_chains(n_req, chain_offsets, chain_idx, workspace, s, a)) return rc;
  hipError_t e = pic::launch_compose_elementwise(a, true, s);
  if (e != hipSuccess) return hip_fail(e, "launching the naive-add kernel");
  return ok();
}

/* ------------------------------------------------------ compose with seams */

size_t pic_compose_seams_workspace(int32_t n_req, int64_t chain_total) {
  return compose_seams_ws_bytes(n_req, chain_total);
}

int pic_validate_compose_seams(int form, int qkv_dtype, int batch, int heads, int dk, int dv,
                               int64_t pool_size, const float* pool_log_scale,
                               const float* pool_T_hat, const float* pool_S0, int32_t n_req,
                               const int64_t* chain_offsets, const int32_t* chain_idx,
                               const int64_t* seam_offsets, int64_t n_seam, const void* q,
                               const void* k, const void* v, const float* alpha,
                               const float* beta, const float* S_in, const float* S_out,
                               const float* O_out, const void* workspace,
                               size_t workspace_bytes) {
  (void)S_in;
  if (form < PIC_FORM_SCALAR || form > PIC_FORM_KDA)
    return fail(PIC_ERR_UNSUPPORTED, "unknown form %d", form);
  if (qkv_dtype != PIC_DT_F32 && qkv_dtype != PIC_DT_BF16)
    return fail(PIC_ERR_UNSUPPORTED, "unknown qkv dtype %d", qkv_dtype);
  if (int rc = check_common_dims(batch, heads, dk, dv)) return rc;
  if (n_seam < 0) return fail(PIC_ERR_DIMS, "n_seam must be >= 0");
  if (mul_sizes({pool_size, batch, heads, dk, std::max(dk, dv)}) < 0 ||
      mul_sizes({n_req, batch, heads, dk, dv}) < 0 ||
      mul_sizes({batch, n_seam, heads, std::max(dk, dv)}) < 0)
    return fail(PIC_ERR_DIMS, "sizes overflow 64-bit indexing");
  if (int rc = check_chains(pool_size, n_req, chain_offsets, chain_idx)) return rc;
  const int64_t total = chain_offsets[n_req];
  if (!seam_offsets) return fail(PIC_ERR_NULL, "seam_offsets is NULL");
  if (seam_offsets[0] != 0)
    return fail(PIC_ERR_OFFSETS, "seam_offsets[0] = %lld, must be 0", (long long)seam_offsets[0]);
  for (int64_t c = 0; c < total; ++c) {
    const int64_t w = seam_offsets[c + 1] - seam_offsets[c];
    if (w < 0) return fail(PIC_ERR_OFFSETS, "seam_offsets decrease at chain entry %lld", (long long)c);
    if (w > pic::kMaxSeam)
      return fail(PIC_ERR_DIMS, "seam window of chain entry %lld has %lld tokens (at most %d)",
                  (long long)c, (long long)w, pic::kMaxSeam);
  }
  if (seam_offsets[total] != n_seam)
    return fail(PIC_ERR_OFFSETS, "seam_offsets[chain_total] = %lld, must equal n_seam = %lld",
                (long long)seam_offsets[total], (long long)n_seam);
  if (n_req > 0 && !S_out) return fail(PIC_ERR_NULL, "S_out is required");
  if (total > 0 && (!pool_S0 || !pool_log_scale))
    return fail(PIC_ERR_NULL, "pool_S0 and pool_log_scale are required");
  if (total > 0 && has_T_hat(form) && !pool_T_hat)
    return fail(PIC_ERR_NULL, "pool_T_hat is required for the dense and KDA forms");
  if (!has_T_hat(form) && pool_T_hat)
    return fail(PIC_ERR_UNSUPPORTED, "pool_T_hat must be NULL for scalar and diagonal forms");
  if (n_seam > 0 && (!q || !k || !v || !alpha || !O_out))
    return fail(PIC_ERR_NULL, "q, k, v, alpha and O_out are required when there are seam tokens");
  if (int rc = check_align({pool_log_scale, pool_T_hat, pool_S0, S_in, S_out, q, k, v, alpha,
                            beta, O_out, workspace}))
    return rc;
  const size_t need = compose_seams_ws_bytes(n_req, total);
  if (!workspace || workspace_bytes < need)
    return fail(PIC_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  return ok();
}

int pic_compose_seams(int form, int qkv_dtype, int batch, int heads, int dk, int dv,
                      int64_t pool_size, const float* pool_log_scale, const float* pool_T_hat,
                      const float* pool_S0, int32_t n_req, const int64_t* chain_offsets,
                      const int32_t* chain_idx, const int64_t* seam_offsets, int64_t n_seam,
                      const void* q, const void* k, const void* v, const float* alpha,
                      const float* beta, const float* S_in, float* S_out, float* O_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = pic_validate_compose_seams(form, qkv_dtype, batch, heads, dk, dv, pool_size,
                                          pool_log_scale, pool_T_hat, pool_S0, n_req,
                                          chain_offsets, chain_idx, seam_offsets, n_seam, q, k,
                                          v, alpha, beta, S_in, S_out, O_out, workspace,
                                          workspace_bytes))
    return rc;
  if (n_req == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t total = chain_offsets[n_req];
  pic::SeamArgs a{};
  a.c = pic::ComposeArgs{form,    batch,    heads,    dk,     dv,       pool_size,
                         pool_log_scale, pool_T_hat, pool_S0, n_req, nullptr, nullptr,
                         total, S_in, S_out, nullptr, nullptr, false, {}, {}};
  a.qkv_bf16 = qkv_dtype == PIC_DT_BF16;
  a.n_seam = n_seam;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = has_T_hat(form) ? beta : nullptr;  // dense and KDA erase along k
  a.O = O_out;
  a.c.inl = n_req <= pic::kInlineReq && total <= pic::kInlineIdx;
  if (a.c.inl) {
    std::copy(chain_offsets, chain_offsets + n_req + 1, a.c.inl_off);
    if (total > 0) std::copy(chain_idx, chain_idx + total, a.c.inl_idx);
    std::copy(seam_offsets, seam_offsets + total + 1, a.inl_seam_off);
  } else {
    char* ws = static_cast<char*>(workspace);
    int64_t* o = reinterpret_cast<int64_t*>(ws);
    int32_t* i = reinterpret_cast<int32_t*>(ws + align_up(sizeof(int64_t) * (size_t(n_req) + 1)));
    int64_t* so = reinterpret_cast<int64_t*>(ws + compose_ws_bytes(n_req, total));
    const hipError_t e = staging().copy(
        {{o, chain_offsets, sizeof(int64_t) * (size_t(n_req) + 1)},
         {i, chain_idx, total > 0 ? sizeof(int32_t) * size_t(total) : size_t(0)},
         {so, seam_offsets, sizeof(int64_t) * (size_t(total) + 1)}},
        s);
    if (e != hipSuccess) return hip_fail(e, "copying the chain and seam tables");
    a.c.d_chain_off = o;
    a.c.d_chain_idx = i;
    a.d_seam_off = so;
  }
  const hipError_t e = pic::launch_compose_seams(a, s);
  if (e != hipSuccess) return hip_fail(e, "launching the seam compose kernel");
  return ok();
}

/* ------------------------------------------------------------ re-rotation */

static size_t rerotate_ws_bytes(int32_t n) {
  if (n < 0) return 0;
  const size_t m = size_t(std::max<int32_t>(n, 1));
  return align_up(sizeof(int32_t) * m) + align_up(sizeof(int64_t) * m);
}

size_t pic_rerotate_workspace(int32_t n) { return rerotate_ws_bytes(n); }


int pic_validate_rerotate(int form, int batch, int heads, int dk, int dv, int64_t pool_size,
                          const float* pool_log_scale, const float* pool_T_hat,
                          const float* pool_S0, int32_t n, const int32_t* idx,
                          const int64_t* shift, int rot_dim, double rope_base, int pairing,
                          const float* log_scale_out, const float* T_hat_out,
                          const float* S0_out, const void* workspace, size_t workspace_bytes) {
  if (form < PIC_FORM_SCALAR || form > PIC_FORM_KDA)
    return fail(PIC_ERR_UNSUPPORTED, "unknown form %d", form);
  if (pairing != PIC_ROPE_INTERLEAVED && pairing != PIC_ROPE_HALF)
    return fail(PIC_ERR_UNSUPPORTED, "unknown pairing %d", pairing);
  if (!(rope_base > 0.0) || !std::isfinite(rope_base))
    return fail(PIC_ERR_UNSUPPORTED, "rope_base must be positive and finite");
  if (int rc = check_common_dims(batch, heads, dk, dv)) return rc;
  if (rot_dim < 8 || rot_dim > dk || rot_dim % 8 != 0)
    return fail(PIC_ERR_DIMS, "rot_dim (%d) must be a multiple of 8 in [8, dk = %d]", rot_dim, dk);
  if (n < 0) return fail(PIC_ERR_DIMS, "n (%d) must be >= 0", n);
  if (pool_size < 0) return fail(PIC_ERR_DIMS, "pool_size must be >= 0");
  const int64_t per = (form == PIC_FORM_DIAG) ? dk : 1;
  if (mul_sizes({pool_size, batch, heads, dk, std::max(dk, dv)}) < 0 ||
      mul_sizes({n, batch, heads, dk, std::max(dk, dv)}) < 0)
    return fail(PIC_ERR_DIMS, "sizes overflow 64-bit indexing");
  if (n == 0) return ok();
  if (!idx || !shift) return fail(PIC_ERR_NULL, "idx and shift are required");
  for (int32_t j = 0; j < n; ++j)
    if (idx[j] < 0 || int64_t(idx[j]) >= pool_size)
      return fail(PIC_ERR_CHAIN, "idx[%d] = %d outside [0, %lld)", j, idx[j], (long long)pool_size);
  if (!pool_log_scale || !pool_S0 || !log_scale_out || !S0_out)
    return fail(PIC_ERR_NULL, "pool_log_scale, pool_S0, log_scale_out and S0_out are required");
  if (has_T_hat(form) && (!pool_T_hat || !T_hat_out))
    return fail(PIC_ERR_NULL, "pool_T_hat and T_hat_out are required for the dense and KDA forms");
  if (!has_T_hat(form) && (pool_T_hat || T_hat_out))
    return fail(PIC_ERR_UNSUPPORTED, "T_hat must be NULL for scalar and diagonal forms");
  if (int rc = check_align({pool_log_scale, pool_T_hat, pool_S0, log_scale_out, T_hat_out, S0_out,
                            workspace}))
    return rc;
  const int64_t units_in = pool_size * batch * heads, units_out = int64_t(n) * batch * heads;
  const int64_t lam_in = units_in * per * 4, lam_out = units_out * per * 4;
  const int64_t t_in = units_in * dk * dk * 4, t_out = units_out * dk * dk * 4;
  const int64_t s_in = units_in * dk * dv * 4, s_out = units_out * dk * dv * 4;
  const void* ins[3] = {pool_log_scale, pool_T_hat, pool_S0};
  const int64_t in_b[3] = {lam_in, t_in, s_in};
  const void* outs[3] = {log_scale_out, T_hat_out, S0_out};
  const int64_t out_b[3] = {lam_out, t_out, s_out};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 3; ++i)
      if (overlap(outs[o], out_b[o], ins[i], in_b[i]))
        return fail(PIC_ERR_UNSUPPORTED, "output %d overlaps the pool", o);
    for (int p = o + 1; p < 3; ++p)
      if (overlap(outs[o], out_b[o], outs[p], out_b[p]))
        return fail(PIC_ERR_UNSUPPORTED, "outputs %d and %d overlap", o, p);
  }
  const size_t need = rerotate_ws_bytes(n);
  if (!workspace || workspace_bytes < need)
    return fail(PIC_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  return ok();
}

int pic_rerotate(int form, int batch, int heads, int dk, int dv, int64_t pool_size,
                 const float* pool_log_scale, const float* pool_T_hat, const float* pool_S0,
                 int32_t n, const int32_t* idx, const int64_t* shift, int rot_dim,
                 double rope_base, int pairing, float* log_scale_out, float* T_hat_out,
                 float* S0_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = pic_validate_rerotate(form, batch, heads, dk, dv, pool_size, pool_log_scale,
                                     pool_T_hat, pool_S0, n, idx, shift, rot_dim, rope_base,
                                     pairing, log_scale_out, T_hat_out, S0_out, workspace,
                                     workspace_bytes))
    return rc;
  if (n == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* d_idx = reinterpret_cast<int32_t*>(ws);
  int64_t* d_shift = reinterpret_cast<int64_t*>(ws + align_up(sizeof(int32_t) * size_t(n)));
  hipError_t e = staging().copy({{d_idx, idx, sizeof(int32_t) * size_t(n)},
                                 {d_shift, shift, sizeof(int64_t) * size_t(n)}},
                                s);
  if (e != hipSuccess) return hip_fail(e, "copying the re-rotation tables");
  pic::RotateArgs a{form,    batch,   heads,   dk,      dv,        pool_log_scale,
                    pool_T_hat, pool_S0, n,    d_idx,   d_shift,   rot_dim,
                    rope_base, pairing == PIC_ROPE_HALF, log_scale_out, T_hat_out, S0_out};
  e = pic::launch_rerotate(a, s);
  if (e != hipSuccess) return hip_fail(e, "launching the re-rotation kernel");
  return ok();
}

/* ------------------------------------------------------------ conv warm-up */

static size_t conv_ws_bytes(int32_t n) {
  if (n < 0) return 0;
  const size_t m = size_t(std::max<int32_t>(n, 1));
  return 2 * align_up(sizeof(int64_t) * m) + align_up(sizeof(int32_t) * m);
}

size_t pic_conv_warmup_workspace(int32_t n) { return conv_ws_bytes(n); }

int pic_validate_conv_warmup(int x_dtype, int batch, int heads, int dc, int width,
                             int64_t n_tokens, const float* weight, const void* x, int32_t n,
                             int32_t n_warm, const int64_t* head_start, const int64_t* hist_end,
                             const int32_t* hist_len, const void* y_out, const void* workspace,
                             size_t workspace_bytes) {
  if (x_dtype != PIC_DT_F32 && x_dtype != PIC_DT_BF16)
    return fail(PIC_ERR_UNSUPPORTED, "unknown dtype %d", x_dtype);
  if (int rc = check_common_dims(batch, heads, dc, dc)) return rc;
  if (width < 1 || width > PIC_MAX_CONV)
    return fail(PIC_ERR_DIMS, "width (%d) must be in [1, %d]", width, PIC_MAX_CONV);
  if (n < 0 || n_warm < 0 || n_warm > PIC_MAX_SEAM || n_tokens < 0)
    return fail(PIC_ERR_DIMS, "n, n_tokens >= 0 and n_warm in [0, %d] required", PIC_MAX_SEAM);
  if (mul_sizes({batch, n_tokens, heads, dc}) < 0 || mul_sizes({batch, n, n_warm, heads, dc}) < 0)
    return fail(PIC_ERR_DIMS, "sizes overflow 64-bit indexing");
  if (n > 0 && (!head_start || !hist_end || !hist_len))
    return fail(PIC_ERR_NULL, "head_start, hist_end and hist_len are required");
  for (int32_t e = 0; e < n; ++e) {
    if (hist_len[e] < 0 || hist_len[e] > width - 1)
      return fail(PIC_ERR_OFFSETS, "hist_len[%d] = %d outside [0, width - 1]", e, hist_len[e]);
    if (hist_len[e] > 0 && (hist_end[e] < hist_len[e] || hist_end[e] > n_tokens))
      return fail(PIC_ERR_OFFSETS, "history of entry %d outside the %lld tokens", e,
                  (long long)n_tokens);
    if (n_warm > 0 && (head_start[e] < 0 || head_start[e] > n_tokens - n_warm))
      return fail(PIC_ERR_OFFSETS, "head of entry %d outside the %lld tokens", e,
                  (long long)n_tokens);
  }
  if (int64_t(n) * n_warm == 0) return ok();
  if (!weight || !x || !y_out) return fail(PIC_ERR_NULL, "weight, x and y_out are required");
  if (int rc = check_align({weight, x, y_out, workspace})) return rc;
  const int64_t es = (x_dtype == PIC_DT_BF16) ? 2 : 4;
  const int64_t y_b = int64_t(batch) * n * n_warm * heads * dc * es;
  if (overlap(y_out, y_b, x, int64_t(batch) * n_tokens * heads * dc * es) ||
      overlap(y_out, y_b, weight, int64_t(heads) * dc * width * 4))
    return fail(PIC_ERR_UNSUPPORTED, "y_out overlaps x or weight");
  const size_t need = conv_ws_bytes(n);
  if (!workspace || workspace_bytes < need)
    return fail(PIC_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  return ok();
}

int pic_conv_warmup(int x_dtype, int batch, int heads, int dc, int width, int64_t n_tokens,
                    const float* weight, const void* x, int32_t n, int32_t n_warm,
                    const int64_t* head_start, const int64_t* hist_end, const int32_t* hist_len,
                    void* y_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = pic_validate_conv_warmup(x_dtype, batch, heads, dc, width, n_tokens, weight, x, n,
                                        n_warm, head_start, hist_end, hist_len, y_out, workspace,
                                        workspace_bytes))
    return rc;
  if (int64_t(n) * n_warm == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const size_t b64 = align_up(sizeof(int64_t) * size_t(n));
  int64_t* d_head = reinterpret_cast<int64_t*>(ws);
  int64_t* d_hend = reinterpret_cast<int64_t*>(ws + b64);
  int32_t* d_hlen = reinterpret_cast<int32_t*>(ws + 2 * b64);
  hipError_t e = staging().copy({{d_head, head_start, sizeof(int64_t) * size_t(n)},
                                 {d_hend, hist_end, sizeof(int64_t) * size_t(n)},
                                 {d_hlen, hist_len, sizeof(int32_t) * size_t(n)}},
                                s);
  if (e != hipSuccess) return hip_fail(e, "copying the warm-up tables");
  pic::ConvArgs a{x_dtype == PIC_DT_BF16, batch, heads, dc, width, n_tokens, weight, x, n,
                  n_warm, d_hend, d_hlen, d_head, y_out};
  e = pic::launch_conv_warmup(a, s);
  if (e != hipSuccess) return hip_fail(e, "launching the warm-up kernel");
  return ok();
}

/* ------------------------------------------------------------ materialize */

int pic_materialize_T(int form, int64_t n_units, int dk, const float* log_scale,
                      const float* T_hat, float* T_out, void* stream) {
  if (form < PIC_FORM_SCALAR || form > PIC_FORM_KDA)
    return fail(PIC_ERR_UNSUPPORTED, "unknown form %d", form);
  if (!dim_ok(dk)) return fail(PIC_ERR_DIMS, "dk (%d) must be a multiple of 16 in [16, 128]", dk);
  if (n_units < 0 || mul_sizes({n_units, dk, dk}) < 0)
    return fail(PIC_ERR_DIMS, "bad n_units");
  if (n_units == 0) return ok();
  if (!log_scale || !T_out) return fail(PIC_ERR_NULL, "log_scale and T_out are required");
  if (has_T_hat(form) && !T_hat) return fail(PIC_ERR_NULL, "T_hat is required");
  if (!has_T_hat(form) && T_hat)
    return fail(PIC_ERR_UNSUPPORTED, "T_hat must be NULL for scalar and diagonal forms");
  if (int rc = check_align({log_scale, T_hat, T_out})) return rc;
  hipError_t e = pic::launch_materialize_T(form, n_units, dk, log_scale, T_hat, T_out,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching the materialize kernel");
  return ok();
}

/* -------------------------------------------------------------- plan dump */

int pic_plan_dump(int kind, int32_t n, const int64_t* offsets, const int32_t* chain_idx,
                  int64_t limit, int64_t* table, int64_t table_rows) {
  if (!table && table_rows > 0) return fail(PIC_ERR_NULL, "table is NULL");
  if (kind == PIC_PLAN_BUILD) {
    if (n < 1) return fail(PIC_ERR_DIMS, "n_seg (%d) must be >= 1", n);
    if (limit < 0) return fail(PIC_ERR_DIMS, "n_tokens must be >= 0");
    if (chain_idx) return fail(PIC_ERR_UNSUPPORTED, "chain_idx must be NULL for a build plan");
    if (int rc = check_seg_offsets(offsets, n, limit)) return rc;
    if (table_rows < n)
      return fail(PIC_ERR_WORKSPACE, "table of %d rows needed, %lld given", n,
                  (long long)table_rows);
    if (!table) return fail(PIC_ERR_NULL, "table is NULL");
    const std::vector<int32_t> order = build_order(offsets, n);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t seg = order[i];
      const int64_t len = offsets[seg + 1] - offsets[seg];
      const int64_t nch = (len + PIC_CHUNK - 1) / PIC_CHUNK;
      int64_t* row = table + int64_t(i) * PIC_PLAN_BUILD_COLS;
      row[0] = seg;
      row[1] = offsets[seg];
      row[2] = len;
      row[3] = nch;
      row[4] = nch ? len - (nch - 1) * PIC_CHUNK : 0;
    }
    return ok();
  }
  if (kind == PIC_PLAN_COMPOSE) {
    if (int rc = check_chains(limit, n, offsets, chain_idx)) return rc;
    const int64_t total = offsets[n];
    if (table_rows < total)
      return fail(PIC_ERR_WORKSPACE, "table of %lld rows needed, %lld given", (long long)total,
                  (long long)table_rows);
    for (int32_t r = 0; r < n; ++r)
      for (int64_t c = offsets[r]; c < offsets[r + 1]; ++c) {
        int64_t* row = table + c * PIC_PLAN_COMPOSE_COLS;
        row[0] = r;
        row[1] = c - offsets[r];
        row[2] = chain_idx[c];
      }
    return ok();
  }
  return fail(PIC_ERR_UNSUPPORTED, "unknown plan kind %d", kind);
}

}  // extern "C"
