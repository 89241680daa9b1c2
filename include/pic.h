/*
 * pic.h -- C ABI of the linear-attention segment transform used by
 * position-independent caching (PIC) for hybrid-attention LLMs (HYPIC),
 * implemented for AMD MI355X (gfx950) with HIP.
 *
 * The method.  A linear-attention layer keeps, per head, a recurrent state
 * S in R^{dk x dv}; every token applies a linear transition T_t to it and
 * adds a write term:  S_t = T_t S_{t-1} + beta_t k_t v_t^T.  For a prompt
 * segment C this library computes the cached pair
 *     T_C    = T_L ... T_1            (product of the token transitions)
 *     S(C|0) = final state of C started from S = 0,
 * which depends on the segment's own tokens only, and on reuse composes
 *     S(C1.C2) = T(C2) S(C1) + S(C2)
 * (left-multiply the running state by T_C, then add S(C|0)), in time
 * independent of the segment length.
 *   [xix.ai HYPIC article (French), paragraph on linear layers: transition
 *    operators, the composition identity, prefix independence, the failure
 *    of plain addition under decay / gating / delta erasure.
 *    remio.ai HYPIC article (Japanese), section on how HYPIC composes
 *    linear-attention states: cache at first prefill, reuse by applying the
 *    cached transition and adding the zero-start contribution; scalar,
 *    diagonal and dense transition forms.]
 *
 * Transition families (the pages name RetNet/Mamba2, GLA and DeltaNet/GDN;
 * the per-token formulas are the plainest reading of each family):
 *     PIC_FORM_SCALAR  T_t = alpha_t I                     beta = 1
 *     PIC_FORM_DIAG    T_t = Diag(alpha_t), alpha_t in (0,1]^dk, beta = 1
 *     PIC_FORM_DENSE   T_t = alpha_t (I - beta_t k_t k_t^T)   (GDN form)
 *     PIC_FORM_KDA     T_t = (I - beta_t k_t k_t^T) Diag(alpha_t),
 *                      alpha_t in (0,1]^dk            (KDA form: per-channel
 *                      gates inside the delta rule)
 * For every form S_t = T_t S_{t-1} + beta_t k_t v_t^T (beta = 1 where the
 * table above fixes it).
 *
 * Split operator.  At realistic gates T_C underflows fp32 within a few
 * thousand tokens, so the operator is returned as
 *     T_C = e^{lambda_C} * That_C,   lambda_C = sum_t ln(alpha_t)
 * with lambda per head (scalar, dense) or per key channel (diagonal), and
 * That_C = prod_t (I - beta_t k_t k_t^T) (dense only; I for the others).
 * KDA: the gates do not factor out of the product, so each token gives up
 * its largest gate m_t = max_i alpha_t,i:
 *     lambda_C = sum_t ln(m_t),  That_C = prod_t (I - beta_t k_t k_t^T) Diag(alpha_t / m_t)
 * (the dense split when all channels share one gate; ||That_C||_2 <= 1 for
 * beta |k|^2 <= 2).  Everywhere below "dense" pairs (a per-head lambda and a
 * That) include the KDA form's: compose and materialize treat the two alike.
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major (last index fastest).  Device pointers
 *     must be 16-byte aligned (PIC_ERR_ALIGN otherwise) and point to memory
 *     of the current HIP device.  Host arrays (offsets, chains) are read during the call only.
 *   - Layout of per-token inputs:  k, q [batch][n_tokens][heads][dk],
 *     v [batch][n_tokens][heads][dv], alpha [batch][n_tokens][heads]
 *     (diag, KDA: [batch][n_tokens][heads][dk]), beta [batch][n_tokens][heads].
 *     "batch" indexes independent layers (or layer-sized groups); segments
 *     are token ranges shared by all of them.
 *   - Layout of pairs (a "pool" of cached segments, and the build output):
 *     log_scale [P][batch][heads] (diag: [P][batch][heads][dk]),
 *     T_hat [P][batch][heads][dk][dk] (dense), S0 [P][batch][heads][dk][dv].
 *     The build writes segment s of the call at pool index s.
 *   - States: S_in, S_out [n_req][batch][heads][dk][dv], fp32.
 *   - Ownership: every buffer belongs to the caller.  The library allocates
 *     no device memory; the per-call tables (segment offsets and order,
 *     chain tables) go into the caller's workspace (size from the
 *     *_workspace query).  Small tables (builds of up to 32 segments,
 *     composes of up to 16 requests and 64 chain entries) travel in the
 *     kernel arguments instead and leave the workspace untouched.  Larger
 *     ones are copied from host memory, and the call then waits for its stream
 *     (the source is gone once the call returns); the library holds no
 *     memory between calls.  A caller that wants those copies asynchronous
 *     opts into a pinned host pool with pic_staging_reserve() and frees it
 *     with pic_staging_release().  Calls are not safe under stream capture.
 *   - Asynchrony: a return of PIC_OK means the work is validated and
 *     enqueued on `stream` (a hipStream_t; NULL = the null stream).  Results
 *     are ready once the stream is synchronised.  Host arrays may be reused
 *     as soon as the call returns.
 *   - Errors: a negative PIC_ERR_* code.  Every argument check happens on
 *     the host before any HIP call; on error nothing is enqueued and no
 *     output is touched, except PIC_ERR_HIP (a launch or copy failed after
 *     validation).  pic_last_error() gives a per-thread message.  No C++
 *     exception crosses this interface.  Calls are thread-safe.
 *   - Preconditions not checked on the device: 0 < alpha <= 1, finite
 *     inputs.  Empty segments are allowed and give the identity pair
 *     (lambda = 0, That = I, S0 = 0); an empty chain gives S_out = S_in.
 *   - Supported sizes: dk, dv multiples of 16 in [16, 128]; heads, batch >= 1;
 *     n_seg >= 1 (build).  Other sizes return PIC_ERR_DIMS.
 */
#ifndef PIC_H_
#define PIC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PIC_ABI_VERSION 11

enum pic_form { PIC_FORM_SCALAR = 0, PIC_FORM_DIAG = 1, PIC_FORM_DENSE = 2, PIC_FORM_KDA = 3 };
enum pic_dtype { PIC_DT_F32 = 0, PIC_DT_BF16 = 1 };

/* Arithmetic of the build's matrix-core products (the state and every
 * accumulation are fp32 in both):
 *   PIC_PREC_FP32  fp32-accurate: an fp32 operand is split into two bf16
 *                  terms and a product takes up to three bf16 products
 *                  (~2^-16 relative per product); all forms and dtypes.
 *   PIC_PREC_FP16  one fp16 product per operand pair (11 significant bits);
 *                  dense form with bf16 k/v, and KDA form with bf16 k/v and
 *                  dk = dv = 128 (gate range: see pic_segment_build).  The
 *                  ungated product That
 *                  is kept at a power-of-two column scale internally, so its
 *                  decay along a segment does not leave fp16's range; keys
 *                  are assumed unit-norm (beta |k|^2 <= 2), |v| well below
 *                  6e4 and |S| below about 2e3 (the state is kept at up to
 *                  32x its size between decays).  Typical relative Frobenius error against fp64
 *                  at 4096-8192 tokens: ~2e-3 on That, ~3e-4 on S(C|0).
 *                  Inputs outside these bounds can overflow an fp16 operand;
 *                  the kernels then flag it on the device (the stored values
 *                  are inf or NaN) and pic_nonfinite_check reports it. */
enum pic_precision { PIC_PREC_FP32 = 0, PIC_PREC_FP16 = 1 };

enum pic_status {
  PIC_OK = 0,
  PIC_ERR_NULL = -1,        /* a required pointer is NULL                        */
  PIC_ERR_DIMS = -2,        /* unsupported or inconsistent sizes                 */
  PIC_ERR_OFFSETS = -3,     /* offsets[0] != 0, decreasing, or last != n_tokens  */
  PIC_ERR_CHAIN = -4,       /* chain offsets bad or an index outside [0, pool)   */
  PIC_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than the query result   */
  PIC_ERR_UNSUPPORTED = -6, /* unknown form or dtype                             */
  PIC_ERR_HIP = -7,         /* a HIP call failed after validation                */
  PIC_ERR_ALIGN = -8,       /* a device pointer is not 16-byte aligned           */
  PIC_ERR_NONFINITE = -9    /* pic_nonfinite_check: an fp16-operand call stored a
                               value that is not finite                          */
};

/* ABI version of the loaded library (PIC_ABI_VERSION at build time). */
int pic_abi_version(void);

/* Static text of a status code. */
const char* pic_status_string(int status);

/* Message of the calling thread's last failing call ("" if none). */
const char* pic_last_error(void);

/* ----------------------------------------------------------------------
 * Pinned staging pool (opt-in).  Plan tables too large for the kernel
 * arguments are copied into the caller's workspace.  Without a pool the copy
 * reads the host arrays directly and the call waits for its stream before it
 * returns.  pic_staging_reserve() allocates, for the current HIP device, a
 * pool of 64 pinned host slots of 64 KiB (4 MiB); from then on tables that
 * fit a slot are staged there and copied asynchronously (a slot is reused
 * once its copy has completed), so back-to-back calls do not wait for the
 * device.  A second reserve on the same device does nothing.
 * pic_staging_release() waits for the pending copies of every pool, frees
 * all of them and returns the library to holding no memory; it must not
 * run concurrently with calls that stage tables.  pic_staging_bytes()
 * gives the pinned bytes held now.  Errors: PIC_ERR_HIP (detail in
 * pic_last_error()).
 * ---------------------------------------------------------------------- */
int pic_staging_reserve(void);
int pic_staging_release(void);
size_t pic_staging_bytes(void);

/* ----------------------------------------------------------------------
 * Segment build: the cached pair of every (segment, layer, head).
 *   [xix.ai HYPIC article, paragraph on linear layers: at a segment's first
 *    prefill, cache (T_C, S(C|0)); both depend only on the segment's tokens.]
 *
 * form        PIC_FORM_*
 * qkv_dtype   storage type of q, k, v: PIC_DT_BF16 or PIC_DT_F32
 * precision   PIC_PREC_FP32, or PIC_PREC_FP16 (dense form with bf16 k/v, or
 *             KDA form with bf16 k/v and dk = dv = 128; any other combination
 *             returns PIC_ERR_UNSUPPORTED).  The KDA build at PIC_PREC_FP32
 *             runs token by token in fp32 on the vector units; at
 *             PIC_PREC_FP16 in chunks of 32 tokens on the matrix cores, whose
 *             operands hold products of up to 16 consecutive gates of a
 *             channel, or their inverses, times k: gates whose 16-token
 *             products in some channel fall below about 2^-16 overflow those
 *             operands, and the stored pair is then not finite and reported
 *             by pic_nonfinite_check.
 * batch, heads, dk, dv, n_tokens   sizes (see layouts above)
 * q           may be NULL; never read: the pair does not depend on queries
 * k, v        device, qkv_dtype
 * alpha       device fp32 gates in (0, 1]
 * beta        device fp32 [batch][n_tokens][heads]; dense and KDA only
 *             (ignored for scalar/diag); NULL means beta = 1
 * seg_offsets HOST int64[n_seg+1]: segment s = tokens [off[s], off[s+1]);
 *             off[0] = 0, non-decreasing, off[n_seg] = n_tokens
 * log_scale   device fp32 out, lambda_C, [n_seg][batch][heads] (diag: [..][dk])
 * T_hat       device fp32 out, That_C [n_seg][batch][heads][dk][dk]; required
 *             for PIC_FORM_DENSE and PIC_FORM_KDA, must be NULL otherwise
 *             (That = I)
 * S0          device fp32 out, S(C|0) [n_seg][batch][heads][dk][dv]
 * workspace   device scratch of at least pic_segment_build_workspace() bytes
 * stream      hipStream_t (NULL = null stream)
 * -------------------------------------------------------------------- */
size_t pic_segment_build_workspace(int form, int batch, int heads, int dk, int dv,
                                   int64_t n_tokens, int32_t n_seg);

int pic_validate_build(int form, int qkv_dtype, int precision, int batch, int heads, int dk, int dv,
                       int64_t n_tokens, const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, const int64_t* seg_offsets,
                       int32_t n_seg, const float* log_scale, const float* T_hat,
                       const float* S0, const void* workspace, size_t workspace_bytes);

int pic_segment_build(int form, int qkv_dtype, int precision, int batch, int heads, int dk, int dv,
                      int64_t n_tokens, const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, const int64_t* seg_offsets,
                      int32_t n_seg, float* log_scale, float* T_hat, float* S0,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * Split build for launches with few (segment, layer, head) units: every
 * segment is cut into up to n_split pieces of whole 64-token chunks (a
 * segment of c chunks gives min(n_split, max(c, 1)) pieces as equal as whole
 * chunks allow), the pieces' pairs are built into the workspace as by
 * pic_segment_build, and each segment's pair is the chain pair of its pieces
 * in token order, merged by the compose of pic_compose:
 *   lambda = sum of the pieces' lambda, That = That_p ... That_1,
 *   S = the composed state of the pieces from zero.
 *   [xix.ai HYPIC article, paragraph on linear layers: the pair of C1.C2 is
 *    S(C1.C2) = T(C2) S(C1) + S(C2), T(C1.C2) = T(C2) T(C1); a segment's pair
 *    is the composition of its parts' pairs.]
 * Equal to pic_segment_build's result up to rounding (the merge is exact in
 * exact arithmetic).  Worth it when n_seg * batch * heads is well below the
 * number of compute units and the segments are long: the pieces fill the
 * GPU, and the merge reads and writes each piece's pair once more.
 *
 * Arguments as pic_segment_build, plus
 * n_split     pieces per segment, >= 1 (1: the plain build)
 * workspace   device scratch of at least pic_segment_build_split_workspace()
 *             bytes: the pieces' pairs, their plan and the merge's tables
 * Errors as pic_segment_build; PIC_ERR_DIMS when n_split < 1 or the pieces'
 * sizes overflow 64-bit indexing.
 * -------------------------------------------------------------------- */
size_t pic_segment_build_split_workspace(int form, int batch, int heads, int dk, int dv,
                                         int64_t n_tokens, int32_t n_seg, int32_t n_split);

/* The pieces pic_segment_build_split cuts (pure host code, no HIP call):
 * writes *n_pieces = P, piece_offsets[0..P] (the pieces' token offsets, in
 * segment order) and seg_pieces[0..n_seg] (segment s's pieces are
 * seg_pieces[s] .. seg_pieces[s+1] - 1).  seg_offsets is checked as in
 * pic_validate_build against n_tokens; piece_capacity is the number of
 * entries piece_offsets holds (PIC_ERR_WORKSPACE, with *n_pieces set, when
 * fewer than P + 1). */
int pic_split_plan(int32_t n_seg, const int64_t* seg_offsets, int64_t n_tokens, int32_t n_split,
                   int64_t* piece_offsets, int64_t piece_capacity, int64_t* seg_pieces,
                   int64_t* n_pieces);

int pic_segment_build_split(int form, int qkv_dtype, int precision, int batch, int heads, int dk,
                            int dv, int64_t n_tokens, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, const int64_t* seg_offsets,
                            int32_t n_seg, int32_t n_split, float* log_scale, float* T_hat,
                            float* S0, void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * Prefill with outputs: the independent prefill of every segment, in which
 * the pair is built, with the per-token outputs of the linear layer.
 *   [remio.ai HYPIC article (Japanese), section on how HYPIC composes
 *    linear-attention states: the pair is built at a segment's first
 *    prefill, a small add-on to it; xix.ai HYPIC article, paragraph on linear
 *    layers.]
 * Every segment starts from the zero state; after token t's update
 * S_t = T_t S_(t-1) + beta_t k_t v_t^T its output is o_t = S_t^T q_t (the
 * readout of the state that includes the token; no scale: a model's 1/sqrt(d)
 * belongs to q).  Besides O the call writes the segment's pair exactly as
 * pic_segment_build does: log_scale and S0 always, T_hat when given (That
 * tracked alongside the prefill; T_hat = NULL leaves it out, which is the
 * plain prefill).
 * Provided for the dense form (PIC_FORM_DENSE) with bf16 q, k, v at fp16
 * operand precision (the arithmetic and preconditions of PIC_PREC_FP16).
 *
 * q, k        device bf16 [batch][n_tokens][heads][dk]
 * v           device bf16 [batch][n_tokens][heads][dv]
 * alpha       device fp32 [batch][n_tokens][heads] in (0, 1]
 * beta        device fp32 [batch][n_tokens][heads], or NULL (= 1)
 * seg_offsets HOST int64[n_seg+1], as for pic_segment_build
 * log_scale   device fp32 out [n_seg][batch][heads]
 * T_hat       device fp32 out [n_seg][batch][heads][dk][dk], or NULL
 * S0          device fp32 out [n_seg][batch][heads][dk][dv]
 * O_out       device bf16 out [batch][n_tokens][heads][dv] (rounded to
 *             nearest even from fp32); must not overlap the inputs
 * workspace   device scratch of at least pic_segment_build_workspace() bytes
 * Errors as for pic_segment_build; PIC_ERR_NULL when q or O_out is NULL with
 * tokens present.
 * -------------------------------------------------------------------- */
int pic_validate_prefill(int batch, int heads, int dk, int dv, int64_t n_tokens, const void* q,
                         const void* k, const void* v, const float* alpha, const float* beta,
                         const int64_t* seg_offsets, int32_t n_seg, const float* log_scale,
                         const float* T_hat, const float* S0, const void* O_out,
                         const void* workspace, size_t workspace_bytes);

int pic_segment_prefill(int batch, int heads, int dk, int dv, int64_t n_tokens, const void* q,
                        const void* k, const void* v, const float* alpha, const float* beta,
                        const int64_t* seg_offsets, int32_t n_seg, float* log_scale,
                        float* T_hat, float* S0, void* O_out, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * Overflow report of the fp16-operand calls (pic_segment_build with
 * PIC_PREC_FP16, pic_segment_prefill).  Those calls are asynchronous and
 * return PIC_OK once launched; a kernel that stores a value that is not
 * finite (an fp16 operand overflowed because the inputs are outside the
 * PIC_PREC_FP16 preconditions) sets a flag word on the device instead.
 * pic_nonfinite_check waits for `stream` (hipStream_t, NULL = null stream),
 * reads the current device's flag and clears it: PIC_OK when no such call
 * since the last check stored a non-finite value, PIC_ERR_NONFINITE when one
 * did (then the outputs of the calls since the last check are suspect).
 * The flag is per device and shared by all streams and threads of the
 * process: check after the work you want covered has been enqueued.
 * Errors: PIC_ERR_HIP when the copy or the synchronisation fails.
 * -------------------------------------------------------------------- */
int pic_nonfinite_check(void* stream);

/* ----------------------------------------------------------------------
 * Compose: fold chains of cached pairs into running states.
 *   [xix.ai HYPIC article, paragraph on linear layers: on reuse,
 *    S <- T_C S + S(C|0), i.e. S(C1.C2) = T(C2) S(C1) + S(C2), constant time
 *    in the segment length.]
 *
 * For request r, chain entries chain_idx[chain_offsets[r] .. chain_offsets[r+1])
 * are applied in order (first entry first):
 *     S <- e^{log_scale_p} * That_p * S + S0_p
 * per (layer, head), starting from S_in[r] (NULL = zero), result in S_out[r].
 *
 * The chain's own pair (optional).  Composition is associative, so a chain
 * p_1..p_n is itself a cached pair: T_chain = T_pn ... T_p1 and
 * S(chain|0) = the result from a zero start.  With log_scale_out and (dense)
 * T_hat_out given, the call also writes
 *     log_scale_out[r] = sum over the chain of log_scale_p
 *     T_hat_out[r]     = That_pn ... That_p1          (dense)
 * (an empty chain gives 0 and I); S(chain|0) is S_out with S_in = NULL.
 *   [xix.ai HYPIC article, paragraph on linear layers: the composition
 *    identity S(C1.C2) = T(C2) S(C1) + S(C2) with T(C1.C2) = T(C2) T(C1).]
 *
 * pool_size      number of pool entries P
 * pool_log_scale device fp32 [P][batch][heads] (diag: [P][batch][heads][dk])
 * pool_T_hat     device fp32 [P][batch][heads][dk][dk]; dense only (else NULL)
 * pool_S0        device fp32 [P][batch][heads][dk][dv]
 * chain_offsets  HOST int64[n_req+1]: off[0] = 0, non-decreasing
 * chain_idx      HOST int32[off[n_req]]: pool indices in [0, pool_size)
 * S_in           device fp32 [n_req][batch][heads][dk][dv] or NULL (= 0)
 * S_out          device fp32 out, same shape; may equal S_in (in place)
 * log_scale_out  device fp32 out [n_req][batch][heads] (diag: [..][dk]), or
 *                NULL (chain pair not wanted)
 * T_hat_out      device fp32 out [n_req][batch][heads][dk][dk]: dense only,
 *                given together with log_scale_out (PIC_ERR_NULL if only one
 *                of the two is given); NULL for scalar / diagonal forms.
 *                Neither output may overlap the pool.
 * -------------------------------------------------------------------- */
size_t pic_compose_workspace(int32_t n_req, int64_t chain_total);

int pic_validate_compose(int form, int batch, int heads, int dk, int dv, int64_t pool_size,
                         const float* pool_log_scale, const float* pool_T_hat,
                         const float* pool_S0, int32_t n_req, const int64_t* chain_offsets,
                         const int32_t* chain_idx, const float* S_in, const float* S_out,
                         const float* log_scale_out, const float* T_hat_out,
                         const void* workspace, size_t workspace_bytes);

int pic_compose(int form, int batch, int heads, int dk, int dv, int64_t pool_size,
                const float* pool_log_scale, const float* pool_T_hat, const float* pool_S0,
                int32_t n_req, const int64_t* chain_offsets, const int32_t* chain_idx,
                const float* S_in, float* S_out, float* log_scale_out, float* T_hat_out,
                void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * Compose that allocates nothing: for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results and errors as pic_compose, without the workspace.
 * The chain tables go into a static device array of
 * PIC_NOALLOC_SCRATCH_BYTES (1 MiB) that the library image holds on every
 * device it runs on until the process ends; a call whose tables need more
 * (pic_compose_workspace(n_req, chain_offsets[n_req]) bytes) returns
 * PIC_ERR_WORKSPACE before doing anything.  The call makes no hipMalloc,
 * hipFree or other allocation.  The tables are copied from the host arrays
 * and the call waits for its stream (or, with a staging pool reserved,
 * copies asynchronously through it).  Every call on one device shares that
 * device's array, which keeps the last call's tables: calls that overlap on
 * one device (other streams or threads) race and are not allowed.
 * -------------------------------------------------------------------- */
#define PIC_NOALLOC_SCRATCH_BYTES (1u << 20)

int pic_compose_noalloc(int form, int batch, int heads, int dk, int dv, int64_t pool_size,
                        const float* pool_log_scale, const float* pool_T_hat,
                        const float* pool_S0, int32_t n_req, const int64_t* chain_offsets,
                        const int32_t* chain_idx, const float* S_in, float* S_out,
                        float* log_scale_out, float* T_hat_out, void* stream);

/* ----------------------------------------------------------------------
 * Naive add (the ablation): S_out[r] = S_in[r] + sum over the chain of S0_p.
 *   [xix.ai HYPIC article, paragraph on linear layers: adding zero-start
 *    final states is exact only for plain linear attention; it leaves out
 *    the T(C2) factor.]
 * Arguments as for pic_compose (no operator needed).
 * -------------------------------------------------------------------- */
int pic_validate_naive_add(int batch, int heads, int dk, int dv, int64_t pool_size,
                           const float* pool_S0, int32_t n_req, const int64_t* chain_offsets,
                           const int32_t* chain_idx, const float* S_in, const float* S_out,
                           const void* workspace, size_t workspace_bytes);

int pic_naive_add(int batch, int heads, int dk, int dv, int64_t pool_size, const float* pool_S0,
                  int32_t n_req, const int64_t* chain_offsets, const int32_t* chain_idx,
                  const float* S_in, float* S_out, void* workspace, size_t workspace_bytes,
                  void* stream);

/* ----------------------------------------------------------------------
 * Compose with seam windows: reuse in which each cached segment's first
 * tokens are kept out of its pair and run again from the running state.
 *   [xix.ai HYPIC article, paragraph on full-attention layers: a window of w
 *    tokens (8 by default) at the start of every inner segment is left out of
 *    the cache and recomputed on reuse under the full prefix; the linear
 *    layers advance the running state through these tokens and pass each
 *    token's per-layer output up to the attention layer above.]
 *
 * For request r and each of its chain entries c (in order, as in
 * pic_compose): first the entry's seam tokens
 * t = seam_offsets[c] .. seam_offsets[c+1]-1, one at a time,
 *     S <- T_t S + beta_t k_t v_t^T       (the form's token transition)
 *     O[t] = S^T q_t                      (read after the token's update)
 * then the entry's pair, S <- e^{log_scale_p} That_p S + S0_p.  The pair of a
 * segment with a seam window is the pair of the tokens after the window.
 *
 * Arguments as for pic_compose, and:
 * qkv_dtype     storage type of q, k, v: PIC_DT_BF16 or PIC_DT_F32
 * seam_offsets  HOST int64[chain_total + 1], chain_total = chain_offsets[n_req]:
 *               seam_offsets[0] = 0, non-decreasing, last = n_seam; a window
 *               holds at most PIC_MAX_SEAM tokens (PIC_ERR_DIMS otherwise);
 *               an empty window is allowed
 * n_seam        number of seam tokens of the call (the token axis below)
 * q, k          device [batch][n_seam][heads][dk] (qkv_dtype)
 * v             device [batch][n_seam][heads][dv] (qkv_dtype)
 * alpha         device fp32 gates [batch][n_seam][heads] (diag, KDA: [..][dk])
 * beta          device fp32 [batch][n_seam][heads], dense and KDA, NULL = 1
 * O_out         device fp32 out [batch][n_seam][heads][dv]
 * form          any PIC_FORM_*; the KDA token transition is
 *               (I - beta k k^T) Diag(alpha), its pairs applied as dense ones
 * q, k, v, alpha and O_out may be NULL only when n_seam = 0.  The chain's own
 * pair is not produced.  The state and all updates are fp32 (seam tokens on
 * the vector units; the pairs as in pic_compose).
 * -------------------------------------------------------------------- */
#define PIC_MAX_SEAM 64

size_t pic_compose_seams_workspace(int32_t n_req, int64_t chain_total);

int pic_validate_compose_seams(int form, int qkv_dtype, int batch, int heads, int dk, int dv,
                               int64_t pool_size, const float* pool_log_scale,
                               const float* pool_T_hat, const float* pool_S0, int32_t n_req,
                               const int64_t* chain_offsets, const int32_t* chain_idx,
                               const int64_t* seam_offsets, int64_t n_seam, const void* q,
                               const void* k, const void* v, const float* alpha,
                               const float* beta, const float* S_in, const float* S_out,
                               const float* O_out, const void* workspace,
                               size_t workspace_bytes);

int pic_compose_seams(int form, int qkv_dtype, int batch, int heads, int dk, int dv,
                      int64_t pool_size, const float* pool_log_scale, const float* pool_T_hat,
                      const float* pool_S0, int32_t n_req, const int64_t* chain_offsets,
                      const int32_t* chain_idx, const int64_t* seam_offsets, int64_t n_seam,
                      const void* q, const void* k, const void* v, const float* alpha,
                      const float* beta, const float* S_in, float* S_out, float* O_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * Plain operator: T_out[u] = e^{log_scale[u]} * That[u] (dense), e^{lambda} I
 * (scalar) or Diag(e^{lambda}) (diag), in fp32 (entries underflow to 0 as fp32
 * must when lambda is very negative).  n_units pairs; layouts
 * log_scale [n_units] (diag [n_units][dk]), T_hat [n_units][dk][dk] (dense,
 * else NULL), T_out [n_units][dk][dk].
 * -------------------------------------------------------------------- */
int pic_materialize_T(int form, int64_t n_units, int dk, const float* log_scale,
                      const float* T_hat, float* T_out, void* stream);

/* ----------------------------------------------------------------------
 * Re-rotation: move cached pairs to another position under rotary position
 * embeddings (RoPE) on the keys.
 *   [xix.ai HYPIC article, paragraph on linear layers: variants with rotary
 *    embeddings need the cached state re-rotated.]
 *
 * A segment built with its keys rotated at positions t = 0, 1, ... and
 * placed `shift` positions later has every key rotated by R_shift on top, so
 *     S0' = R S0,   That' = R That R^T,   lambda' = lambda
 * where R turns channel pair i (i < rot_dim / 2) by the angle
 * shift * base^(-2i/rot_dim): (x_a, x_b) -> (cos x_a - sin x_b, sin x_a + cos x_b),
 * with the pair (2i, 2i+1) for PIC_ROPE_INTERLEAVED and (i, i + rot_dim/2) for
 * PIC_ROPE_HALF; channels from rot_dim on are unchanged.  Exact for the scalar,
 * dense and KDA forms' transitions when R commutes with the gates: always for
 * scalar and dense, and for the diagonal and KDA forms only when the two
 * channels of every rotated pair share their gate (not checked).  Angles are
 * formed in fp64, the rotation applied in fp32.
 *
 * Output entry j is pool entry idx[j] moved by shift[j] (negative shifts move
 * back; 0 copies).  Arguments:
 * pool_*          the pool as in pic_compose (pool_T_hat: dense and KDA only)
 * n               number of output entries (0: nothing to do)
 * idx, shift      HOST int32[n] pool indices in [0, pool_size), int64[n] shifts
 * rot_dim         rotated channels: a multiple of 8 in [8, dk] (PIC_ERR_DIMS)
 * rope_base       > 0 and finite (PIC_ERR_UNSUPPORTED otherwise), e.g. 10000
 * pairing         PIC_ROPE_INTERLEAVED or PIC_ROPE_HALF
 * log_scale_out, T_hat_out, S0_out   device fp32 outputs laid out as the pool
 *                 with n entries (T_hat_out: dense and KDA only, else NULL);
 *                 they must not overlap the pool (PIC_ERR_UNSUPPORTED)
 * -------------------------------------------------------------------- */
enum pic_rope_pairing { PIC_ROPE_INTERLEAVED = 0, PIC_ROPE_HALF = 1 };

size_t pic_rerotate_workspace(int32_t n);

int pic_validate_rerotate(int form, int batch, int heads, int dk, int dv, int64_t pool_size,
                          const float* pool_log_scale, const float* pool_T_hat,
                          const float* pool_S0, int32_t n, const int32_t* idx,
                          const int64_t* shift, int rot_dim, double rope_base, int pairing,
                          const float* log_scale_out, const float* T_hat_out,
                          const float* S0_out, const void* workspace, size_t workspace_bytes);

int pic_rerotate(int form, int batch, int heads, int dk, int dv, int64_t pool_size,
                 const float* pool_log_scale, const float* pool_T_hat, const float* pool_S0,
                 int32_t n, const int32_t* idx, const int64_t* shift, int rot_dim,
                 double rope_base, int pairing, float* log_scale_out, float* T_hat_out,
                 float* S0_out, void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * Convolution warm-up: for variants with a short causal depthwise
 * convolution of width W in front of the linear layer,
 *     y_t = sum_{j < W} weight[h][c][j] * x_(t-j)       (j = 0 the token itself)
 * a segment's first W-1 outputs read the previous segment's raw inputs, so
 * they are kept out of its cached pair and recomputed on reuse: this call
 * writes them in the seam layout, ready for pic_compose_seams (as its q, k or
 * v, one call per stream), with the pair covering the tokens after them.
 * Any per-token activation or normalisation the model applies after the
 * convolution is the caller's, between this call and the seam compose.
 *   [xix.ai HYPIC article, paragraph on linear layers: variants with a short
 *    convolution need the convolution state warmed up.]
 *
 * x_dtype      PIC_DT_BF16 or PIC_DT_F32: the type of x and y_out
 * dc           channels per head (dk for q / k, dv for v): as dk in the sizes rule
 * width        W in [1, PIC_MAX_CONV]
 * weight       device fp32 [heads][dc][width]
 * x            device [batch][n_tokens][heads][dc], raw inputs (the caller's
 *              store of the cached segments' inputs)
 * n, n_warm    entries and output tokens per entry (0 <= n_warm <= PIC_MAX_SEAM;
 *              usually W - 1)
 * head_start   HOST int64[n]: entry e's head tokens are x[:, head_start[e] + t],
 *              t < n_warm (head_start + n_warm <= n_tokens)
 * hist_end, hist_len  HOST int64[n], int32[n]: entry e's history is
 *              x[:, hist_end[e] - hist_len[e] .. hist_end[e] - 1], the raw
 *              inputs just before its segment (0 <= hist_len <= W - 1; 0 = no
 *              history, as in an independent prefill; absent taps read 0)
 * y_out        device [batch][n * n_warm][heads][dc] (x_dtype), entry e at rows
 *              e * n_warm ..; must not overlap x or weight
 * Accumulation in fp32; bf16 outputs are rounded to nearest even.
 * -------------------------------------------------------------------- */
#define PIC_MAX_CONV 16

size_t pic_conv_warmup_workspace(int32_t n);

int pic_validate_conv_warmup(int x_dtype, int batch, int heads, int dc, int width,
                             int64_t n_tokens, const float* weight, const void* x, int32_t n,
                             int32_t n_warm, const int64_t* head_start, const int64_t* hist_end,
                             const int32_t* hist_len, const void* y_out, const void* workspace,
                             size_t workspace_bytes);

int pic_conv_warmup(int x_dtype, int batch, int heads, int dc, int width, int64_t n_tokens,
                    const float* weight, const void* x, int32_t n, int32_t n_warm,
                    const int64_t* head_start, const int64_t* hist_end, const int32_t* hist_len,
                    void* y_out, void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * Plan dump: the host-side bookkeeping a build or compose call would use,
 * written to a host table so it can be checked exactly.  Pure host code: no
 * HIP call, no device pointer.
 *   [xix.ai HYPIC article, paragraph on linear layers: one cached pair per
 *    segment, found by segment boundaries; the serving layer recognises the
 *    boundaries and looks the pairs up.]
 *
 * kind = PIC_PLAN_BUILD: n = n_seg >= 1, offsets = seg_offsets (n+1 entries,
 *   checked as in pic_validate_build against limit = n_tokens), chain_idx
 *   must be NULL.  Writes n rows of PIC_PLAN_BUILD_COLS int64 each, in the
 *   order the segments are visited (longest first, ties by index):
 *     {segment, start, length, n_chunks, tail}
 *   with n_chunks = ceil(length / PIC_CHUNK) and tail = the number of tokens
 *   in the last chunk (0 for an empty segment).
 * kind = PIC_PLAN_COMPOSE: n = n_req >= 0, offsets = chain_offsets (n+1),
 *   chain_idx as in pic_compose, limit = pool_size.  Writes chain_total rows
 *   of PIC_PLAN_COMPOSE_COLS int64 each, in application order:
 *     {request, step within the chain, pool index}
 * table_rows is the capacity of `table` in rows (PIC_ERR_WORKSPACE if too
 * small).  Errors as for the matching validate call.
 * -------------------------------------------------------------------- */
enum pic_plan_kind { PIC_PLAN_BUILD = 0, PIC_PLAN_COMPOSE = 1 };
#define PIC_PLAN_BUILD_COLS 5
#define PIC_PLAN_COMPOSE_COLS 3
#define PIC_CHUNK 64

int pic_plan_dump(int kind, int32_t n, const int64_t* offsets, const int32_t* chain_idx,
                  int64_t limit, int64_t* table, int64_t table_rows);

#ifdef __cplusplus
}
#endif

#endif /* PIC_H_ */
