/*
 * fa.h -- C ABI of the MI355X (gfx950) fused causal attention library, libfa.so.
 *
 * The library computes scaled-dot-product attention with an online (streaming)
 * softmax over KV tiles, never forming the S x S score matrix:
 *
 *   forward   O = softmax(mask(scale * Q K^T)) V,  L[i] = logsumexp of row i
 *   backward  dQ, dK, dV of sum(dO * O), recomputing the scores from Q, K, V
 *             and L, with the row dot products D[i] = sum_d dO[i,d] * O[i,d].
 *
 * Definitions: "Phase T14: 融合 Flash-Attention Kernel — Design Document"
 * (section "什么是 flash-attention": the online-softmax recurrence, L = m + log l,
 * the flash backward formulas; decisions ② and ③: L is the only saved forward
 * state and D removes the softmax Jacobian) and "Phase 14: Flash Attention 2 for
 * SM120 — Design Document" (sections "FA2 算法", "GQA 支持", "Causal Mask").
 *
 * Layouts (all contiguous, head dimension fastest, element type = dtype):
 *   q, o, dO, dq      [B][Hq][S][D]
 *   k, v, dk, dv      [B][Hkv][S][D]
 *   lse               [B][Hq][S]        float32, natural log
 * Query head h reads KV head h / (Hq / Hkv): groups of consecutive query heads
 * share one KV head (GQA; Hq == Hkv is plain multi-head attention).
 *
 * causal = 1 masks key j for query i when j > i (the single sequence length
 * makes top-left and bottom-right alignment the same); causal = 0 masks nothing.
 *
 * Precision: fp32 inputs are computed in fp32 throughout.  bf16 / fp16 inputs
 * feed the matrix cores in their own type (P and dS are rounded to it, nearest
 * even); every accumulation, the softmax and L are fp32.  O, dq, dk, dv are
 * written in the input dtype.
 *
 * Ownership and threading: every pointer is a device pointer owned by the
 * caller; the library allocates nothing.  Its only state is the per-thread
 * instrumentation pointer set by fa_profile_events (off unless a caller sets
 * it; see there).
 * All work is enqueued on `stream` and the call returns without waiting.
 * Outputs are overwritten, never accumulated into.  Calls on different
 * streams with disjoint outputs may run concurrently.
 *
 * Errors: arguments are checked on the host before anything is enqueued; on
 * any error nothing is launched and no output is touched.  An unsupported
 * case is reported, never served by a slower substitute: the udemi.tech
 * "Flash Attention" page forces the flash backend so that an impossible call
 * raises instead of falling back, and "FlashAttention 与 SDPA Backend"
 * (section 失败场景与生产实现差距) warns that an API accepting an argument
 * does not mean every fast path supports it.
 *   FA_ERR_INVALID_ARG   null required pointer; B, Hq, Hkv, S or D < 0;
 *                        B, Hq or Hkv == 0 while there are query or key
 *                        rows; Hq % Hkv != 0; scale not finite; a pointer
 *                        not 16-byte aligned; dtype not one of fa_dtype_t.
 *   FA_ERR_UNSUPPORTED   D not 64 or 128; scale <= 0; a sequence length
 *                        above 2^29 (or a grid beyond INT_MAX workgroups).
 *   FA_ERR_WORKSPACE     workspace smaller than fa_bwd_workspace_bytes().
 *   FA_ERR_HIP           a HIP launch reported an error (hipGetLastError).
 * A problem with B * Hq * S == 0 is a no-op that returns FA_OK once the
 * scalar checks above pass (pointers are not inspected then).
 * NaN or Inf in the inputs is not checked and propagates to the outputs.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_WORKSPACE = 3,
  FA_ERR_HIP = 4
} fa_status_t;

/*
 * Forward pass.  Writes o and (when lse is not NULL) the per-row natural-log
 * logsumexp of the scaled, masked scores, L[i] = m_i + log(l_i)
 * ("Phase T14", decision ②: the only forward state the backward needs).
 *   q, k, v : inputs, layouts above, element type dtype
 *   o       : output [B][Hq][S][D], dtype
 *   lse     : output [B][Hq][S] float32, or NULL to skip it
 *   scale   : multiplies Q K^T before the softmax (1/sqrt(D) for standard
 *             attention); must be finite and > 0
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int S, int D, float scale, int causal,
                   fa_dtype_t dtype, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for this problem (a multiple of 256;
 * 0 for an empty problem).  It holds the fp32 row dot products
 * D[i] = sum_d dO[i,d] * O[i,d], one per query row: the O(N) precompute of
 * "Phase T14", decision ③, which the backward reads in place of the softmax
 * Jacobian.  The library never allocates, so the caller provides it.
 * Returns 0 for arguments fa_bwd would reject.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D);

/*
 * Backward pass ("Phase T14", section "什么是 flash-attention" and decision ③).
 *   q, k, v, o, lse : the forward's inputs and its unchanged outputs o and lse
 *                     (lse must not be NULL here)
 *   dO              : gradient of the loss with respect to o, [B][Hq][S][D]
 *   dq, dk, dv      : outputs, same layouts and dtype as q, k, v; dk and dv of a
 *                     KV head are summed over the query heads that read it
 *   workspace       : device scratch of at least fa_bwd_workspace_bytes(...)
 *                     bytes, 16-byte aligned; may be NULL when that size is 0.
 *                     Its contents on entry are ignored and on return undefined;
 *                     two calls in flight at once need two workspaces.
 * The scores are recomputed as P = exp(scale * Q K^T - L); the caller must pass
 * the same scale and causal flag as to the forward.
 */
fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int S, int D, float scale, int causal,
                   fa_dtype_t dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_bwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments (without the workspace), results and errors as fa_bwd.  The row
 * dot products live instead in a static device array of the library,
 * FA_BWD_NOALLOC_MAX_ROWS fp32 values (16 MiB), one per GPU, held until the
 * process ends; the call allocates and frees nothing.
 *   FA_ERR_WORKSPACE    B * Hq * S > FA_BWD_NOALLOC_MAX_ROWS (the static array
 *                       is too small for the problem; use fa_bwd)
 *   FA_ERR_INVALID_ARG  also when `stream` belongs to a device other than the
 *                       calling thread's current device
 *   FA_ERR_HIP          also when the array's device address cannot be looked
 *                       up (done once per device, on the first call there)
 * Every call on one GPU uses that GPU's one array, which keeps the last call's
 * contents (each call writes every entry it reads).  Calls that overlap on one
 * GPU (on different streams, or from different host threads without ordering)
 * race on the array and may return wrong gradients: serialise them.
 */
#define FA_BWD_NOALLOC_MAX_ROWS (1 << 22)
fa_status_t fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dO, void* dq, void* dk, void* dv,
                           int B, int Hq, int Hkv, int S, int D, float scale, int causal,
                           fa_dtype_t dtype, hipStream_t stream);

/* Static, human-readable name of a status code ("FA_OK", ...); never NULL.
 * The codes follow the error convention above (an impossible request is an
 * error, not a fallback: udemi.tech "Flash Attention", forcing the flash
 * backend; "FlashAttention 与 SDPA Backend", section 失败场景与生产实现差距). */
const char* fa_status_string(fa_status_t s);

/*
 * Extended problems: queries and keys of different lengths, a sliding window,
 * and packed variable-length batches.
 *
 *   Visibility of key j to query i of one sequence, offset = Skv_b - Sq_b:
 *     causal        j <= i + offset          (bottom-right alignment: "Phase 14",
 *                                             section Causal Mask, kv_offset)
 *     window >= 0   j >= i + offset - window (a left window of window + 1 keys
 *                                             when causal; window >= Skv hides
 *                                             nothing and runs as no window)
 *   A query that sees no key has an empty softmax: its O row is 0, its L is
 *   -inf, and it contributes no gradient.
 *
 *   Dense batches (cu_seqlens_q == cu_seqlens_k == NULL):
 *     q, o, dO, dq [B][Hq][Sq][D]; k, v, dk, dv [B][Hkv][Skv][D]; lse [B][Hq][Sq]
 *   Packed variable-length batches (both non-NULL, device int32 arrays of B + 1
 *   non-decreasing offsets starting at 0): sequence b owns query rows
 *   cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
 *   cu_seqlens_k[b+1]-1, and
 *     q, o, dO, dq [Hq][total_q][D]; k, v, dk, dv [Hkv][total_k][D];
 *     lse [Hq][total_q]
 *   where total_q = cu_seqlens_q[B] and total_k = cu_seqlens_k[B] are also
 *   passed by value, and Sq / Skv are upper bounds of the per-sequence lengths
 *   (they size the launch).  The kernels clamp offsets into [0, total] and
 *   lengths to the bounds, so malformed offsets give wrong results, never
 *   accesses outside the described buffers.
 *
 *   Linear position bias (ALiBi; "FlashAttention 与 SDPA Backend", section
 *   失败场景与生产实现差距, lists it in the support matrix of a real kernel):
 *   with alibi_slopes non-NULL (a device array of Hq fp32 values, 4-byte
 *   aligned), query i and key j of query head h get -alibi_slopes[h] *
 *   |i + offset - j| added to their scaled score before the softmax (0 on the
 *   bottom-right diagonal; the form is this library's reading, the page does
 *   not define it).  The slopes are read on the device and not checked.  The
 *   split-KV forward returns FA_ERR_UNSUPPORTED for it.
 */
typedef struct {
  int B, Hq, Hkv;
  int Sq, Skv;                 /* lengths (dense) or length bounds (packed) */
  int D;                       /* 64 or 128 */
  float scale;                 /* finite, > 0 */
  int causal;                  /* 0 or 1 */
  int window;                  /* < 0: no window */
  const int* cu_seqlens_q;     /* device, B + 1 entries, or NULL */
  const int* cu_seqlens_k;     /* device, B + 1 entries, or NULL */
  int total_q, total_k;        /* packed only: cu_seqlens_q[B], cu_seqlens_k[B] */
  fa_dtype_t dtype;
  const float* alibi_slopes;   /* device, Hq fp32 slopes, or NULL (no bias); see above */
} fa_params_t;

/* Forward of an extended problem.  Same outputs and errors as fa_fwd; also
 * FA_ERR_INVALID_ARG for a NULL params, only one of the cu_seqlens pointers
 * given, a cu_seqlens pointer not 4-byte aligned, or negative totals.
 * A problem with no query row is a no-op; with no key row, k and v may be
 * NULL and every O row is 0, every L -inf. */
fa_status_t fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                      const fa_params_t* params, hipStream_t stream);

/* Workspace of fa_bwd_ex (fp32 row dot products, one per query row; a multiple of
 * 256 bytes), or 0 when none is needed or the params are rejected. */
size_t fa_bwd_ex_workspace_bytes(const fa_params_t* params);

/* Backward of an extended problem (as fa_bwd).  dk and dv of keys no query can
 * see are written as 0; the call is a no-op only when there are neither query
 * nor key rows.  Buffers of an empty side (q, o, lse, dO, dq without query
 * rows; k, v, dk, dv without key rows) may be NULL. */
fa_status_t fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dO, void* dq, void* dk, void* dv, const fa_params_t* params,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Split-KV forward for decode-shaped problems: few query rows per KV head and
 * many keys, as when decoding against a KV cache.  "Phase 14", section
 * 已知局限与后续优化方向, asks for a dedicated decode kernel that reduces in
 * parallel along the keys; "FlashAttention 与 SDPA Backend" names the split-KV
 * merge as one of a real kernel's choices.  Each sequence's keys are cut into
 * ranges processed in parallel, each range leaves a normalised partial output
 * O_s and logsumexp L_s, and a second kernel merges them:
 * L = log sum_s exp(L_s), O = sum_s exp(L_s - L) O_s.
 * Same problem, layouts, outputs and errors as fa_fwd_ex, plus:
 *   num_splits : > 0 chooses the number of key ranges (capped at one per
 *                key tile of 128 keys, 64 for fp32); <= 0 lets the library
 *                choose enough ranges to fill the GPU
 *   workspace  : device scratch of at least
 *                fa_fwd_splitkv_workspace_bytes(params, num_splits) bytes,
 *                16-byte aligned, holding the partial results; contents on
 *                entry are ignored; two calls in flight need two workspaces
 * FA_ERR_UNSUPPORTED when (Hq / Hkv) * Sq > 32: the query rows of one KV group
 * share one 32-column matrix block, which is what lets the G heads of a group
 * read K and V once; also when params->alibi_slopes is not NULL.
 * FA_ERR_WORKSPACE when the workspace is too small, and
 * FA_ERR_INVALID_ARG when it is NULL or misaligned.  Results match fa_fwd_ex's
 * up to fp32 rounding order and are deterministic for a given split count.
 */
size_t fa_fwd_splitkv_workspace_bytes(const fa_params_t* params, int num_splits);
fa_status_t fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                           const fa_params_t* params, int num_splits, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Instrumentation for benchmarks (not part of the computation).  After
 * fa_profile_events(ev, n) with ev != NULL, each later compute call made from
 * the same host thread records ev[0..] on its stream around every kernel it
 * launches: fa_fwd records ev[0] before and ev[1] after its one kernel;
 * fa_bwd records ev[0] before the row-dot kernel, ev[1] before the dK/dV
 * kernel, ev[2] before the dQ kernel and ev[3] after it; fa_fwd_splitkv
 * records ev[0] before its split kernel, ev[1] before its merge kernel and
 * ev[2] after it (fa_fwd_ex / fa_bwd_ex as fa_fwd / fa_bwd).  Indices >= n are not
 * recorded.  The caller owns the events (created with hipEventCreate).  The
 * setting is state of the calling thread that lasts until changed: every later
 * compute call on that thread records into the same events.  A caller must
 * therefore call fa_profile_events(NULL, 0), which turns recording off, before
 * it destroys the events; otherwise later calls record freed events.
 */
void fa_profile_events(hipEvent_t* events, int n);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
