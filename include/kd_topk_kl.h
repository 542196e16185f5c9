/*
 * kd_topk_kl.h -- C ABI of the fused, chunked top-K KL distillation loss
 * (forward + backward) for AMD Instinct MI355X (gfx950).
 *
 * What is computed
 * ----------------
 * The method is the one described in "Efficient Knowledge Distillation for
 * LLMs: Offline Top-K Logits and a Fused Chunked KL Loss" as reported by
 * "Making Knowledge Distillation Cheap Enough to Run at Scale" (aipuls.nl,
 * section "Summary") and "Hugging Face and Multiverse Computing cut KD
 * memory costs" (agent-gateway.com): the teacher's top-K logits per token
 * are cached offline, and the KL loss between the teacher's distribution and
 * the student's LM-head output is evaluated over successive token slices,
 * so that the sequence-by-vocabulary logit matrix never exists in memory.
 *
 * For token t (0 <= t < T), with z[t,v] = sum_j H[t,j] W[v,j] (no bias):
 *   p[t,:]  = softmax over all V of z[t,:]/tau          (student)
 *   q[t,k]  = softmax over the K slots of topk_logit[t,:]/tau  (teacher)
 *   KL_t    = sum_k q[t,k] (log q[t,k] - log p[t, topk_idx[t,k]])
 *   N       = sum_t mask[t]   (mask NULL: N = T)
 *   loss    = tau^2 / N * sum_t mask[t] KL_t            (0 when N = 0)
 *   G[t,v]  = tau / N * mask[t] * (p[t,v] - sum_k q[t,k] [topk_idx[t,k]==v])
 *   dH      = G W        dW = G^T H      (dW optionally accumulated)
 * The direction (teacher as target, student log-softmax over the whole
 * vocabulary, mean over selected tokens) follows the asibiont.com article,
 * section "A Concrete Implementation Sketch"; temperature scaling by tau and
 * tau^2 is this library's reading where the pages are silent.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All tensors are dense, row-major, contiguous, in device memory of the
 *   current HIP device; the caller allocates and owns every buffer.  The
 *   library allocates nothing and keeps no state between calls, apart from
 *   the optional, per-thread measurement hook kd_set_launch_log and the
 *   fixed per-GPU scratch of kd_topk_kl_fwd_noalloc.
 * - H and W, and the dH and dW outputs, start on a 16-byte boundary (the
 *   kernels move their rows 16 bytes at a time; any HIP or torch
 *   allocation qualifies, and since d % 8 == 0 so does every row of one);
 *   other pointers need only their element's alignment.  A misaligned H,
 *   W, dH or dW is KD_ERR_INVALID_ARG.
 * - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *   the default stream).  Outputs are valid once that stream has
 *   synchronised.  No call synchronises the host.
 * - Return value: KD_OK or one KD_ERR_* code.  Every argument check runs on
 *   the host before any HIP call, so a rejected call enqueues nothing.
 *   KD_ERR_HIP reports a failed launch; kd_status_string() then includes
 *   the HIP error text of the last failure on the calling thread.
 * - Calls on different streams may run concurrently when each has its own
 *   workspace and outputs.
 */
#ifndef KD_TOPK_KL_H
#define KD_TOPK_KL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of H and W. */
typedef enum { KD_F32 = 0, KD_BF16 = 1 } kd_dtype;

enum {
  KD_OK = 0,
  KD_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, K > V, bad tau */
  KD_ERR_WORKSPACE = 2,   /* workspace missing or smaller than required    */
  KD_ERR_UNSUPPORTED = 3, /* valid but unsupported: d % 8 != 0, K > KD_MAX_K,
                             sizes beyond 32-bit index range, unknown dtype */
  KD_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed     */
  KD_ERR_SCRATCH = 5      /* kd_topk_kl_fwd_noalloc: the sizes need more than
                             KD_NOALLOC_SCRATCH_BYTES of scratch            */
};

/* Flags for kd_topk_kl_fwd_bwd. */
enum {
  KD_FLAG_ACCUMULATE_DW = 1u /* dW += G^T H instead of dW = G^T H          */
};

/* Largest supported K (teacher cache width). */
#define KD_MAX_K 1024

/*
 * kd_topk_kl_workspace_size -- bytes of scratch device memory needed by
 * kd_topk_kl_fwd_bwd and kd_topk_kl_bwd (and, larger than it needs,
 * kd_topk_kl_fwd) for these sizes.
 *
 * The workspace holds the per-slice intermediates of the chunked loss
 * ("Making Knowledge Distillation Cheap Enough to Run at Scale", aipuls.nl,
 * section "Summary": memory bounded by one slice): the slice's shifted
 * student probabilities, then its logit gradient (chunk x V, in the input
 * element type), per-row and per-vocabulary-segment softmax statistics,
 * the teacher distribution of the slice, split-K partial sums of dH for the
 * slice and O(T) per-row scalars; on the tuned bf16 path also the
 * transposed, gradient-scaled hidden states of the slice (d x chunk).  It
 * grows with chunk*V and chunk*d, never with T*V.
 *
 * Arguments: sizes as for kd_topk_kl_fwd_bwd; `chunk` is clamped to [1, T].
 * `bytes_out` (host pointer) receives the size.  Returns KD_OK,
 * KD_ERR_INVALID_ARG (bad sizes or NULL bytes_out) or KD_ERR_UNSUPPORTED.
 */
int kd_topk_kl_workspace_size(int64_t T, int64_t d, int64_t V, int32_t K,
                              int32_t chunk, kd_dtype dtype,
                              size_t *bytes_out);

/*
 * kd_topk_kl_fwd_bwd -- loss, dH and dW of the top-K KL distillation loss,
 * processed in token slices of `chunk` rows (the fused, chunked loss of
 * "Hugging Face and Multiverse Computing cut KD memory costs",
 * agent-gateway.com; the offline top-K cache of "Making Knowledge
 * Distillation Cheap Enough to Run at Scale", aipuls.nl, section "Summary").
 *
 *   H          [T, d]  student final hidden states, dtype (bf16 or fp32)
 *   W          [V, d]  student LM-head weight, dtype
 *   dtype      element type of H and W
 *   topk_idx   [T, K]  int32 teacher top-K vocabulary ids.  Contract: each
 *                      row holds K distinct ids in [0, V).  Ids outside
 *                      [0, V) are never dereferenced (memory-safe) but the
 *                      results for their rows are unspecified.
 *   topk_logit [T, K]  fp32 teacher logits of those ids (any order)
 *   mask       [T]     uint8, 1 = valid token, 0 = padding; NULL = all valid
 *   T, d, V, K         sizes; T, d, V, K >= 1, K <= V, K <= KD_MAX_K,
 *                      d % 8 == 0, T*d, V*d, T*K < 2^31
 *   tau        temperature, finite and > 0
 *   chunk      token rows per slice (>= 1; clamped to T)
 *   flags      0 or KD_FLAG_ACCUMULATE_DW
 *   loss       [1]     fp32 output (device)
 *   row_loss   [T]     fp32 output mask[t]*KL_t (unscaled), or NULL
 *   dH         [T, d]  fp32 output (overwritten)
 *   dW         [V, d]  fp32 output (overwritten, or accumulated into)
 *   workspace  device scratch of at least kd_topk_kl_workspace_size()
 *              bytes, 256-byte aligned; its contents on entry are ignored
 *   stream     hipStream_t (as void*) on which all work is enqueued
 *
 * Defined edge results: N = 0 gives loss = 0, dH = 0 and a zero dW
 * contribution; a padding row t gives dH[t,:] = 0 and row_loss[t] = 0.
 * Reductions are ordered, so repeated calls give bitwise-identical results.
 */
int kd_topk_kl_fwd_bwd(const void *H, const void *W, kd_dtype dtype,
                       const int32_t *topk_idx, const float *topk_logit,
                       const uint8_t *mask, int64_t T, int64_t d, int64_t V,
                       int32_t K, float tau, int32_t chunk, uint32_t flags,
                       float *loss, float *row_loss, float *dH, float *dW,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * kd_topk_kl_fwd_workspace_size -- bytes of scratch device memory needed by
 * kd_topk_kl_fwd for these sizes: the per-slice row statistics, teacher
 * softmax, gathered logits and sorted ids, and the row losses (no
 * probabilities or gradient buffers; 81 MB at T = 32768, V = 201088,
 * K = 100, chunk 8192, against 4.2 GB for the fused call).  At most
 * kd_topk_kl_workspace_size for the same sizes.  Arguments, return codes
 * and checks as for kd_topk_kl_workspace_size.
 */
int kd_topk_kl_fwd_workspace_size(int64_t T, int64_t d, int64_t V, int32_t K,
                                  int32_t chunk, kd_dtype dtype, size_t *bytes_out);

/*
 * kd_topk_kl_fwd -- the loss alone (no gradients): the forward half of the
 * loss for evaluation, or for training with kd_topk_kl_bwd when the
 * backward runs later (the student training step of "Making Knowledge
 * Distillation Cheap Enough to Run at Scale", aipuls.nl, section
 * "Summary").  Arguments as for kd_topk_kl_fwd_bwd; in addition
 *   lse   [T] fp32 output logsumexp_v z[t,v]/tau of every row (padding rows
 *         too), or NULL.
 * loss and row_loss are bitwise those of kd_topk_kl_fwd_bwd.  It runs the
 * logits GEMM and the row reductions only: about a third of the work.  The
 * workspace needs at least kd_topk_kl_fwd_workspace_size bytes (a workspace
 * sized by kd_topk_kl_workspace_size is larger and also does).
 */
int kd_topk_kl_fwd(const void *H, const void *W, kd_dtype dtype,
                   const int32_t *topk_idx, const float *topk_logit,
                   const uint8_t *mask, int64_t T, int64_t d, int64_t V,
                   int32_t K, float tau, int32_t chunk, float *loss,
                   float *row_loss, float *lse, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Bytes of device scratch kd_topk_kl_fwd_noalloc holds per GPU. */
#define KD_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * kd_topk_kl_fwd_noalloc -- kd_topk_kl_fwd for callers that cannot allocate
 * device memory at call time (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): it takes no workspace and calls
 * no allocating routine.  Its scratch is a fixed device array of
 * KD_NOALLOC_SCRATCH_BYTES per GPU, set up by the runtime when the library
 * is loaded and held until the process ends; its address on a device is
 * looked up once, on the first call made with that device current.
 *
 * Arguments, outputs and results as for kd_topk_kl_fwd (the same kernels:
 * loss, row_loss and lse are bitwise those of kd_topk_kl_fwd for the same
 * chunk).  The scratch needs, with C = min(chunk, T) and nseg = ceil(V/256),
 *     at most 4 T + C (20 K + 10 nseg + 4) + 3072 bytes
 * (about 10 MB for T = 32768, V = 201088, K = 100, chunk = 1024); larger
 * problems are rejected with KD_ERR_SCRATCH before any HIP call.  Nothing in
 * the scratch needs to be zero on entry (every call writes what it reads).
 * All calls on one GPU share its scratch: calls that overlap in time on one
 * GPU (two streams, two threads) race and give undefined results; calls on
 * different GPUs do not interact.  Returns KD_OK, KD_ERR_INVALID_ARG,
 * KD_ERR_UNSUPPORTED, KD_ERR_SCRATCH or KD_ERR_HIP.
 */
int kd_topk_kl_fwd_noalloc(const void *H, const void *W, kd_dtype dtype,
                           const int32_t *topk_idx, const float *topk_logit,
                           const uint8_t *mask, int64_t T, int64_t d, int64_t V,
                           int32_t K, float tau, int32_t chunk, float *loss,
                           float *row_loss, float *lse, void *stream);

/*
 * kd_topk_kl_bwd -- dH and dW of grad_loss * loss, recomputing the logits
 * slice by slice (nothing is kept from kd_topk_kl_fwd).  Arguments as for
 * kd_topk_kl_fwd_bwd; in addition
 *   grad_loss  device pointer to one fp32: the upstream gradient of the
 *              loss (NULL: 1).  It scales the logit gradient G before both
 *              GEMMs, so dH and dW equal grad_loss times kd_topk_kl_fwd_bwd's
 *              up to fp32 rounding.
 * loss and row_loss are not produced.
 */
int kd_topk_kl_bwd(const void *H, const void *W, kd_dtype dtype,
                   const int32_t *topk_idx, const float *topk_logit,
                   const uint8_t *mask, int64_t T, int64_t d, int64_t V,
                   int32_t K, float tau, int32_t chunk, uint32_t flags,
                   const float *grad_loss, float *dH, float *dW,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * kd_grad_cast -- dst[i] = src[i] * (*scale) for i < n, in dst_dtype (bf16
 * rounded to nearest even): hands a gradient computed in fp32 back to a
 * bf16 or fp32 parameter, scaled by a device-resident upstream gradient
 * (scale NULL: 1).  src [n] fp32 and dst [n] are device memory and may be
 * the same buffer when dst_dtype is KD_F32.  Returns KD_OK,
 * KD_ERR_INVALID_ARG (NULL pointer, n < 0), KD_ERR_UNSUPPORTED or KD_ERR_HIP.
 */
int kd_grad_cast(const float *src, void *dst, kd_dtype dst_dtype, int64_t n,
                 const float *scale, void *stream);

/* Modes of kd_entropy_filter. */
enum {
  KD_FILTER_ENTROPY_ABOVE = 0,       /* keep tokens with entropy > param   */
  KD_FILTER_TOP_ENTROPY_FRACTION = 1 /* keep the fraction param of valid
                                        tokens with the highest entropy    */
};

/* Bytes of device scratch kd_entropy_filter needs for T tokens (host
 * pointer bytes_out).  Returns KD_OK, KD_ERR_INVALID_ARG or
 * KD_ERR_UNSUPPORTED (T >= 2^31). */
int kd_entropy_filter_workspace_size(int64_t T, size_t *bytes_out);

/*
 * kd_entropy_filter -- distillation token filtering by teacher entropy
 * (asibiont.com article, sections "Distillation Token Filtering" and "A
 * Concrete Implementation Sketch": tokens whose teacher distribution is
 * nearly one-hot are skipped, by an entropy threshold or by keeping a fixed
 * fraction of the batch's tokens with the highest entropy).  The teacher
 * distribution is the loss's: q[t,:] = softmax(topk_logit[t,:] / tau) over
 * the K cached logits, and entropy[t] = -sum_k q[t,k] log q[t,k] (no
 * epsilon inside the log; q > 0).  Writes a token mask for the loss entry
 * points:
 *   KD_FILTER_ENTROPY_ABOVE         mask_out[t] = mask[t] && entropy[t] > param
 *   KD_FILTER_TOP_ENTROPY_FRACTION  with N = sum mask, the n = floor(param*N
 *        + 1/2) valid tokens of highest entropy (equal entropies: lower t
 *        first) get 1, all others 0; param in [0, 1]
 *
 *   topk_logit  [T, K] fp32 teacher logits (device)
 *   mask        [T] uint8 (1 = valid) or NULL (all valid); may alias mask_out
 *   tau         temperature, finite and > 0
 *   mask_out    [T] uint8 output (device)
 *   entropy_out [T] fp32 output, or NULL
 *   workspace   at least kd_entropy_filter_workspace_size(T) bytes,
 *               256-byte aligned
 * Entropies are computed in fp32, so a token whose entropy lies within
 * fp32 rounding of the threshold (or of the kept set's boundary) may fall
 * either way.  Returns KD_OK, KD_ERR_INVALID_ARG, KD_ERR_UNSUPPORTED
 * (K > KD_MAX_K, T*K >= 2^31), KD_ERR_WORKSPACE or KD_ERR_HIP.
 */
int kd_entropy_filter(const float *topk_logit, const uint8_t *mask, int64_t T,
                      int32_t K, float tau, int32_t mode, float param,
                      uint8_t *mask_out, float *entropy_out, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Kernel ids for kd_set_launch_log (bit i of the mask selects id i). */
enum {
  KD_KERNEL_VALID_COUNT = 0, /* N = sum(mask), gradient and loss scales     */
  KD_KERNEL_PREP_ROWS = 1,   /* teacher softmax over K, id sort, segments    */
  KD_KERNEL_GEMM_LOGITS = 2, /* z = H_c W^T + per-segment softmax + gather   */
  KD_KERNEL_LSE_FIX = 3,     /* row logsumexp, KL_t, teacher correction      */
  KD_KERNEL_GEMM_DH = 4,     /* split-K partials of dH = G W                 */
  KD_KERNEL_REDUCE_DH = 5,   /* ordered sum of the dH partials               */
  KD_KERNEL_GEMM_DW = 6,     /* dW (+)= G^T H_c                              */
  KD_KERNEL_FINAL_LOSS = 7,  /* loss = tau^2/N sum_t row_loss                */
  KD_KERNEL_TRANSPOSE_H = 8, /* H_c^T staging for the dW GEMM (bf16 path)    */
  KD_KERNEL_FLAGGED_ROWS = 9, /* bf16 path: rows whose a-priori shift was too
                                low, recomputed with the row maximum         */
  /* id 10 is not used */
  /* kd_teacher_topk */
  KD_KERNEL_TK_SAMPLE = 11,  /* logits of the sampled vocabulary segments    */
  KD_KERNEL_TK_THETA = 12,   /* per-row threshold from the sampled logits    */
  KD_KERNEL_TK_FILTER = 13,  /* logits of the other segments + candidates    */
  KD_KERNEL_TK_SELECT = 14,  /* exact top-K of each row's candidates         */
  KD_KERNEL_TK_STREAM = 15,  /* row-streaming top-K (generic path, overflow) */
  KD_KERNEL_GRAD_CAST = 16,  /* kd_grad_cast                                 */
  KD_KERNEL_ENTROPY_FILTER = 17, /* kd_entropy_filter (all of its kernels)   */
  KD_KERNEL_DIVERGENCE = 18  /* kd_topk_div_fwd_bwd (all kernels but the
                                final loss sum)                             */
};

/* Divergences of kd_topk_div_fwd_bwd. */
enum {
  KD_DIV_REVERSE_KL = 1, /* KL(p^ || q)                                       */
  KD_DIV_JSD = 2         /* (KL(q || m) + KL(p^ || m)) / 2, m = (p^ + q) / 2  */
};

/*
 * kd_topk_div_workspace_size -- bytes of device scratch kd_topk_div_fwd_bwd
 * needs: the logit gradient at the ids and the sorted (id, pair) lists,
 * O(T K + V) words, plus partial dW rows for ids with more than 1024 pairs
 * (at most 2 ceil(T K / 1024) rows of d floats).  `bytes_out` is a host
 * pointer.  Returns KD_OK, KD_ERR_INVALID_ARG or KD_ERR_UNSUPPORTED.
 */
int kd_topk_div_workspace_size(int64_t T, int64_t d, int64_t V, int32_t K,
                               size_t *bytes_out);

/*
 * kd_topk_div_fwd_bwd -- loss, dH and dW of a divergence between teacher
 * and student over the teacher's cached top-K support: the loss variants
 * that the open question of "Hugging Face and Multiverse Computing cut KD
 * memory costs" (agent-gateway.com, closing paragraph: how much signal the
 * top-K cache keeps) calls for, next to the forward KL of kd_topk_kl_fwd_bwd
 * (the asibiont.com article, section "A Concrete Implementation Sketch",
 * distils with a divergence between the softened distributions).
 *
 * Both distributions live on row t's K cached ids: the teacher
 * q = softmax(topk_logit[t,:] / tau) and the student restricted to the ids
 * and renormalised, p^ = softmax(z[t, topk_idx[t,:]] / tau), z = H W^T:
 *   kind KD_DIV_REVERSE_KL  D_t = sum_k p^_k (log p^_k - log q_k)
 *   kind KD_DIV_JSD         D_t = 1/2 sum_k q_k log(q_k / m_k)
 *                                 + 1/2 sum_k p^_k log(p^_k / m_k)
 *   loss = tau^2 / N * sum_t mask[t] D_t    (0 when N = 0)
 * The logit gradient is non-zero at the K ids only, so dH and dW come from
 * gathers of K rows of W and H per token: no [T, V] or chunk x V buffer and
 * no dense GEMM (O(T K d) work).
 *
 * Arguments as for kd_topk_kl_fwd_bwd (no chunk: nothing of size V is
 * formed per token).  dH [T, d] is overwritten; dW [V, d] is overwritten,
 * or accumulated into with KD_FLAG_ACCUMULATE_DW (rows of ids no token
 * references get 0, or keep their value).  Ids outside [0, V) are never
 * dereferenced.  Sums are ordered (the (id, token) pairs are sorted with a
 * stable radix sort), so repeated calls give bitwise-identical results.
 * Returns KD_OK, KD_ERR_INVALID_ARG (unknown kind, NULL pointer, bad sizes
 * or tau), KD_ERR_UNSUPPORTED, KD_ERR_WORKSPACE or KD_ERR_HIP.
 */
int kd_topk_div_fwd_bwd(int32_t kind, const void *H, const void *W,
                        kd_dtype dtype, const int32_t *topk_idx,
                        const float *topk_logit, const uint8_t *mask,
                        int64_t T, int64_t d, int64_t V, int32_t K, float tau,
                        uint32_t flags, float *loss, float *row_loss,
                        float *dH, float *dW, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Largest supported K and hidden size of kd_teacher_topk. */
#define KD_TOPK_MAX_K 256
#define KD_TOPK_MAX_D 16384

/*
 * kd_teacher_topk_workspace_size -- bytes of scratch device memory needed by
 * kd_teacher_topk for these sizes (per slice of `chunk` rows: the logits of
 * ns sampled vocabulary segments of 256 ids, ns = 32, or more when K *
 * ceil(V / 256) > 131072, up to 128; 8192 candidate slots of 8 bytes and
 * four words per row; bf16 with d % 64 == 0 only, otherwise 256 bytes).  It
 * grows with chunk, never with T*V.  Arguments and return values as for
 * kd_teacher_topk; `bytes_out` is a host pointer.
 */
int kd_teacher_topk_workspace_size(int64_t T, int64_t d, int64_t V, int32_t K,
                                   int32_t chunk, kd_dtype dtype,
                                   size_t *bytes_out);

/*
 * kd_teacher_topk -- the offline teacher cache of the method: for every
 * token row t, the K largest teacher logits z[t,v] = sum_j H[t,j] W[v,j]
 * and their ids ("Making Knowledge Distillation Cheap Enough to Run at
 * Scale", aipuls.nl, section "Summary": the teacher runs once and its
 * top-100 logits per position are cached), computed slice by slice without
 * the token-by-vocabulary logit matrix.
 *
 *   H           [T, d]  teacher final hidden states, dtype (bf16 or fp32)
 *   W           [V, d]  teacher LM-head weight, dtype
 *   T, d, V, K          sizes; T, d, V, K >= 1, K <= V, K <= KD_TOPK_MAX_K,
 *                       d % 8 == 0, d <= KD_TOPK_MAX_D, T*d, V*d, T*K < 2^31
 *   chunk       token rows per slice (>= 1; clamped to T)
 *   topk_idx    [T, K]  int32 output: ids, by logit descending; equal
 *                       logits are ordered by id ascending (-0 equals +0)
 *   topk_logit  [T, K]  fp32 output: z at those ids (no temperature)
 *   workspace   device scratch of at least kd_teacher_topk_workspace_size()
 *               bytes, 256-byte aligned; contents on entry are ignored
 *   stream      hipStream_t (as void*) on which all work is enqueued
 *
 * z is accumulated in fp32 from the inputs (bf16 products are exact).  With
 * bf16 inputs and d % 64 == 0 it comes from the matrix-core GEMM; other
 * inputs, and rows whose candidate count exceeds the 8192 slots (logits
 * with strong structure against the sampled segments), are evaluated by a
 * row-streaming kernel whose fp32 sums may differ from the GEMM's in the
 * last bits.  Inputs must be finite (NaN logits have no defined rank).
 * Returns KD_OK, KD_ERR_INVALID_ARG (NULL pointer, bad size, K > V),
 * KD_ERR_UNSUPPORTED, KD_ERR_WORKSPACE or KD_ERR_HIP; checks run on the
 * host before any HIP call.  Results are deterministic.
 */
int kd_teacher_topk(const void *H, const void *W, kd_dtype dtype, int64_t T,
                    int64_t d, int64_t V, int32_t K, int32_t chunk,
                    int32_t *topk_idx, float *topk_logit, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * kd_set_launch_log -- measurement hook for profilers and benchmarks; it is
 * not needed to compute the loss.  While installed on the calling thread,
 * every launch of a kernel whose id bit is set in
 * `kernel_mask` is bracketed by hipEventRecord(start_events[i]) and
 * hipEventRecord(end_events[i]) on the call's stream, its id is stored in
 * kinds[i] (if kinds is not NULL) and *count is incremented, for
 * i = *count < capacity; launches beyond `capacity` are not recorded.
 * start_events/end_events hold hipEvent_t handles (as void*) created by the
 * caller in the same HIP runtime as this library; all arrays are host
 * memory owned by the caller and must outlive the calls they log.  The hook
 * applies to every entry point above.  A zero
 * `kernel_mask` (or NULL count) removes the hook.  Returns KD_OK, or
 * KD_ERR_INVALID_ARG for a non-zero mask with NULL events or capacity < 0.
 */
int kd_set_launch_log(uint32_t kernel_mask, void *const *start_events,
                      void *const *end_events, int32_t *kinds,
                      int32_t capacity, int32_t *count);

/* Static, NUL-terminated description of a status code.  For KD_ERR_HIP the
 * text also carries the HIP error string of the last failure on the calling
 * thread.  Never NULL. */
const char *kd_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KD_TOPK_KL_H */
