/*
 * rlk.h -- C ABI of the fused row-wise log-softmax library for AMD MI355X
 * (gfx950).  Plain pointers and sizes only; no HIP or torch types appear in
 * the signatures (the stream is passed as a void* that holds a hipStream_t).
 *
 * What is computed (sources are web pages on the subject, cited by title and
 * section):
 *   - "Final Logit Softcap" (RL-Kernel operator documentation), Summary and
 *     Tensor and Precision Contract: the elementwise cap y = c * tanh(x / c)
 *     with a runtime cap, its derivative 1 - tanh^2(x / c), fp32 internal
 *     math and one trailing cast;
 *   - "Add Triton kernels for vocab-parallel logprobs, entropy and KL"
 *     (DeepSpeed pull request 8838), Changes and the review comment on
 *     reading each logit once: per-token logprobs (k = 1 and top-k),
 *     entropy and KL against a second logit tensor, computed from online
 *     row statistics (running max, sum of exponentials and a weighted sum)
 *     in a single read of each logit, with a support-mismatch rule;
 *   - "perf(logp): fused zero-workspace backward for the generic CUDA fused
 *     logp" (RL-Kernel pull request 495), Summary and Behavior changes: the
 *     backward g * (onehot - softmax) written straight in the logits dtype
 *     with no [N, V] temporary, and targets outside [0, V) (such as -100)
 *     giving output 0 and an exactly zero gradient.
 *
 * Conventions common to every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates, frees and copies nothing and keeps no state between calls.
 *   - Logits are fp32, bf16 or fp16 (rlk_dtype).  All arithmetic is fp32; head
 *     outputs are fp32; gradients with respect to the logits are written in
 *     the logits dtype with a single round-to-nearest-even cast.
 *   - A logits matrix is [N, V] row-major with row stride ld >= V elements
 *     (padding between rows is never read).  Gradients are written
 *     contiguous [N, V].  Inputs are never modified; outputs must not alias
 *     inputs.
 *   - softcap: 0.0f turns the fused cap off; any other value must be finite
 *     and > 0.  The standalone softcap calls require a finite cap > 0.  The
 *     fused cap forms y = c tanh(x / c) around a constant, so y carries an
 *     absolute error of about c * 2^-23 whatever x (below every tolerance of
 *     the tests up to c = 200); the standalone calls are accurate relative to
 *     y.
 *   - N == 0 (or n == 0) returns RLK_OK without any HIP call.
 *   - Every argument is validated on the host before anything is launched;
 *     on error nothing is launched and rlk_last_error() describes the
 *     problem.  The launch goes to the device that owns the first tensor
 *     pointer (all pointers must live on it, else RLK_ERR_DEVICE); the
 *     caller's current device is restored afterwards.  Calls are
 *     asynchronous on `stream` (0 = the null stream); faults inside a kernel
 *     surface at the caller's next synchronisation.
 *   - A call enqueues kernel launches on `stream` and nothing else (no
 *     allocation, synchronisation, memset or copy), so calls may be captured
 *     into a HIP graph with hipStreamBeginCapture and replayed; a replay
 *     reads the captured buffers' current contents and gives the bits of an
 *     eager call on them.
 *   - A *_bwd call must receive the `stats` buffer written by the matching
 *     *_fwd call with identical inputs and arguments, ordered after it (same
 *     stream, or after a synchronisation).
 *   - Results are deterministic and batch-invariant: a row's outputs depend
 *     only on that row's data, V and the arguments, never on N, on the other
 *     rows or on the row stride.
 */
#ifndef RLK_H
#define RLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RLK_ABI_VERSION 1

/* Largest top-k width accepted by rlk_logp_fwd / rlk_logp_bwd. */
#define RLK_MAX_TOPK 4096

typedef enum { RLK_F32 = 0, RLK_BF16 = 1, RLK_F16 = 2 } rlk_dtype;

typedef enum {
    RLK_OK = 0,
    RLK_ERR_ARG = 1,    /* null pointer, bad cap, bad enum value          */
    RLK_ERR_DTYPE = 2,  /* dtype outside rlk_dtype (fp64, ints, ...)      */
    RLK_ERR_SHAPE = 3,  /* N < 0, V < 1, ld < V, k out of range, overflow */
    RLK_ERR_DEVICE = 4, /* pointer not device memory, or on another GPU   */
    RLK_ERR_LAUNCH = 5  /* the HIP runtime refused a launch               */
} rlk_status;

typedef enum { RLK_HEAD_LOGP = 0, RLK_HEAD_ENTROPY = 1, RLK_HEAD_KL = 2 } rlk_head;

/* RLK_KL_REVERSE: KL(policy || ref) = sum p (log p - log q).
 * RLK_KL_FORWARD: KL(ref || policy) = sum q (log q - log p). */
typedef enum { RLK_KL_REVERSE = 0, RLK_KL_FORWARD = 1 } rlk_kl_dir;

/* Row layout of a two-stride view (the `_strided` entry points).  Row i of N
 * is (b, t) = (i / rows_per_batch, i % rows_per_batch) and starts at element
 * b * batch_stride + t * row_stride; the vocabulary dimension is unit-stride.
 * A [B, T, V] tensor with strides (sB, sT, 1) is {T, sB, sT} with N = B * T;
 * e.g. logits[:, :-1] of a contiguous [B, T + 1, V] tensor is
 * {T, (T + 1) * V, V}, read in place ("Add Triton kernels for vocab-parallel
 * logprobs, entropy and KL", review comment: rows addressed with up to two
 * strides so a sequence slice is not copied).  A plain [N, V] matrix with row
 * stride ld is {N, 0, ld}.  rows_per_batch >= 1 and strides >= 0; input rows
 * may overlap (broadcast views), gradient rows must not. */
typedef struct {
    int64_t rows_per_batch;
    int64_t batch_stride;
    int64_t row_stride;
} rlk_rows;

/* ABI version of the loaded library (RLK_ABI_VERSION at build time). */
int rlk_abi_version(void);

/* Bytes of the per-row forward->backward record for `head` (N rows of
 * width V); the caller allocates it in device memory.  The layout is
 * private to the library.  Returns 0 for N <= 0, an unknown head, or a
 * size that does not fit size_t. */
size_t rlk_stats_bytes(rlk_head head, int64_t N, int64_t V);

/* Static text of a status code. */
const char* rlk_status_str(rlk_status s);

/* Detail of the last error raised on the calling host thread ("" if none). */
const char* rlk_last_error(void);

/* ------------------------------------------------------------- softcap
 * "Final Logit Softcap", Summary and Tensor and Precision Contract.
 * y[i] = cap * tanh(x[i] / cap) for n elements, x in x_dtype, y in y_dtype
 * (RLK_F32: the fp32 output of the fused kernel; x_dtype: the cast-back
 * `forward` variant).  fp32 math with one trailing cast.  -inf maps to -cap.
 * cap must be finite and > 0 (else RLK_ERR_ARG). */
rlk_status rlk_softcap_fwd(const void* x, rlk_dtype x_dtype, void* y, rlk_dtype y_dtype,
                           int64_t n, float cap, void* stream);

/* grad_x[i] = grad_y[i] * (1 - tanh^2(x[i] / cap)), recomputed from the saved
 * input x; grad_y is fp32, grad_x is written in x_dtype. */
rlk_status rlk_softcap_bwd(const void* x, rlk_dtype x_dtype, const float* grad_y, void* grad_x,
                           int64_t n, float cap, void* stream);

/* ------------------------------------------------------------ logprobs
 * Pull request 8838 (Changes) and pull request 495 (Summary, Behavior
 * changes).  targets is int64 [N, k] (k = 1: per-token logprobs; k > 1:
 * top-k ids, 1 <= k <= RLK_MAX_TOPK).  With y = softcap(x) (or x):
 *   logp[i, j] = y[i, t_ij] - logsumexp(y[i, :])  if 0 <= t_ij < V,
 *   logp[i, j] = 0                                otherwise (ignored),
 * NaN for a valid target in a row whose logits are all -inf, -inf for a
 * valid target on a masked (-inf) column.  stats: rlk_stats_bytes(LOGP). */
rlk_status rlk_logp_fwd(const void* logits, rlk_dtype dtype, int64_t N, int64_t V, int64_t ld,
                        const int64_t* targets, int64_t k, float softcap, float* logp,
                        void* stats, void* stream);

/* grad_logits[i, v] = (h_iv - p_iv * G_i) * dy/dx, where G_i is the sum of
 * grad_logp[i, j] over valid slots and h_iv the sum over valid slots with
 * t_ij == v (duplicates add, ascending j, in fp32 before the single cast).
 * A row without any valid slot is exactly zero; otherwise a row whose logits
 * are all -inf is NaN.  grad_logp is fp32 [N, k]; grad_logits is [N, V]
 * contiguous in `dtype`. */
rlk_status rlk_logp_bwd(const void* logits, rlk_dtype dtype, int64_t N, int64_t V, int64_t ld,
                        const int64_t* targets, int64_t k, float softcap, const void* stats,
                        const float* grad_logp, void* grad_logits, void* stream);

/* -------------------------------------------------------------- entropy
 * Pull request 8838, review comment: H = log S - W / S computed from one
 * read of each logit.  entropy[i] = -sum_v p_iv log p_iv (0 log 0 = 0);
 * NaN for a row whose logits are all -inf. */
rlk_status rlk_entropy_fwd(const void* logits, rlk_dtype dtype, int64_t N, int64_t V, int64_t ld,
                           float softcap, float* entropy, void* stats, void* stream);

/* grad_logits[i, v] = -g_i p_iv (log p_iv + H_i) * dy/dx (masked columns: 0;
 * rows whose logits are all -inf: NaN). */
rlk_status rlk_entropy_bwd(const void* logits, rlk_dtype dtype, int64_t N, int64_t V, int64_t ld,
                           float softcap, const void* stats, const float* grad_entropy,
                           void* grad_logits, void* stream);

/* ------------------------------------------------------------------- KL
 * Pull request 8838, review comment: KL(A || B) = W / S_A - log S_A +
 * log S_B from one read of both tensors.  kl[i] is NaN if either row is all
 * -inf, +inf if the second distribution masks a column the first supports
 * (decided on the logits, even where the probability underflows), else the
 * sum above.  policy and ref share dtype and V; each has its own row stride
 * and its own cap. */
rlk_status rlk_kl_fwd(const void* policy, const void* ref, rlk_dtype dtype, int64_t N, int64_t V,
                      int64_t ld_policy, int64_t ld_ref, rlk_kl_dir dir, float softcap_policy,
                      float softcap_ref, float* kl, void* stats, void* stream);

/* Gradient with respect to the policy logits only (the reference is
 * detached):  reverse: g p (log p - log q - D) * dy/dx  (masked policy
 * columns: 0; support-mismatch rows: NaN on the policy's support, 0 off it);
 * forward: g (p - q) * dy/dx.  Rows where either input is all -inf: NaN. */
rlk_status rlk_kl_bwd(const void* policy, const void* ref, rlk_dtype dtype, int64_t N, int64_t V,
                      int64_t ld_policy, int64_t ld_ref, rlk_kl_dir dir, float softcap_policy,
                      float softcap_ref, const void* stats, const float* grad_kl,
                      void* grad_policy, void* stream);

/* ------------------------------------------------ two-stride row views
 * The same heads on rows laid out by rlk_rows (inputs read in place, the
 * gradient written through its own layout, e.g. straight into the slice of a
 * full [B, T + 1, V] gradient buffer).  Semantics, outputs ([N], [N, k] in
 * row order i = b * T + t), errors and the stats record are exactly those of
 * the matching plain call; results are bitwise identical to it. */
rlk_status rlk_logp_fwd_strided(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                                const rlk_rows* rows, const int64_t* targets, int64_t k,
                                float softcap, float* logp, void* stats, void* stream);
rlk_status rlk_logp_bwd_strided(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                                const rlk_rows* rows, const int64_t* targets, int64_t k,
                                float softcap, const void* stats, const float* grad_logp,
                                void* grad_logits, const rlk_rows* grad_rows, void* stream);
rlk_status rlk_entropy_fwd_strided(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                                   const rlk_rows* rows, float softcap, float* entropy,
                                   void* stats, void* stream);
rlk_status rlk_entropy_bwd_strided(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                                   const rlk_rows* rows, float softcap, const void* stats,
                                   const float* grad_entropy, void* grad_logits,
                                   const rlk_rows* grad_rows, void* stream);
rlk_status rlk_kl_fwd_strided(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                              int64_t V, const rlk_rows* policy_rows, const rlk_rows* ref_rows,
                              rlk_kl_dir dir, float softcap_policy, float softcap_ref, float* kl,
                              void* stats, void* stream);
rlk_status rlk_kl_bwd_strided(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                              int64_t V, const rlk_rows* policy_rows, const rlk_rows* ref_rows,
                              rlk_kl_dir dir, float softcap_policy, float softcap_ref,
                              const void* stats, const float* grad_kl, void* grad_policy,
                              const rlk_rows* grad_rows, void* stream);

/* ------------------------------------------------- KL: both directions,
 * reference gradient.  "Add Triton kernels for vocab-parallel logprobs,
 * entropy and KL", Changes: both KL directions are offered and the reference
 * is detached there; a caller that trains both distributions needs the
 * gradient with respect to the reference too.
 *
 * rlk_kl_fwd_both: reverse KL(P||R) and forward KL(R||P) from one read of
 * the pair; each output and row record is bit-identical to the one
 * rlk_kl_fwd writes for that direction, so either record feeds rlk_kl_bwd /
 * rlk_kl_bwd_ref of its direction. */
rlk_status rlk_kl_fwd_both(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                           int64_t V, int64_t ld_policy, int64_t ld_ref, float softcap_policy,
                           float softcap_ref, float* kl_reverse, void* stats_reverse,
                           float* kl_forward, void* stats_forward, void* stream);
rlk_status rlk_kl_fwd_both_strided(const void* policy, const void* ref, rlk_dtype dtype,
                                   int64_t N, int64_t V, const rlk_rows* policy_rows,
                                   const rlk_rows* ref_rows, float softcap_policy,
                                   float softcap_ref, float* kl_reverse, void* stats_reverse,
                                   float* kl_forward, void* stats_forward, void* stream);

/* Gradient with respect to the reference logits (ref's layout, dtype, cap),
 * from the record of the same direction's forward:
 *   reverse KL(P||R): g (q - p) * dr/dref on every row where both inputs
 *     exist (a support-mismatch row included: no infinite term enters it);
 *   forward KL(R||P): g q (log q - log p - D) * dr/dref, 0 on the
 *     reference's masked columns, NaN on its support of a mismatch row.
 * Rows where either input is all -inf: NaN.  grad_ref is [N, V] contiguous
 * (strided: its own rlk_rows). */
rlk_status rlk_kl_bwd_ref(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                          int64_t V, int64_t ld_policy, int64_t ld_ref, rlk_kl_dir dir,
                          float softcap_policy, float softcap_ref, const void* stats,
                          const float* grad_kl, void* grad_ref, void* stream);
rlk_status rlk_kl_bwd_ref_strided(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                                  int64_t V, const rlk_rows* policy_rows,
                                  const rlk_rows* ref_rows, rlk_kl_dir dir, float softcap_policy,
                                  float softcap_ref, const void* stats, const float* grad_kl,
                                  void* grad_ref, const rlk_rows* grad_rows, void* stream);

/* ------------------------------------------------- vocabulary shards
 * The single-GPU half of vocabulary parallelism ("Add Triton kernels for
 * vocab-parallel logprobs, entropy and KL", Changes and review comment:
 * local statistics from one read, rescaled to the global maximum and summed;
 * the mismatch flag travels with the maximum).  A shard holds the columns
 * [v0, v0 + V_shard) of rows of width V_total.
 *   1. each shard: rlk_*_fwd_partial -> one 32-byte record per row
 *      (rlk_partial_bytes), and for logprobs the statistic input of every
 *      target it owns ([N, k] floats, unowned slots 0);
 *   2. gather the P records (and target values) in rank order into
 *      [P, N] (and [P, N, k]) device buffers -- the only cross-rank step;
 *   3. rlk_combine folds them in rank order with the merges of the row
 *      kernels and writes the heads and the row record, identically on every
 *      rank that combines the same gathered data;
 *   4. backward per shard: rlk_logp_bwd_shard, or the plain
 *      rlk_entropy_bwd / rlk_kl_bwd on the shard's columns with the combined
 *      record.  A one-shard combine gives bitwise the plain forward. */
#define RLK_MAX_SHARDS 64

/* Bytes of N partial records (32 per row); 0 for N <= 0 or a size that
 * does not fit size_t. */
size_t rlk_partial_bytes(int64_t N);

rlk_status rlk_logp_fwd_partial(const void* logits, rlk_dtype dtype, int64_t N, int64_t V_shard,
                                int64_t ld, int64_t v0, int64_t V_total, const int64_t* targets,
                                int64_t k, float softcap, void* partial, float* target_vals,
                                void* stream);
rlk_status rlk_entropy_fwd_partial(const void* logits, rlk_dtype dtype, int64_t N,
                                   int64_t V_shard, int64_t ld, float softcap, void* partial,
                                   void* stream);
rlk_status rlk_kl_fwd_partial(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                              int64_t V_shard, int64_t ld_policy, int64_t ld_ref, rlk_kl_dir dir,
                              float softcap_policy, float softcap_ref, void* partial,
                              void* stream);

/* Fold P shard records [P, N] (rank order; bounds = host array of P + 1
 * increasing columns, bounds[0] = 0, bounds[P] = V_total) and write the
 * head outputs (logp [N, k], entropy [N] or KL [N]) and the row record
 * `stats` (rlk_stats_bytes).  Logprobs also needs targets [N, k],
 * target_vals [P, N, k] and the softcap; `dir` is read for KL only. */
rlk_status rlk_combine(rlk_head head, rlk_kl_dir dir, int64_t P, const int64_t* bounds, int64_t N,
                       const void* partials, const int64_t* targets, int64_t k,
                       const float* target_vals, float softcap, float* out, void* stats,
                       void* stream);

/* Logprobs backward of one shard with the combined record; targets are
 * global column ids; grad_logits is [N, V_shard] contiguous. */
rlk_status rlk_logp_bwd_shard(const void* logits, rlk_dtype dtype, int64_t N, int64_t V_shard,
                              int64_t ld, int64_t v0, int64_t V_total, const int64_t* targets,
                              int64_t k, float softcap, const void* stats,
                              const float* grad_logp, void* grad_logits, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RLK_H */
