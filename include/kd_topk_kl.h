/*
 * kd_topk_kl.h -- C ABI of the MI355X (gfx950) fused chunked top-K KL
 * distillation loss.
 *
 * The operation.  A student's final projection (lm_head) is fused into a
 * KL-divergence distillation loss against an offline teacher cache that keeps,
 * per position, only the teacher's top-K token ids and logits.  Positions are
 * processed in chunks of C rows: each chunk's logits H_c W^T are formed,
 * consumed and discarded, so the T x V student logit matrix never exists, and
 * the backward pass recomputes a chunk's logits instead of storing them.
 * Sources (web pages describing the method; they give no formulas or code):
 *   [TH] ai-thai.com/posts/846, Thai translation of the Hugging Face post
 *        "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a
 *        Fused Chunked KL Loss": section "Offline distillation" (the top-100
 *        cache), section "Fused Chunked KL Loss", items "Dense KL" (teacher
 *        distribution rebuilt from the cached logits), "Fused chunked KL"
 *        (projection fused into the loss, per-slice logits discarded, backward
 *        recomputes each slice, memory linear in sequence length).
 *   [RU] iitog.ru, "Multiverse Computing сократила видеопамять для дистилляции
 *        нейросетей до 15,6 раза": the paragraph on the two system changes.
 * Definition (the plain reading of those passages; the pages fix no formula):
 *   a_tv   = (H_t . W_v) / tau                     student logits over the full vocabulary
 *   lse_t  = log sum_v exp(a_tv)                    (full-vocabulary logsumexp)
 *   p_tk   = softmax_k(topk_logit_tk / tau)         teacher, renormalised over the K cached ids
 *   L_t    = sum_k p_tk (log p_tk - a_{t,idx_tk} + lse_t)      = KL(p_t || q_t) on the cached ids
 *   loss   = (1/N) sum_{t: ignore_t == 0} L_t,  N = #{t: ignore_t == 0}; loss = 0 when N = 0
 *   G_tv   = g/(tau N) (exp(a_tv - lse_t) - P_tv),  P_tv = sum_{k: idx_tk = v} p_tk  (0 on ignored rows)
 *   grad_H = G W,  grad_W = G^T H                   (g = upstream gradient of loss)
 * There is no temperature-squared factor and no gradient to the teacher inputs.
 *
 * Memory and ownership.
 *   - Every array argument is DEVICE memory owned by the caller; the library
 *     allocates nothing and keeps no state between calls.  Scratch memory
 *     comes from the caller's workspace, sized by kd_topk_kl_workspace_size;
 *     its size depends on (C, V, K, d) and not on T.
 *   - All work is enqueued on the caller's HIP stream (`stream`, a
 *     hipStream_t; NULL = the default stream).  Calls return after enqueueing
 *     and never synchronise; results are ready when the stream reaches them.
 *   - Calls on different streams with separate workspaces may run
 *     concurrently; two in-flight calls must not share a workspace.
 *   - Results are run-to-run bitwise deterministic for a given problem,
 *     chunk size and device (fixed reduction orders, no float atomics).
 *
 * Layouts (row-major, contiguous):
 *   H          [T, d]  element type `dtype`
 *   W          [V, d]  element type `dtype` (the nn.Linear weight layout)
 *   topk_idx   [T, K]  int32, ids in [0, V)
 *   topk_logit [T, K]  fp32 teacher logits (-inf allowed: probability 0), or
 *                      bf16 bit patterns with KD_FLAG_LOGIT_BF16
 *   ignore     [T]     uint8, non-zero = position excluded; NULL = none excluded
 *   loss       [1]     fp32; lse, row_loss [T] fp32
 *   grad_H     [T, d]  element type `dtype` (rounded to nearest even from fp32), overwritten
 *   grad_W     [V, d]  fp32, overwritten (added to with KD_FLAG_ACCUMULATE_GRAD_W)
 * Alignment: H, W, grad_H, grad_W and workspace 16 bytes; the fp32/int32
 * arrays 4 bytes; a bf16 topk_logit 2 bytes.  Outputs must not alias inputs or each other.
 *
 * Errors.  Every argument check runs on the host before anything is enqueued;
 * on error nothing is enqueued and the outputs are untouched.  No C++
 * exception crosses this interface.  Out-of-range ids and kept positions whose
 * teacher logits are all -inf (or NaN) are preconditions, not checked on the
 * hot path: they give undefined values but never an out-of-bounds memory
 * access (ids are clamped into [0, V) before any load or store);
 * kd_topk_kl_validate reports them.  Cache contents of ignored positions are
 * never read.
 */
#ifndef KD_TOPK_KL_H
#define KD_TOPK_KL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KD_OK = 0,
    KD_ERR_NULL = 1,         /* a required pointer is NULL */
    KD_ERR_SHAPE = 2,        /* T < 0, d < 1, V < 1, K < 1, K > V, chunk < 0 */
    KD_ERR_VALUE = 3,        /* temperature not finite or <= 0, unknown flags, reserved != 0 */
    KD_ERR_ALIGN = 4,        /* a pointer violates the alignment above */
    KD_ERR_WORKSPACE = 5,    /* workspace_bytes below kd_topk_kl_workspace_size */
    KD_ERR_UNSUPPORTED = 6,  /* dtype unknown, d % 8 != 0, K > 1024, V > 2^21, T >= 2^31, chunk or d > 2^20,
                                or (fp32) an operand beyond 2^31 bytes */
    KD_ERR_HIP = 7,          /* a HIP launch failed (asynchronous faults surface at the caller's next sync) */
    KD_ERR_INTERNAL = 8
} kd_status;

typedef enum { KD_BF16 = 0, KD_F32 = 1 } kd_dtype;

typedef enum { KD_OP_FORWARD = 0, KD_OP_BACKWARD = 1, KD_OP_FUSED = 2 } kd_op;

/* Options (kd_problem.flags), for use inside a training step:
 *   KD_FLAG_ACCUMULATE_GRAD_W  backward and fused add G^T H to the caller's
 *                              grad_W instead of overwriting it (e.g. straight
 *                              into a parameter's gradient buffer, or for an
 *                              output projection tied to the input embedding,
 *                              whose other gradient is already there);
 *   KD_FLAG_LOGIT_BF16         topk_logit holds bfloat16 values (a cache of
 *                              half the size); they are widened exactly to fp32. */
enum { KD_FLAG_ACCUMULATE_GRAD_W = 1, KD_FLAG_LOGIT_BF16 = 2 };

typedef struct {
    int64_t T;            /* positions (batch x sequence, flattened) */
    int64_t d;            /* hidden size, multiple of 8 */
    int64_t V;            /* vocabulary size */
    int64_t K;            /* cached teacher entries per position, 1 <= K <= min(V, 1024) */
    int64_t chunk;        /* rows per chunk C; 0 = library default (kd_topk_kl_default_chunk) */
    int32_t dtype;        /* kd_dtype of H, W and grad_H */
    float temperature;    /* tau > 0, divides both teacher and student logits */
    int32_t flags;        /* KD_FLAG_* bits (0 = overwrite grad_W, fp32 teacher logits); others: KD_ERR_VALUE */
    int32_t reserved;     /* must be 0 (KD_ERR_VALUE otherwise) */
} kd_problem;

/* Chunk size used when prob->chunk == 0 (depends on d, V and dtype only). */
int64_t kd_topk_kl_default_chunk(const kd_problem* prob);

/* Bytes of workspace `op` needs for `prob`; writes them to *bytes and returns
 * KD_OK, or returns the status that the entry itself would return for an
 * invalid `prob` or `op` (*bytes is then untouched).  The value depends on
 * (C, V, K, d, dtype), not on T. */
kd_status kd_topk_kl_workspace_size(const kd_problem* prob, kd_op op, size_t* bytes);

/* Forward ([TH] "Fused chunked KL": per chunk, project, take the
 * full-vocabulary logsumexp, gather the student at the cached ids, accumulate,
 * discard).  Writes loss[1], lse[T] (needed by kd_topk_kl_backward; written
 * for every position, ignored ones too) and, if non-NULL, row_loss[T] (0 on
 * ignored positions). */
kd_status kd_topk_kl_forward(const kd_problem* prob, const void* H, const void* W,
                             const int32_t* topk_idx, const void* topk_logit,
                             const uint8_t* ignore, float* loss, float* lse, float* row_loss,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Backward ([TH] "Fused chunked KL": each chunk's logits are recomputed, not
 * stored).  Takes lse[T] from kd_topk_kl_forward and the upstream gradient
 * grad_loss[1] (device fp32; NULL means 1).  Overwrites grad_H[T, d] and
 * grad_W[V, d]. */
kd_status kd_topk_kl_backward(const kd_problem* prob, const void* H, const void* W,
                              const int32_t* topk_idx, const void* topk_logit,
                              const uint8_t* ignore, const float* lse, const float* grad_loss,
                              void* grad_H, float* grad_W,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Forward and backward in one pass over the chunks ([TH] "Fused Chunked KL
 * Loss", item "Fused chunked KL": the output projection is fused into the
 * loss and the positions are handled slice by slice, so neither the T x V
 * student logits nor a T x V gradient ever exists).  Here each chunk's logits
 * are projected once and reused for the loss and both gradients, instead of
 * being recomputed in a separate backward pass.  grad_loss[1] is the upstream
 * gradient (device fp32; NULL means 1).  Writes loss[1], grad_H[T, d] and
 * grad_W[V, d] (overwritten, or added to with KD_FLAG_ACCUMULATE_GRAD_W) and,
 * if non-NULL, lse[T] and row_loss[T], with the same values as the forward
 * entry.  Errors as for the other entries. */
kd_status kd_topk_kl_fused(const kd_problem* prob, const void* H, const void* W,
                           const int32_t* topk_idx, const void* topk_logit,
                           const uint8_t* ignore, const float* grad_loss,
                           float* loss, float* lse, float* row_loss,
                           void* grad_H, float* grad_W,
                           void* workspace, size_t workspace_bytes, void* stream);

/* The fused entry without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and errors as
 * kd_topk_kl_fused otherwise.  Its workspace is a static 256 MiB device
 * array of the library, one per GPU, held from the library's first use on
 * that GPU until the process ends; the call uses the array of the current
 * device (`stream` must belong to it) and allocates nothing.
 *   - prob->chunk == 0: the largest chunk (at most the default chunk and the
 *     positions rounded up to 64) whose fused workspace fits 256 MiB, e.g.
 *     about 600 rows at a 201,088-token vocabulary.  A problem whose workspace
 *     exceeds 256 MiB even for one row, or an explicit chunk whose workspace
 *     exceeds it (kd_topk_kl_workspace_size(prob, KD_OP_FUSED) > 256 MiB),
 *     returns KD_ERR_WORKSPACE with nothing enqueued.
 *   - Every call on a GPU shares that GPU's array and leaves its contents
 *     behind; each call rewrites whatever it reads there first, so nothing
 *     needs clearing between calls.  Calls that overlap in time on one GPU
 *     (different streams or threads) race on the array and must be ordered
 *     by the caller. */
kd_status kd_topk_kl_fused_noalloc(const kd_problem* prob, const void* H, const void* W,
                                   const int32_t* topk_idx, const void* topk_logit,
                                   const uint8_t* ignore, const float* grad_loss,
                                   float* loss, float* lse, float* row_loss,
                                   void* grad_H, float* grad_W, void* stream);

/* Debug check of the cache preconditions: writes to bad_count[0] (device
 * int64) the number of ids outside [0, V) plus the number of kept positions
 * whose teacher logits are all -inf or contain NaN. */
kd_status kd_topk_kl_validate(const kd_problem* prob, const int32_t* topk_idx,
                              const void* topk_logit, const uint8_t* ignore,
                              int64_t* bad_count, void* stream);

/* Writes out_H = g * grad_H and out_W = g * grad_W, g = grad_loss[0] (device
 * fp32; NULL means 1).  For callers that run kd_topk_kl_fused with
 * grad_loss = NULL (g = 1) before the upstream gradient is known -- an
 * autograd function whose forward already produced the gradients -- and apply
 * g afterwards: G, and so both gradients, are proportional to g.
 *   grad_H, out_H  [T, d] element type `dtype` (rounded to nearest even);
 *                  out_H may be grad_H itself (in place).
 *   grad_W         [V, d] fp32, as the backward and fused entries leave it.
 *   out_W          [V, d] fp32 (out_w_dtype = KD_F32; may be grad_W itself) or
 *                  bf16 (out_w_dtype = KD_BF16, rounded to nearest even: the
 *                  weight's own type for a bf16 model; must not overlap grad_W).
 * Each input/output pair may be NULL (both) to skip it; out of place, the
 * inputs are left untouched, so the kept gradients can be scaled again by
 * another g.  Only prob->T, d, V, dtype are used (checked as elsewhere).
 * Errors: KD_ERR_NULL (one of a pair missing), KD_ERR_ALIGN (16 bytes for the
 * arrays, 4 for grad_loss), KD_ERR_UNSUPPORTED (out_w_dtype unknown),
 * KD_ERR_VALUE (an output partly overlaps its input). */
kd_status kd_topk_kl_scale_grads(const kd_problem* prob, const float* grad_loss, const void* grad_H,
                                 const float* grad_W, void* out_H, void* out_W, int32_t out_w_dtype, void* stream);

/* Kernel stages of every call, for timing. */
typedef enum {
    KD_STAGE_LOGITS = 0,   /* logits GEMM of a chunk (with its softmax-statistics epilogue) */
    KD_STAGE_ROWS = 1,     /* per-row kernel of a chunk (lse, teacher, gather, loss, G) */
    KD_STAGE_GRAD_H = 2,   /* grad_H GEMM of a chunk (its split reduction is not included) */
    KD_STAGE_GRAD_W = 3,   /* grad_W GEMM of a chunk */
    KD_NUM_STAGES = 4
} kd_stage;

/* Profiling hook.  While a table is installed for `stage`, the library
 * brackets each launch of that stage with hipEventRecord(begin[i]) and
 * hipEventRecord(end[i]) on the launch stream, for i = *recorded, *recorded+1,
 * ... below `capacity`, incrementing the host counter *recorded at enqueue
 * time.  The events (hipEvent_t) are created and owned by the caller.
 * begin == NULL removes the table.  The tables are process-wide and not
 * synchronised: install them only while no other thread calls the library. */
kd_status kd_topk_kl_set_stage_events(int stage, void* const* begin, void* const* end, int capacity,
                                      int* recorded);

/* Static description of a status code. */
const char* kd_status_string(kd_status status);

#ifdef __cplusplus
}
#endif

#endif /* KD_TOPK_KL_H */
