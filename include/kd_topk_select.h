/*
 * kd_topk_select.h -- C ABI of the teacher top-K cache producer (MI355X,
 * gfx950), the step that builds the offline cache the loss in kd_topk_kl.h
 * consumes.
 *
 * Source: [TH] ai-thai.com/posts/846, Thai translation of the Hugging Face
 * post "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a
 * Fused Chunked KL Loss", section "Offline distillation": the teacher is run
 * once over the data and, per position, only its top-100 logits and their
 * token ids are stored.
 *
 * Operation: for every row t of logits [T, V], the K largest values and their
 * column ids, written to topk_idx[t, 0..K) and topk_logit[t, 0..K) in
 * decreasing order.  Equal values are ordered by increasing id.  The order is
 * the total order of the IEEE bit patterns (-0.0 below +0.0, -inf the
 * smallest number, NaN below everything), so the result is unique.  bf16
 * inputs are widened exactly to the fp32 outputs; a selected NaN is returned
 * as a NaN, not with its original bits.
 *
 * Memory: device pointers owned by the caller; the library allocates nothing,
 * keeps no state, enqueues on `stream` (a hipStream_t, NULL = default) and
 * returns without synchronising.  Every argument check runs on the host before
 * anything is enqueued; on error nothing is enqueued.
 *
 * Layouts: logits [T, ld] row-major (ld >= V elements of `dtype`; the first V
 * of each row are used), aligned to its element size (rows are read with
 * 16-byte loads from their first 16-byte boundary on); topk_idx [T, K] int32
 * and topk_logit [T, K] fp32, 4-byte aligned.
 */
#ifndef KD_TOPK_SELECT_H
#define KD_TOPK_SELECT_H

#include "kd_topk_kl.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t T;          /* rows (positions) */
    int64_t V;          /* values per row (vocabulary size), < 2^31 */
    int64_t K;          /* kept per row, 1 <= K <= min(V, 1024) */
    int64_t ld;         /* row pitch in elements, >= V */
    int32_t dtype;      /* kd_dtype of the logits: KD_BF16 or KD_F32 */
    int32_t reserved;   /* must be 0 */
} kd_select_problem;

/* Errors: KD_ERR_NULL (a pointer is NULL while T > 0), KD_ERR_SHAPE (T < 0,
 * V < 1, K < 1, K > V, ld < V), KD_ERR_VALUE (reserved != 0),
 * KD_ERR_UNSUPPORTED (dtype, K > 1024, V or T beyond 2^31 - 1), KD_ERR_ALIGN,
 * KD_ERR_HIP. */
kd_status kd_topk_select(const kd_select_problem* prob, const void* logits, int32_t* topk_idx, float* topk_logit,
                         void* stream);

/*
 * Teacher cache straight from the teacher's last hidden states: for every
 * position t, the K largest of the logits z[t, v] = H[t, :] . W[v, :] over the
 * whole vocabulary, with their ids, in the order of kd_topk_select (the same
 * source passage: the teacher runs once and only its top-K logits per position
 * are kept).  The logits are computed with fp32 accumulation of the operand
 * dtype, chunk by chunk (`chunk` positions at a time, 0 = 4096): each chunk's
 * fp32 logits go to the workspace and are reduced there, so the [T, V] logit
 * matrix never exists and the workspace does not depend on T.
 *
 * Layouts: H [T, d] and W [V, d] row-major (the nn.Linear weight layout), bf16
 * or fp32, 16-byte aligned, d a multiple of 8; topk_idx [T, K] int32 and
 * topk_logit [T, K] fp32, 4-byte aligned; workspace 16-byte aligned, at least
 * kd_teacher_topk_workspace_size bytes.  Ownership, streams and the error
 * convention as above; KD_ERR_UNSUPPORTED also for d % 8 != 0, V > 2^21,
 * chunk > 2^20, or (fp32) an operand beyond 2^31 bytes; KD_ERR_WORKSPACE when
 * workspace_bytes is too small.
 */
typedef struct {
    int64_t T;          /* positions */
    int64_t d;          /* hidden size */
    int64_t V;          /* vocabulary size */
    int64_t K;          /* kept per position, 1 <= K <= min(V, 1024) */
    int64_t chunk;      /* positions per chunk, 0 = default */
    int32_t dtype;      /* kd_dtype of H and W */
    int32_t reserved;   /* must be 0 */
} kd_teacher_problem;

kd_status kd_teacher_topk_workspace_size(const kd_teacher_problem* prob, size_t* bytes);
kd_status kd_teacher_topk(const kd_teacher_problem* prob, const void* H, const void* W, int32_t* topk_idx,
                          float* topk_logit, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KD_TOPK_SELECT_H */
