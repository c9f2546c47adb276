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

#ifdef __cplusplus
}
#endif

#endif /* KD_TOPK_SELECT_H */
