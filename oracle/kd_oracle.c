/*
 * kd_oracle.c -- plain fp64 CPU oracle of the fused top-K KL distillation loss.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the test-suite, the package smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code with the HIP library.
 *
 * Pages cited (the method's only description available here):
 *   [TH]  ai-thai.com/posts/846, Thai translation of the Hugging Face post
 *         "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and
 *         a Fused Chunked KL Loss".
 *   [RU]  iitog.ru, "Multiverse Computing сократила видеопамять для
 *         дистилляции нейросетей до 15,6 раза".
 *   [PT]  ai2day.live/pt, "Um Novo Método Reduz Drasticamente o Custo de
 *         Compressão de Grandes Modelos de IA".
 *
 * What is computed.  The pages fix no formula; the definition implemented is
 * the plain reading of their description:
 *   - the teacher distribution over a position is built from the K cached
 *     top-K logits alone ([TH] "Fused Chunked KL Loss" section, "Dense KL"
 *     item: the full teacher table is rebuilt from the cached top-100
 *     logits), i.e. p_k = softmax_k(l_k / tau), zero off the cached ids;
 *   - the student distribution is the full-vocabulary softmax of the
 *     projected hidden state, q = softmax_v(H_t . W_v / tau) ([TH] "Fused
 *     chunked KL" item: hidden states -> logits -> loss);
 *   - the distance is the KL divergence of student from teacher ([PT] "O que
 *     os investigadores alteraram?"; [TH] "why is KD expensive"), taken in
 *     the forward direction KL(p || q), restricted to the K cached ids:
 *       L_t = sum_k p_k (log p_k - log q_{t, idx_k});
 *   - loss = (1/N) sum over non-ignored positions of L_t (token mean, N =
 *     number of non-ignored positions; N = 0 gives loss 0 and zero grads).
 *   - no tau^2 factor (none is stated).
 * The gradient (the pages defer the closed form to the full paper, [TH]
 * closing paragraph) is the exact derivative of the above:
 *   dloss/dz_tv = G_tv = g/(tau N) * (q_tv * sum_k p_k - P_tv),  P_tv = sum_{k: idx_k = v} p_k,
 *   grad_H = G W,  grad_W = G^T H.
 * The chunk loop over positions is the fused chunked schedule of [TH] ("Fused
 * chunked KL" item: per slice, project, accumulate, discard); with chunk = T
 * it is the dense evaluation, which the pages use as the correctness baseline
 * and state to be mathematically equal to the chunked ones ([TH] "three
 * equivalent ways").
 *
 * All arithmetic is fp64.  Operands arrive as fp32 arrays holding exact
 * values (bf16 and fp32 inputs widen exactly).  Every output element is
 * produced by one thread in a fixed order, so results do not depend on the
 * OpenMP thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Teacher side of one position ([TH] "Dense KL": distribution from the cached
 * top-K logits).  Writes p[K] and logp[K]; entries with logit -inf get p = 0.
 * Returns 0, or -1 if every logit is -inf (no distribution). */
static int teacher_probs(int64_t K, const float* logit, double tau, double* p, double* logp)
{
    double M = -INFINITY;
    for (int64_t k = 0; k < K; k++) {
        double b = (double)logit[k] / tau;
        if (b > M) M = b;
    }
    if (M == -INFINITY) return -1;
    double S = 0.0;
    for (int64_t k = 0; k < K; k++) S += exp((double)logit[k] / tau - M);
    double logS = log(S);
    for (int64_t k = 0; k < K; k++) {
        double b = (double)logit[k] / tau;
        if (b == -INFINITY) { p[k] = 0.0; logp[k] = -INFINITY; continue; }
        logp[k] = b - M - logS;
        p[k] = exp(logp[k]);
    }
    return 0;
}

/* Student logits of one position: a_v = (H_t . W_v) / tau for every v, with
 * the dot product summed in plain j order.  Returns lse = log sum_v exp(a_v). */
static double student_logits(int64_t d, int64_t V, const float* h, const float* W,
                             double tau, double* a)
{
    double m = -INFINITY;
    for (int64_t v = 0; v < V; v++) {
        const float* w = W + v * d;
        double z = 0.0;
        for (int64_t j = 0; j < d; j++) z += (double)h[j] * (double)w[j];
        a[v] = z / tau;
        if (a[v] > m) m = a[v];
    }
    double s = 0.0;
    for (int64_t v = 0; v < V; v++) s += exp(a[v] - m);
    return m + log(s);
}

/* Row loss L_t = sum_k p_k (log p_k - a_{idx_k} + lse), terms with p_k = 0 skipped. */
static double row_kl(int64_t K, const int32_t* idx, const double* p, const double* logp,
                     const double* a, double lse)
{
    double L = 0.0;
    for (int64_t k = 0; k < K; k++) {
        if (p[k] == 0.0) continue;
        L += p[k] * (logp[k] - a[idx[k]] + lse);
    }
    return L;
}

/* G row (scaled by s = g / (tau N)):  G_v = s (exp(a_v - lse) * sum_k p_k - P_v). */
static void row_grad_logits(int64_t V, int64_t K, const int32_t* idx, const double* p,
                            const double* a, double lse, double s, double* G)
{
    double psum = 0.0;
    for (int64_t k = 0; k < K; k++) psum += p[k];
    for (int64_t v = 0; v < V; v++) G[v] = s * exp(a[v] - lse) * psum;
    for (int64_t k = 0; k < K; k++) G[idx[k]] -= s * p[k];
}

static int64_t count_kept(int64_t T, const uint8_t* ignore)
{
    int64_t N = 0;
    for (int64_t t = 0; t < T; t++) N += (ignore == NULL || ignore[t] == 0);
    return N;
}

/*
 * Full evaluation over all T positions, processed in chunks of C rows
 * (C <= 0 or C >= T: one chunk, the dense evaluation).
 *
 *   H[T,d], W[V,d], topk_logit[T,K]: fp32 arrays of exact operand values.
 *   topk_idx[T,K] int32 in [0, V).  ignore[T] u8 (NULL = none), non-zero = excluded.
 *   tau > 0, g = upstream gradient of the loss.
 * Outputs (fp64): loss[1]; lse[T] (every position, ignored ones too);
 * row_loss[T] (0 for ignored); grad_H[T,d] and grad_W[V,d] (either may be NULL).
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure,
 * -3 if a kept position's teacher logits are all -inf.
 */
int kdo_full(int64_t T, int64_t d, int64_t V, int64_t K, int64_t C,
             const float* H, const float* W, const int32_t* topk_idx,
             const float* topk_logit, const uint8_t* ignore, double tau, double g,
             double* loss, double* lse, double* row_loss, double* grad_H, double* grad_W)
{
    if (T < 0 || d < 1 || V < 1 || K < 1 || K > V || !(tau > 0.0) || !loss) return -1;
    if (C <= 0 || C > T) C = T;
    const int64_t N = count_kept(T, ignore);
    const double s = (N > 0) ? g / (tau * (double)N) : 0.0;
    if (grad_H) memset(grad_H, 0, sizeof(double) * (size_t)(T * d));
    if (grad_W) memset(grad_W, 0, sizeof(double) * (size_t)(V * d));
    *loss = 0.0;
    if (T == 0) return 0;

    double* A  = (double*)malloc(sizeof(double) * (size_t)(C * V));   /* chunk student logits a */
    double* Gc = (double*)malloc(sizeof(double) * (size_t)(C * V));   /* chunk dloss/dz */
    double* P  = (double*)malloc(sizeof(double) * (size_t)(C * K));
    double* LP = (double*)malloc(sizeof(double) * (size_t)(C * K));
    double* Lr = (double*)malloc(sizeof(double) * (size_t)T);
    if (!A || !Gc || !P || !LP || !Lr) { free(A); free(Gc); free(P); free(LP); free(Lr); return -2; }
    int bad = 0;

    for (int64_t t0 = 0; t0 < T; t0 += C) {
        const int64_t rows = (T - t0 < C) ? (T - t0) : C;
        /* forward over the slice: logits, lse, teacher side, row loss, G */
        #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
        for (int64_t r = 0; r < rows; r++) {
            const int64_t t = t0 + r;
            double* a = A + r * V;
            double l = student_logits(d, V, H + t * d, W, tau, a);
            if (lse) lse[t] = l;
            const int kept = (ignore == NULL || ignore[t] == 0);
            double* G = Gc + r * V;
            if (!kept) {
                Lr[t] = 0.0;
                for (int64_t v = 0; v < V; v++) G[v] = 0.0;
                continue;
            }
            double* p = P + r * K;
            double* lp = LP + r * K;
            if (teacher_probs(K, topk_logit + t * K, tau, p, lp) != 0) { bad |= 1; Lr[t] = NAN; continue; }
            Lr[t] = row_kl(K, topk_idx + t * K, p, lp, a, l);
            row_grad_logits(V, K, topk_idx + t * K, p, a, l, s, G);
        }
        /* backward over the slice: grad_H rows (row-local), grad_W (sum over the slice) */
        if (grad_H) {
            #pragma omp parallel for schedule(dynamic, 1)
            for (int64_t r = 0; r < rows; r++) {
                double* gh = grad_H + (t0 + r) * d;
                const double* G = Gc + r * V;
                for (int64_t v = 0; v < V; v++) {
                    const double gv = G[v];
                    if (gv == 0.0) continue;
                    const float* w = W + v * d;
                    for (int64_t j = 0; j < d; j++) gh[j] += gv * (double)w[j];
                }
            }
        }
        if (grad_W) {
            #pragma omp parallel for schedule(static)
            for (int64_t v = 0; v < V; v++) {
                double* gw = grad_W + v * d;
                for (int64_t r = 0; r < rows; r++) {
                    const double gv = Gc[r * V + v];
                    if (gv == 0.0) continue;
                    const float* h = H + (t0 + r) * d;
                    for (int64_t j = 0; j < d; j++) gw[j] += gv * (double)h[j];
                }
            }
        }
    }
    double sum = 0.0;
    for (int64_t t = 0; t < T; t++) sum += Lr[t];
    *loss = (N > 0) ? sum / (double)N : 0.0;
    if (row_loss) memcpy(row_loss, Lr, sizeof(double) * (size_t)T);
    free(A); free(Gc); free(P); free(LP); free(Lr);
    return bad ? -3 : 0;
}

/*
 * Row-local quantities for a subset of positions (for checks at sizes where the
 * full evaluation is too slow): lse, row loss and grad_H of each selected row.
 * These depend only on that row and on N, which is counted from ignore[T].
 *
 *   rows[n]: selected positions; H_rows[n,d], idx_rows[n,K], logit_rows[n,K]
 *   hold those positions' data.  Outputs: lse_out[n], row_loss_out[n],
 *   grad_H_out[n,d] (may be NULL).
 */
int kdo_rows(int64_t T, int64_t d, int64_t V, int64_t K, int64_t n, const int64_t* rows,
             const float* H_rows, const float* W, const int32_t* idx_rows,
             const float* logit_rows, const uint8_t* ignore, double tau, double g,
             double* lse_out, double* row_loss_out, double* grad_H_out)
{
    if (T < 0 || d < 1 || V < 1 || K < 1 || K > V || !(tau > 0.0) || n < 0) return -1;
    const int64_t N = count_kept(T, ignore);
    const double s = (N > 0) ? g / (tau * (double)N) : 0.0;
    int bad = 0;
    #pragma omp parallel reduction(|:bad)
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)V);
        double* G = (double*)malloc(sizeof(double) * (size_t)V);
        double* p = (double*)malloc(sizeof(double) * (size_t)K);
        double* lp = (double*)malloc(sizeof(double) * (size_t)K);
        if (!a || !G || !p || !lp) {
            bad |= 2;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < n; i++) {
                const int64_t t = rows[i];
                if (t < 0 || t >= T) { bad |= 1; continue; }
                double l = student_logits(d, V, H_rows + i * d, W, tau, a);
                lse_out[i] = l;
                double* gh = grad_H_out ? grad_H_out + i * d : NULL;
                if (gh) for (int64_t j = 0; j < d; j++) gh[j] = 0.0;
                if (ignore && ignore[t]) { row_loss_out[i] = 0.0; continue; }
                if (teacher_probs(K, logit_rows + i * K, tau, p, lp) != 0) { bad |= 4; row_loss_out[i] = NAN; continue; }
                row_loss_out[i] = row_kl(K, idx_rows + i * K, p, lp, a, l);
                if (!gh) continue;
                row_grad_logits(V, K, idx_rows + i * K, p, a, l, s, G);
                for (int64_t v = 0; v < V; v++) {
                    const double gv = G[v];
                    const float* w = W + v * d;
                    for (int64_t j = 0; j < d; j++) gh[j] += gv * (double)w[j];
                }
            }
        }
        free(a); free(G); free(p); free(lp);
    }
    if (bad & 2) return -2;
    if (bad & 1) return -1;
    if (bad & 4) return -3;
    return 0;
}

int kdo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
