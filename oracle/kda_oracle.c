/*
 * kda_oracle.c -- fp64 CPU oracle for KDA (Kimi Delta Attention) prefill.
 *
 * TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
 * CPU-baseline leg are the only callers. The GPU library never links or calls it,
 * and this file shares no code, header or constant with it.
 *
 * What is computed. KDA keeps one fixed-size recurrent state per head that every
 * new token updates instead of appending to a growing key/value cache
 * (akiraxclaw.com "Kimi K3 開源基礎設施：三個專案怎麼分工？", section
 * "FlashKDA：先把 KDA kernel 跑快"; augursoft.site "Kimi K3 的三個系統設計",
 * section "第一個設計"). The update of that K x V state S for token t is a
 * per-key-channel decay followed by a delta-rule write, and the output reads the
 * state after the write:
 *
 *     S <- Diag(exp(g_t)) S                        (decay, natural-log gate)
 *     S <- S + beta_t k_t (v_t - S^T k_t)^T        (= (I - beta_t k_t k_t^T) S + beta_t k_t v_t^T)
 *     o_t = S^T q_t
 *
 * This file writes that out token by token in double precision, with no
 * chunking, blocking or reordering. Inputs are fp32 arrays holding exactly the
 * values the GPU receives (bf16 inputs are passed as their exact fp32 values).
 *
 * Layouts (row-major, contiguous): q, k, g [T, H, K]; v [T, H, V]; beta [T, H];
 * cu_seqlens int64 [N+1] with cu_seqlens[0] = 0 and cu_seqlens[N] = T;
 * initial_state [N, H, K, V] (NULL means zero).
 * Only the heads listed in heads[0..n_heads) are evaluated; the outputs are laid
 * out for that subset: out [T, n_heads, V], final_state [N, n_heads, K, V]
 * (either may be NULL).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static int run_pair(const float *q, const float *k, const float *v, const float *g,
                    const float *beta, int64_t t_begin, int64_t t_end, int64_t H,
                    int64_t K, int64_t V, int64_t h, const float *s0, double *out,
                    int64_t out_stride_t, double *final_state)
{
    double *S = (double *)malloc((size_t)(K * V) * sizeof(double));
    double *pred = (double *)malloc((size_t)V * sizeof(double));
    double *delta = (double *)malloc((size_t)V * sizeof(double));
    double *acc = (double *)malloc((size_t)V * sizeof(double));
    if (!S || !pred || !delta || !acc) {
        free(S); free(pred); free(delta); free(acc);
        return -2;
    }
    for (int64_t i = 0; i < K * V; ++i)
        S[i] = s0 ? (double)s0[i] : 0.0;

    for (int64_t t = t_begin; t < t_end; ++t) {
        const float *qt = q + (t * H + h) * K;
        const float *kt = k + (t * H + h) * K;
        const float *vt = v + (t * H + h) * V;
        const float *gt = g + (t * H + h) * K;
        const double bt = (double)beta[t * H + h];

        /* [decay] row c of S is multiplied by alpha = exp(g_t[c]) */
        for (int64_t c = 0; c < K; ++c) {
            const double alpha = exp((double)gt[c]);
            for (int64_t j = 0; j < V; ++j)
                S[c * V + j] *= alpha;
        }
        /* [/decay] */

        /* [predict] pred = S^T k_t on the decayed state */
        for (int64_t j = 0; j < V; ++j)
            pred[j] = 0.0;
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                pred[j] += (double)kt[c] * S[c * V + j];
        /* [/predict] */

        /* [write] S += k_t delta^T with delta = beta_t (v_t - pred) */
        for (int64_t j = 0; j < V; ++j)
            delta[j] = bt * ((double)vt[j] - pred[j]);
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                S[c * V + j] += (double)kt[c] * delta[j];
        /* [/write] */

        /* [output] o_t = S^T q_t on the state after the write */
        for (int64_t j = 0; j < V; ++j)
            acc[j] = 0.0;
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                acc[j] += (double)qt[c] * S[c * V + j];
        if (out)
            for (int64_t j = 0; j < V; ++j)
                out[t * out_stride_t + j] = acc[j];
        /* [/output] */
    }

    if (final_state)
        memcpy(final_state, S, (size_t)(K * V) * sizeof(double));
    free(S); free(pred); free(delta); free(acc);
    return 0;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int kda_oracle_prefill(const float *q, const float *k, const float *v, const float *g,
                       const float *beta, const int64_t *cu_seqlens, int64_t num_seqs,
                       int64_t total_tokens, int64_t H, int64_t K, int64_t V,
                       const float *initial_state, const int64_t *heads, int64_t n_heads,
                       double *out, double *final_state, int num_threads)
{
    if (!q || !k || !v || !g || !beta || !cu_seqlens || !heads)
        return -1;
    if (num_seqs < 1 || total_tokens < 0 || H < 1 || K < 1 || V < 1 || n_heads < 0)
        return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != total_tokens)
        return -1;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return -1;
    for (int64_t i = 0; i < n_heads; ++i)
        if (heads[i] < 0 || heads[i] >= H)
            return -1;

    const int64_t pairs = num_seqs * n_heads;
    int status = 0;
#ifdef _OPENMP
    if (num_threads > 0)
        omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t n = p / n_heads, i = p % n_heads, h = heads[i];
        const float *s0 = initial_state ? initial_state + (n * H + h) * K * V : NULL;
        double *o = out ? out + i * V : NULL;
        double *fs = final_state ? final_state + (n * n_heads + i) * K * V : NULL;
        int rc = run_pair(q, k, v, g, beta, cu_seqlens[n], cu_seqlens[n + 1], H, K, V, h,
                          s0, o, n_heads * V, fs);
        if (rc != 0) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = rc;
        }
    }
    return status;
}

/*
 * Backward (reverse mode) of the same recurrence, token by token in double
 * precision. The pages describe only the forward prefill; the gradients here are
 * the plain derivatives of the recurrence above for the loss
 *     L = sum_t <dO_t, o_t> + <dS_T, S_T>
 * with dO (and dS_T, the gradient reaching the final state; NULL means zero)
 * given. Going back over token t with dS the gradient w.r.t. S_t:
 *     Sd = Diag(alpha_t) S_{t-1},  pred = Sd^T k_t,  delta = beta_t (v_t - pred),
 *     dS += q_t dO_t^T,        dq_t = S_t dO_t,
 *     ddelta = dS^T k_t,       dk_t = dS delta + Sd dpred,
 *     dbeta_t = ddelta . (v_t - pred),  dv_t = beta_t ddelta,  dpred = -beta_t ddelta,
 *     dSd = dS + k_t dpred^T,  dg_t[c] = sum_j dSd[c,j] Sd[c,j],
 *     dS_{t-1} = Diag(alpha_t) dSd.
 * The states S_{t-1} are recomputed from checkpoints kept every CKPT tokens by
 * the same forward step, operation for operation, so they are bitwise the
 * states of a single forward pass.
 *
 * Layouts: as the forward, plus d_out [T, H, V], d_final_state [N, H, K, V]
 * (NULL = zero); outputs for the heads subset: dq, dk, dg [T, n_heads, K],
 * dv [T, n_heads, V], dbeta [T, n_heads], d_initial_state [N, n_heads, K, V]
 * (d_initial_state may be NULL).
 */
#define CKPT 64

/* One forward step: S holds S_{t-1} on entry and S_t on return; Sd gets the
 * decayed state, pred and delta the step's prediction and write. */
static void forward_step(double *S, double *Sd, double *pred, double *delta, const float *kt,
                         const float *vt, const float *gt, double bt, int64_t K, int64_t V)
{
    for (int64_t c = 0; c < K; ++c) {
        const double alpha = exp((double)gt[c]);
        for (int64_t j = 0; j < V; ++j)
            Sd[c * V + j] = alpha * S[c * V + j];
    }
    for (int64_t j = 0; j < V; ++j)
        pred[j] = 0.0;
    for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j)
            pred[j] += (double)kt[c] * Sd[c * V + j];
    for (int64_t j = 0; j < V; ++j)
        delta[j] = bt * ((double)vt[j] - pred[j]);
    for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j)
            S[c * V + j] = Sd[c * V + j] + (double)kt[c] * delta[j];
}

static int run_pair_backward(const float *q, const float *k, const float *v, const float *g,
                             const float *beta, const float *dout, int64_t t_begin,
                             int64_t t_end, int64_t H, int64_t K, int64_t V, int64_t h,
                             const float *s0, const float *dsT, int64_t n_heads,
                             double *dq, double *dk, double *dv, double *dg, double *dbeta,
                             double *ds0)
{
    const int64_t L = t_end - t_begin;
    const int64_t nck = (L + CKPT - 1) / CKPT;
    const size_t KV = (size_t)(K * V);
    double *ck = (double *)malloc((nck > 0 ? nck : 1) * KV * sizeof(double));
    double *blk = (double *)malloc((CKPT + 1) * KV * sizeof(double));
    double *S = (double *)malloc(KV * sizeof(double));
    double *Sd = (double *)malloc(KV * sizeof(double));
    double *dS = (double *)malloc(KV * sizeof(double));
    double *pred = (double *)malloc((size_t)V * sizeof(double));
    double *delta = (double *)malloc((size_t)V * sizeof(double));
    double *ddelta = (double *)malloc((size_t)V * sizeof(double));
    double *dpred = (double *)malloc((size_t)V * sizeof(double));
    if (!ck || !blk || !S || !Sd || !dS || !pred || !delta || !ddelta || !dpred) {
        free(ck); free(blk); free(S); free(Sd); free(dS); free(pred); free(delta); free(ddelta); free(dpred);
        return -2;
    }

    /* forward once, keeping the state at the start of every CKPT-token block */
    for (size_t i = 0; i < KV; ++i)
        S[i] = s0 ? (double)s0[i] : 0.0;
    for (int64_t t = t_begin; t < t_end; ++t) {
        if ((t - t_begin) % CKPT == 0)
            memcpy(ck + ((t - t_begin) / CKPT) * KV, S, KV * sizeof(double));
        forward_step(S, Sd, pred, delta, k + (t * H + h) * K, v + (t * H + h) * V,
                     g + (t * H + h) * K, (double)beta[t * H + h], K, V);
    }

    for (size_t i = 0; i < KV; ++i)
        dS[i] = dsT ? (double)dsT[i] : 0.0;

    for (int64_t b = nck - 1; b >= 0; --b) {
        const int64_t b0 = t_begin + b * CKPT;
        const int64_t b1 = (b0 + CKPT < t_end) ? b0 + CKPT : t_end;
        /* blk[i] = S_{b0 + i - 1}, the state before token b0 + i; blk[b1 - b0] = after the block */
        memcpy(blk, ck + b * KV, KV * sizeof(double));
        for (int64_t t = b0; t < b1; ++t) {
            memcpy(blk + (t - b0 + 1) * KV, blk + (t - b0) * KV, KV * sizeof(double));
            forward_step(blk + (t - b0 + 1) * KV, Sd, pred, delta, k + (t * H + h) * K,
                         v + (t * H + h) * V, g + (t * H + h) * K, (double)beta[t * H + h], K, V);
        }
        for (int64_t t = b1 - 1; t >= b0; --t) {
            const float *qt = q + (t * H + h) * K;
            const float *kt = k + (t * H + h) * K;
            const float *vt = v + (t * H + h) * V;
            const float *gt = g + (t * H + h) * K;
            const float *dot = dout + (t * H + h) * V;
            const double bt = (double)beta[t * H + h];
            const double *Sprev = blk + (t - b0) * KV;
            const double *Snew = blk + (t - b0 + 1) * KV;
            const int64_t row = t * n_heads;
            double *dq_t = dq + row * K, *dk_t = dk + row * K, *dg_t = dg + row * K;
            double *dv_t = dv + row * V;

            /* recompute the step's decayed state, prediction and write */
            for (int64_t c = 0; c < K; ++c) {
                const double alpha = exp((double)gt[c]);
                for (int64_t j = 0; j < V; ++j)
                    Sd[c * V + j] = alpha * Sprev[c * V + j];
            }
            for (int64_t j = 0; j < V; ++j)
                pred[j] = 0.0;
            for (int64_t c = 0; c < K; ++c)
                for (int64_t j = 0; j < V; ++j)
                    pred[j] += (double)kt[c] * Sd[c * V + j];
            for (int64_t j = 0; j < V; ++j)
                delta[j] = bt * ((double)vt[j] - pred[j]);

            /* [b_output] o_t = S_t^T q_t */
            for (int64_t c = 0; c < K; ++c)
                for (int64_t j = 0; j < V; ++j)
                    dS[c * V + j] += (double)qt[c] * (double)dot[j];
            for (int64_t c = 0; c < K; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < V; ++j)
                    acc += Snew[c * V + j] * (double)dot[j];
                dq_t[c] = acc;
            }
            /* [/b_output] */

            /* [b_write] S_t = Sd + k_t delta^T */
            for (int64_t j = 0; j < V; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < K; ++c)
                    acc += dS[c * V + j] * (double)kt[c];
                ddelta[j] = acc;
            }
            for (int64_t c = 0; c < K; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < V; ++j)
                    acc += dS[c * V + j] * delta[j];
                dk_t[c] = acc;
            }
            /* [/b_write] */

            /* [b_delta] delta = beta_t (v_t - pred) */
            {
                double acc = 0.0;
                for (int64_t j = 0; j < V; ++j)
                    acc += ddelta[j] * ((double)vt[j] - pred[j]);
                dbeta[row] = acc;
            }
            for (int64_t j = 0; j < V; ++j) {
                dv_t[j] = bt * ddelta[j];
                dpred[j] = -bt * ddelta[j];
            }
            /* [/b_delta] */

            /* [b_predict] pred = Sd^T k_t */
            for (int64_t c = 0; c < K; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < V; ++j)
                    acc += Sd[c * V + j] * dpred[j];
                dk_t[c] += acc;
            }
            for (int64_t c = 0; c < K; ++c)
                for (int64_t j = 0; j < V; ++j)
                    dS[c * V + j] += (double)kt[c] * dpred[j];
            /* [/b_predict] */

            /* [b_decay] Sd = Diag(exp(g_t)) S_{t-1} */
            for (int64_t c = 0; c < K; ++c) {
                const double alpha = exp((double)gt[c]);
                double acc = 0.0;
                for (int64_t j = 0; j < V; ++j)
                    acc += dS[c * V + j] * Sd[c * V + j];
                dg_t[c] = acc;
                for (int64_t j = 0; j < V; ++j)
                    dS[c * V + j] *= alpha;
            }
            /* [/b_decay] */
        }
    }
    if (ds0)
        memcpy(ds0, dS, KV * sizeof(double));
    free(ck); free(blk); free(S); free(Sd); free(dS); free(pred); free(delta); free(ddelta); free(dpred);
    return 0;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int kda_oracle_backward(const float *q, const float *k, const float *v, const float *g,
                        const float *beta, const float *d_out, const int64_t *cu_seqlens,
                        int64_t num_seqs, int64_t total_tokens, int64_t H, int64_t K, int64_t V,
                        const float *initial_state, const float *d_final_state,
                        const int64_t *heads, int64_t n_heads, double *dq, double *dk, double *dv,
                        double *dg, double *dbeta, double *d_initial_state, int num_threads)
{
    if (!q || !k || !v || !g || !beta || !d_out || !cu_seqlens || !heads)
        return -1;
    if (!dq || !dk || !dv || !dg || !dbeta)
        return -1;
    if (num_seqs < 1 || total_tokens < 0 || H < 1 || K < 1 || V < 1 || n_heads < 0)
        return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != total_tokens)
        return -1;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return -1;
    for (int64_t i = 0; i < n_heads; ++i)
        if (heads[i] < 0 || heads[i] >= H)
            return -1;

    const int64_t pairs = num_seqs * n_heads;
    int status = 0;
#ifdef _OPENMP
    if (num_threads > 0)
        omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t n = p / n_heads, i = p % n_heads, h = heads[i];
        const size_t kv = (size_t)(K * V);
        const float *s0 = initial_state ? initial_state + (n * H + h) * kv : NULL;
        const float *dsT = d_final_state ? d_final_state + (n * H + h) * kv : NULL;
        double *ds0 = d_initial_state ? d_initial_state + (n * n_heads + i) * kv : NULL;
        int rc = run_pair_backward(q, k, v, g, beta, d_out, cu_seqlens[n], cu_seqlens[n + 1], H, K,
                                   V, h, s0, dsT, n_heads, dq + i * K, dk + i * K, dv + i * V,
                                   dg + i * K, dbeta + i, ds0);
        if (rc != 0) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = rc;
        }
    }
    return status;
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
