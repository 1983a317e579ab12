/*
 * CPU oracle of the MoE layer forward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 restatement of what the pages define.  Nothing here is
 * blocked, fused or reordered beyond what the definitions state.  Page
 * references ([NOTES], [ENG]) are spelled out in oracle.h.
 *
 * Readings taken where the pages are silent or loose:
 *  - the top-K ranks the (biased) fp32 logits, which orders experts exactly as
 *    the softmax scores do (the softmax is monotone); ties go to the lower
 *    expert index, and -0 compares equal to +0;
 *  - "renormalise the K scores" is p_k / sum of the K chosen p, which equals
 *    the softmax over the K chosen logits used in [ENG] §1;
 *  - the per-expert bias is added to the logits before both the selection and
 *    the softmax ([ENG] §1.2, "logits = gate(x) + bias");
 *  - the expert FFN is SwiGLU, h = W2 (SiLU(W1 x) * W3 x); the pages only say
 *    each expert is an FFN, so this form is not pinned by them;
 *  - under a capacity C, the assignments of an expert are kept in flat order
 *    t*K + k (token order, then slot) and the ones of rank >= C are dropped;
 *    the weights of survivors are not renormalised.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double value_at(const void* p, int dtype, int64_t i) {
    if (dtype == ORACLE_F32) return (double)((const float*)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static size_t elem_size(int dtype) { return dtype == ORACLE_F32 ? 4 : 2; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* [NOTES] §1.2 and §2 (first step): the router is a linear map from the
 * token's hidden vector to one score per expert. */
void oracle_router_logits(int64_t T, int64_t d, int64_t E, int dtype,
                          const void* x, const void* w_router, double* logits) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            double s = 0.0;
            for (int64_t j = 0; j < d; ++j)
                s += value_at(x, dtype, t * d + j) * value_at(w_router, dtype, j * E + e);
            logits[t * E + e] = s;
        }
    }
}

/* [NOTES] §2 steps 1-3 and §2.1; [ENG] §1 and §1.2.
 * Step 1: scores s = softmax over all E experts ([NOTES] §1.2 says the softmax
 *         runs over every expert).
 * Step 2: the K highest-scoring experts.
 * Step 3: their K scores renormalised so that they sum to one. */
void oracle_route(int64_t T, int64_t E, int64_t K, const float* logits,
                  const float* bias, int32_t* ids, double* w, double* probs) {
#pragma omp parallel
    {
        float* lp = (float*)malloc((size_t)E * sizeof(float));
        double* p = (double*)malloc((size_t)E * sizeof(double));
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            /* biased logits: one fp32 addition per expert ([ENG] §1.2) */
            for (int64_t e = 0; e < E; ++e) {
                float b = bias ? bias[e] : 0.0f;
                lp[e] = logits[t * E + e] + b;
            }
            /* softmax over all E, in double */
            double m = lp[0];
            for (int64_t e = 1; e < E; ++e)
                if (lp[e] > m) m = lp[e];
            double z = 0.0;
            for (int64_t e = 0; e < E; ++e) {
                p[e] = exp((double)lp[e] - m);
                z += p[e];
            }
            for (int64_t e = 0; e < E; ++e) p[e] /= z;
            if (probs)
                for (int64_t e = 0; e < E; ++e) probs[t * E + e] = p[e];
            /* top-K: K rounds, each taking the largest remaining logit; scanning
             * experts in ascending order and replacing only on a strictly larger
             * value leaves the lower index in front on ties */
            memset(taken, 0, (size_t)E);
            for (int64_t k = 0; k < K; ++k) {
                int64_t best = -1;
                for (int64_t e = 0; e < E; ++e) {
                    if (taken[e]) continue;
                    if (best < 0 || lp[e] > lp[best]) best = e;
                }
                taken[best] = 1;
                ids[t * K + k] = (int32_t)best;
            }
            /* renormalisation over the K chosen scores */
            double sel = 0.0;
            for (int64_t k = 0; k < K; ++k) sel += p[ids[t * K + k]];
            for (int64_t k = 0; k < K; ++k) w[t * K + k] = p[ids[t * K + k]] / sel;
        }
        free(lp);
        free(p);
        free(taken);
    }
}

/* [NOTES] §2.1 (regroup tokens so that those bound for one expert are
 * adjacent: a sort plus a cumulative sum) and §3.1 (average T*K/E tokens per
 * expert; a capacity cap truncates the overflow).
 * The rank of assignment i = t*K + k is the number of earlier assignments
 * (smaller flat index) that chose the same expert; a running per-expert count
 * taken in flat order is exactly that number. */
void oracle_dispatch(int64_t T, int64_t E, int64_t K, int64_t capacity,
                     const int32_t* ids, int32_t* counts, int32_t* kept,
                     int32_t* offsets, int32_t* assign_row, int32_t* row_assign) {
    int64_t n = T * K;
    int32_t* rank = (int32_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = ids[i];
        rank[i] = counts[e];
        counts[e] += 1;
    }
    for (int64_t e = 0; e < E; ++e)
        kept[e] = (capacity < 0 || counts[e] < capacity) ? counts[e] : (int32_t)capacity;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + kept[e];
    for (int64_t r = 0; r < n; ++r) row_assign[r] = -1;
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = ids[i];
        if (capacity < 0 || rank[i] < capacity) {
            assign_row[i] = offsets[e] + rank[i];
            row_assign[assign_row[i]] = (int32_t)i;
        } else {
            assign_row[i] = -1;
        }
    }
    free(rank);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* [NOTES] §2 third step: every expert is a feed-forward network applied to
 * the token vector; here the SwiGLU form h = W2 (SiLU(W1 x) * (W3 x)). */
void oracle_expert(int64_t d, int64_t F, int dtype, const void* x_row,
                   const void* w1e, const void* w3e, const void* w2e, double* h) {
    double* a = (double*)malloc((size_t)F * sizeof(double));
    for (int64_t f = 0; f < F; ++f) {
        double g1 = 0.0, g3 = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            double xj = value_at(x_row, dtype, j);
            g1 += value_at(w1e, dtype, f * d + j) * xj;
            g3 += value_at(w3e, dtype, f * d + j) * xj;
        }
        a[f] = silu(g1) * g3;
    }
    for (int64_t i = 0; i < d; ++i) {
        double s = 0.0;
        for (int64_t f = 0; f < F; ++f) s += value_at(w2e, dtype, i * F + f) * a[f];
        h[i] = s;
    }
    free(a);
}

/* [NOTES] §2 fourth step and §2.3: y = sum_j w_j h_j over the chosen experts;
 * [NOTES] §2.2: an expert that was not chosen contributes exactly nothing, so
 * only the chosen (and, under a capacity, kept) experts are evaluated. */
void oracle_layer_output(int64_t T, int64_t d, int64_t E, int64_t K, int64_t F,
                         int dtype, const void* x, const void* w1, const void* w3,
                         const void* w2, const int32_t* ids, const double* w,
                         const int32_t* assign_row, int64_t n_tok,
                         const int64_t* tokens, double* y) {
    (void)T;
    (void)E;
    const size_t es = elem_size(dtype);
    const char* xb = (const char*)x;
    const char* w1b = (const char*)w1;
    const char* w3b = (const char*)w3;
    const char* w2b = (const char*)w2;
#pragma omp parallel
    {
        double* h = (double*)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t s = 0; s < n_tok; ++s) {
            int64_t t = tokens[s];
            double* yt = y + s * d;
            for (int64_t i = 0; i < d; ++i) yt[i] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                if (assign_row && assign_row[t * K + k] < 0) continue; /* dropped */
                int64_t e = ids[t * K + k];
                oracle_expert(d, F, dtype, xb + (size_t)(t * d) * es,
                              w1b + (size_t)(e * F * d) * es, w3b + (size_t)(e * F * d) * es,
                              w2b + (size_t)(e * d * F) * es, h);
                for (int64_t i = 0; i < d; ++i) yt[i] += w[t * K + k] * h[i];
            }
        }
        free(h);
    }
}

/* [NOTES] §1.2: aux_loss = N * sum_i f_i * P_i, f_i the fraction of routing
 * choices that went to expert i, P_i the router's mean probability for it.
 * f_i counts the K choices of every token before any capacity drop. */
double oracle_aux_loss(int64_t T, int64_t E, int64_t K, const int32_t* counts,
                       const double* probs) {
    double total = 0.0;
    for (int64_t e = 0; e < E; ++e) {
        double f = (double)counts[e] / (double)(T * K);
        double P = 0.0;
        for (int64_t t = 0; t < T; ++t) P += probs[t * E + e];
        P /= (double)T;
        total += f * P;
    }
    return (double)E * total;
}

/* [ENG] §1.2: an overloaded expert's bias drops by alpha, an underloaded one's
 * rises by alpha; the target load is the average T*K/E of [NOTES] §3.1,
 * compared in integers as counts*E against T*K. */
void oracle_bias_update(int64_t T, int64_t E, int64_t K, const int32_t* counts,
                        float alpha, float* bias) {
    for (int64_t e = 0; e < E; ++e) {
        int64_t load = (int64_t)counts[e] * E;
        if (load > T * K)
            bias[e] = bias[e] - alpha;
        else if (load < T * K)
            bias[e] = bias[e] + alpha;
    }
}

/* [NOTES] §3.2: the z-loss squares each token's log-sum-exp of the router
 * scores (it keeps the scores from growing); the scores are the router's own
 * output, before the per-expert balancing bias of [ENG] §1.2. */
double oracle_z_loss(int64_t T, int64_t E, const float* logits) {
    double total = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        double m = logits[t * E];
        for (int64_t e = 1; e < E; ++e)
            if (logits[t * E + e] > m) m = logits[t * E + e];
        double s = 0.0;
        for (int64_t e = 0; e < E; ++e) s += exp((double)logits[t * E + e] - m);
        double lse = m + log(s);
        total += lse * lse;
    }
    return total / (double)T;
}

/* [NOTES] §3.2: the approximate aux loss keeps only the probabilities of the
 * experts each token selected (the soft assignment to the other experts is
 * not counted). */
double oracle_aux_topk(int64_t T, int64_t E, int64_t K, const int32_t* counts,
                       const int32_t* ids, const double* probs) {
    double sum_fp = 0.0;
    for (int64_t e = 0; e < E; ++e) {
        const double frac = (double)counts[e] / ((double)T * (double)K);
        double chosen = 0.0; /* probability mass of e over the tokens that chose e */
        for (int64_t t = 0; t < T; ++t)
            for (int64_t k = 0; k < K; ++k)
                if (ids[t * K + k] == e) chosen += probs[t * E + e];
        sum_fp += frac * (chosen / (double)T);
    }
    return sum_fp * (double)E;
}

/* [NOTES] §2.3, the combine that concatenates the K expert outputs of a token
 * in slot order and applies one linear layer to the concatenation:
 *   y[t, o] = sum over slots k, features i of  h[assign_row[t,k], i] * Wc[o, k*d + i].
 * A slot dropped by capacity (assign_row < 0) contributes a zero block. */
void oracle_combine_concat(int64_t T, int64_t K, int64_t d, int64_t d_out, int dtype,
                           const void* h, const int32_t* assign_row, const void* w_cat, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t o = 0; o < d_out; ++o) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int32_t row = assign_row[t * K + k];
                if (row < 0) continue; /* dropped slot: a block of zeros */
                for (int64_t i = 0; i < d; ++i)
                    acc += value_at(h, dtype, (int64_t)row * d + i) * value_at(w_cat, dtype, o * K * d + k * d + i);
            }
            y[t * d_out + o] = acc;
        }
    }
}
