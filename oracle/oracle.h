/*
 * CPU oracle of the MoE layer forward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow fp64 C.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product library never does.  It shares no
 * code, header or table with the HIP path.
 *
 * Sources (web pages on Mixture-of-Experts layers):
 *   [NOTES]  "MoE notes: what one token goes through in an MoE layer"
 *            (www.cf-1.com/news/5905749), sections 1.2, 2, 2.1-2.3, 3.1.
 *   [ENG]    "MoE 大模型推理工程深度实践：专家路由、负载均衡与分布式部署"
 *            (ybb.press/quantum-computing/18594), sections 1 and 1.2.
 *
 * Element types: ORACLE_F32 arrays are float, ORACLE_BF16 arrays are the
 * uint16 bit patterns of bfloat16 values; every value is widened exactly to
 * double before use.  All matrices are row-major.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Router scores before the softmax: L[t,e] = sum_j x[t,j] * Wr[j,e], in double.
 * x [T,d], Wr [d,E], L [T,E].  [NOTES] §1.2 (router is a linear layer) and §2
 * first step. */
void oracle_router_logits(int64_t T, int64_t d, int64_t E, int dtype,
                          const void* x, const void* w_router, double* logits);

/* Routing of fp32 logits.  l'[t,e] = fl32(logits[t,e] + bias[e]) (bias may be
 * NULL = +0), top-K by (l' descending, expert index ascending), softmax over all
 * E experts in double, renormalised over the K chosen.  Outputs: ids [T,K]
 * (int32), w [T,K] (double), probs [T,E] (double, may be NULL). */
void oracle_route(int64_t T, int64_t E, int64_t K, const float* logits,
                  const float* bias, int32_t* ids, double* w, double* probs);

/* Grouping of the (token, slot) assignments per expert, by definition.
 * counts [E], kept [E], offsets [E+1], assign_row [T*K], row_assign [T*K].
 * capacity < 0 means unlimited. */
void oracle_dispatch(int64_t T, int64_t E, int64_t K, int64_t capacity,
                     const int32_t* ids, int32_t* counts, int32_t* kept,
                     int32_t* offsets, int32_t* assign_row, int32_t* row_assign);

/* One expert applied to one token: h = W2_e (SiLU(W1_e x) * (W3_e x)).
 * x [d], w1e/w3e [F,d], w2e [d,F], h [d] (double). */
void oracle_expert(int64_t d, int64_t F, int dtype, const void* x_row,
                   const void* w1e, const void* w3e, const void* w2e, double* h);

/* Layer output for a list of tokens: y[t] = sum over kept slots k (ascending)
 * of w[t,k] * expert_{ids[t,k]}(x[t]).  x [T,d], w1/w3 [E,F,d], w2 [E,d,F],
 * ids/assign_row [T,K], w [T,K] double; tokens [n_tok]; y [n_tok, d] double. */
void oracle_layer_output(int64_t T, int64_t d, int64_t E, int64_t K, int64_t F,
                         int dtype, const void* x, const void* w1, const void* w3,
                         const void* w2, const int32_t* ids, const double* w,
                         const int32_t* assign_row, int64_t n_tok,
                         const int64_t* tokens, double* y);

/* Load-balancing auxiliary loss  aux = E * sum_e f_e * P_e  with
 * f_e = counts[e] / (T*K) and P_e = mean over tokens of probs[t,e]. */
double oracle_aux_loss(int64_t T, int64_t E, int64_t K, const int32_t* counts,
                       const double* probs);

/* One step of the per-expert bias adjustment, in float arithmetic:
 * counts[e]*E > T*K -> bias[e] -= alpha ; counts[e]*E < T*K -> bias[e] += alpha. */
void oracle_bias_update(int64_t T, int64_t E, int64_t K, const int32_t* counts,
                        float alpha, float* bias);

/* Router z-loss ([NOTES] §3.2): (1/T) sum_t (log sum_e exp(logits[t,e]))^2,
 * over the router scores before any per-expert bias.  logits [T,E] fp32. */
double oracle_z_loss(int64_t T, int64_t E, const float* logits);

/* The cheaper auxiliary loss of [NOTES] §3.2 that counts only the
 * probabilities of the K chosen experts: E * sum_e f_e * P'_e with
 * f_e = counts[e] / (T*K) and P'_e = (1/T) sum_t sum_k [ids[t,k] == e] probs[t,e]
 * (probs: the routing softmax over all E, bias included). */
double oracle_aux_topk(int64_t T, int64_t E, int64_t K, const int32_t* counts,
                       const int32_t* ids, const double* probs);

/* Number of OpenMP threads the oracle runs with. */
int oracle_num_threads(void);

/* Concatenation combine ([NOTES] §2.3): y[t] = Wc . concat_k h[assign_row[t,k]]
 * (slot order; a dropped slot is a zero block).  h [S,d], Wc [d_out, K*d]
 * (out-features-major, like a linear layer's weight), assign_row [T,K],
 * y [T, d_out] double. */
void oracle_combine_concat(int64_t T, int64_t K, int64_t d, int64_t d_out, int dtype,
                           const void* h, const int32_t* assign_row, const void* w_cat, double* y);

#endif
