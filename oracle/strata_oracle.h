/*
 * strata_oracle.h -- TEST INFRASTRUCTURE, not part of the product.
 *
 * Plain, slow, fp64 CPU reference of one routed-expert MoE layer (Q2_0 SwiGLU
 * experts behind a bf16 router with softmax, stable top-k and renormalised
 * weights, then the weighted combine).  Only tests/, __graft_entry__.smoke()
 * and the cpu_baseline leg of bench.py may load it.  It shares no code, header,
 * table or helper with the HIP library; shapes are run-time parameters so the
 * same code also runs the tiny brute-force instance.
 *
 * Sources (the pages are cited by title and section):
 *  - "Strata in the source: one verify window, three workers and a cache that
 *    learns" (ai.thesatyajit.com), section "The byte budget, in code": the
 *    Q2_0 block (64 weights = 16 bytes of 2-bit codes + an fp16 scale) and the
 *    expert geometry H=2560, FF=640 for gate, up and down.
 *  - same page, section "The CPU kernels": the code -> value table
 *    {0,1,2,3} -> {-1,0,1,2} x scale and the bit order of the code field.
 *  - "MoE 遇上消费级显卡动态路由专家权重..." (zwxr.cn), the routing-journey
 *    passage (算 logits / 选 top-10 / Combine): bf16 router GEMV to 512
 *    logits, softmax over all experts, stable descending argsort, gather,
 *    renormalisation with ggml's lower clamp, and the combine sum w[i]*parts[i].
 *
 * Every function returns 0 on success, a negative value on bad arguments.
 */
#ifndef STRATA_ORACLE_H
#define STRATA_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Q2_0 block constants (page 4, "The byte budget, in code"). */
#define ORC_QK 64 /* weights per block */
#define ORC_BB 18 /* bytes per block: fp16 scale then 16 code bytes */

/* Bytes of one expert blob: gate [FF][H], up [FF][H], down [H][FF]. */
size_t orc_blob_bytes(int H, int FF);

/* IEEE binary16 and bfloat16 bit patterns -> exact double. */
double orc_half_to_double(uint16_t h);
double orc_bf16_to_double(uint16_t b);

/* Code i (0..63) of one 18-byte block, and its dequantised value. */
int orc_q2_code(const uint8_t *block, int i);
double orc_q2_value(const uint8_t *block, int i);

/* Dequantise a row-major Q2_0 matrix [rows][cols] (cols % 64 == 0). */
int orc_decode_matrix(const uint8_t *mat, int rows, int cols, double *w);

/* xhat = x / sqrt(mean(x^2) + eps) for one row of n values. */
int orc_rmsnorm(const double *x, int n, double eps, double *xhat);

/* silu(z) = z * sigmoid(z). */
double orc_silu(double z);

/* Router for one token: logits[e] = sum_k bf16(R[e][k]) * xhat[k] (+ bias[e]). */
int orc_router_logits(const double *xhat, const uint16_t *R, const float *bias,
                      int E, int H, double *logits);

/* Softmax over all E logits, stable descending top-K (ties -> lower expert
 * id first, ranked on the fp32 rounding of the probability), gather and
 * renormalise w_k = p_k / max(sum p, clamp).  probs may be NULL. */
int orc_softmax_topk(const double *logits, int E, int K, double clamp,
                     int32_t *ids, double *w, double *probs);

/* One SwiGLU expert on one token: o = W_d (silu(W_g x) * (W_u x)). */
int orc_expert(const uint8_t *blob, const double *xhat, int H, int FF, double *o);

/* Route T tokens: optional RMSNorm (rmsnorm != 0), router, softmax, top-K.
 * x is [T][H] fp32; xhat_out [T][H] receives the router/expert input. */
int orc_route(int T, int E, int H, int K, const float *x, int rmsnorm, double eps,
              const uint16_t *R, const float *bias, double clamp, int32_t *ids,
              double *w, double *xhat_out);

/* Experts for T tokens: o[(t*K+k)][H] = expert_{ids[t][k]}(xhat[t]).
 * blobs[e] points at expert e's blob; it may be NULL if e is not routed. */
int orc_experts(int T, int E, int H, int FF, int K, const double *xhat,
                const int32_t *ids, const uint8_t *const *blobs, double *o);

/* Combine: y[t] = sum_k w[t][k] * o[t*K+k] (k in routing order). */
int orc_combine(int T, int H, int K, const double *o, const double *w, double *y);

/* Threads OpenMP will use (reported as the baseline's core count). */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
