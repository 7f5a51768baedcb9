/*
 * strata_oracle.c -- TEST INFRASTRUCTURE, not part of the product.
 *
 * The plain fp64 definition of one routed-expert MoE layer, written as
 * directly as the pages state it.  Only tests/, __graft_entry__.smoke() and
 * the cpu_baseline leg of bench.py may load this library; the HIP library
 * never links or calls it.  No blocking, fusion or reordering beyond what the
 * definitions below state; OpenMP only splits independent rows.
 *
 * Readings of points the pages leave open:
 *  - block field order: fp16 scale in bytes 0-1, then 16 code bytes;
 *  - matrix order in a blob: gate, up, down; each blocked along its input
 *    dimension: gate/up are [FF][H], down is [H][FF], row-major;
 *  - expert function: SwiGLU, h = silu(g) * u;
 *  - top-k ties: stable, lower expert id first; the ranking key is the
 *    probability rounded to fp32 (the precision the GPU kernel decides in);
 *  - renormalisation clamp: the caller passes it (2^-14 in the tests).
 */
#include "strata_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* "Strata in the source...", section "The byte budget, in code":
 * BLOB = 3 * (H * FF * BB / QK), three matrices of H x FF weights. */
size_t orc_blob_bytes(int H, int FF)
{
    if (H <= 0 || FF <= 0 || H % ORC_QK || FF % ORC_QK)
        return 0;
    return 3u * ((size_t)H * (size_t)FF * ORC_BB / ORC_QK);
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits. */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), ex - 25); /* 1.man * 2^(ex-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits. */
double orc_bf16_to_double(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int ex = (b >> 7) & 0xff;
    int man = b & 0x7f;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -133); /* subnormal: man * 2^-126 * 2^-7 */
    else if (ex == 255)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + man), ex - 134); /* 1.man * 2^(ex-127) */
    return sign ? -v : v;
}

/* "Strata in the source...", section "The CPU kernels": the AVX-512 unpack
 * reads the 16 code bytes as eight little-endian u16, and within each the
 * multishift control 0,2,4,...,14 with mask 3 yields 8 codes.  So code i sits
 * at bits 2i..2i+1 of the little-endian 128-bit code field: byte i/4,
 * shift 2*(i%4).  The code field follows the 2-byte scale. */
int orc_q2_code(const uint8_t *block, int i)
{
    return (block[2 + i / 4] >> (2 * (i % 4))) & 3;
}

/* Same section: codes {0,1,2,3} mean {-1,0,1,2} x scale. */
double orc_q2_value(const uint8_t *block, int i)
{
    uint16_t hbits = (uint16_t)(block[0] | ((uint16_t)block[1] << 8));
    double d = orc_half_to_double(hbits);
    return (double)(orc_q2_code(block, i) - 1) * d;
}

int orc_decode_matrix(const uint8_t *mat, int rows, int cols, double *w)
{
    if (!mat || !w || rows <= 0 || cols <= 0 || cols % ORC_QK)
        return -1;
    int nb = cols / ORC_QK;
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < nb; ++b) {
            const uint8_t *blk = mat + ((size_t)r * nb + b) * ORC_BB;
            for (int i = 0; i < ORC_QK; ++i)
                w[(size_t)r * cols + (size_t)b * ORC_QK + i] = orc_q2_value(blk, i);
        }
    return 0;
}

int orc_rmsnorm(const double *x, int n, double eps, double *xhat)
{
    if (!x || !xhat || n <= 0)
        return -1;
    double ss = 0.0;
    for (int i = 0; i < n; ++i)
        ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / n + eps);
    for (int i = 0; i < n; ++i)
        xhat[i] = x[i] * inv;
    return 0;
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* zwxr.cn page, routing journey: a BF16 GEMV projects the activation onto the
 * 512-wide routing space.  Each bf16 x value product is exact in fp64. */
int orc_router_logits(const double *xhat, const uint16_t *R, const float *bias,
                      int E, int H, double *logits)
{
    if (!xhat || !R || !logits || E <= 0 || H <= 0)
        return -1;
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int k = 0; k < H; ++k)
            acc += orc_bf16_to_double(R[(size_t)e * H + k]) * xhat[k];
        if (bias)
            acc += (double)bias[e];
        logits[e] = acc;
    }
    return 0;
}

/* zwxr.cn page, routing journey: softmax over all experts, stable descending
 * argsort, gather the first K, renormalise with a lower clamp. */
int orc_softmax_topk(const double *logits, int E, int K, double clamp,
                     int32_t *ids, double *w, double *probs)
{
    if (!logits || !ids || !w || E <= 0 || K <= 0 || K > E)
        return -1;
    double *p = (double *)malloc(sizeof(double) * E);
    int *order = (int *)malloc(sizeof(int) * E);
    if (!p || !order) {
        free(p);
        free(order);
        return -2;
    }
    double m = logits[0];
    for (int e = 1; e < E; ++e)
        if (logits[e] > m)
            m = logits[e];
    double s = 0.0;
    for (int e = 0; e < E; ++e) {
        p[e] = exp(logits[e] - m);
        s += p[e];
    }
    for (int e = 0; e < E; ++e)
        p[e] /= s;
    /* Stable insertion sort, descending on the fp32-rounded probability:
     * an element moves left only past strictly smaller keys, so equal keys
     * keep ascending expert-id order. */
    for (int e = 0; e < E; ++e) {
        float key = (float)p[e];
        int j = e;
        while (j > 0 && (float)p[order[j - 1]] < key) {
            order[j] = order[j - 1];
            --j;
        }
        order[j] = e;
    }
    double sel = 0.0;
    for (int k = 0; k < K; ++k) {
        ids[k] = order[k];
        sel += p[order[k]];
    }
    double den = sel > clamp ? sel : clamp;
    for (int k = 0; k < K; ++k)
        w[k] = p[ids[k]] / den;
    if (probs)
        memcpy(probs, p, sizeof(double) * E);
    free(p);
    free(order);
    return 0;
}

/* Dot of row r of a Q2_0 matrix with n inputs (n % 64 == 0), decoding weight
 * by weight. */
static double q2_row_dot(const uint8_t *mat, int r, int n, const double *v)
{
    int nb = n / ORC_QK;
    double acc = 0.0;
    for (int b = 0; b < nb; ++b) {
        const uint8_t *blk = mat + ((size_t)r * nb + b) * ORC_BB;
        /* the block's scale, decoded once; weight i is (code_i - 1) * d */
        double d = orc_half_to_double((uint16_t)(blk[0] | ((uint16_t)blk[1] << 8)));
        for (int i = 0; i < ORC_QK; ++i)
            acc += (double)(orc_q2_code(blk, i) - 1) * d * v[b * ORC_QK + i];
    }
    return acc;
}

/* One SwiGLU expert: gate, up and down stored in that order in the blob
 * ("The byte budget, in code"), each blocked along its input dimension. */
int orc_expert(const uint8_t *blob, const double *xhat, int H, int FF, double *o)
{
    if (!blob || !xhat || !o || orc_blob_bytes(H, FF) == 0)
        return -1;
    size_t mat_bytes = (size_t)H * FF / ORC_QK * ORC_BB;
    const uint8_t *gate = blob;
    const uint8_t *up = blob + mat_bytes;
    const uint8_t *down = blob + 2 * mat_bytes;
    double *h = (double *)malloc(sizeof(double) * FF);
    if (!h)
        return -2;
#pragma omp parallel for schedule(static)
    for (int j = 0; j < FF; ++j) {
        double g = q2_row_dot(gate, j, H, xhat);
        double u = q2_row_dot(up, j, H, xhat);
        h[j] = orc_silu(g) * u;
    }
#pragma omp parallel for schedule(static)
    for (int r = 0; r < H; ++r)
        o[r] = q2_row_dot(down, r, FF, h);
    free(h);
    return 0;
}

int orc_route(int T, int E, int H, int K, const float *x, int rmsnorm, double eps,
              const uint16_t *R, const float *bias, double clamp, int32_t *ids,
              double *w, double *xhat_out)
{
    if (T <= 0 || E <= 0 || H <= 0 || K <= 0 || K > E || !x || !R || !ids || !w ||
        !xhat_out)
        return -1;
    double *logits = (double *)malloc(sizeof(double) * (size_t)T * E);
    if (!logits)
        return -2;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int t = 0; t < T; ++t) {
        double *xh = xhat_out + (size_t)t * H;
        for (int k = 0; k < H; ++k)
            xh[k] = (double)x[(size_t)t * H + k];
        if (rmsnorm)
            bad |= orc_rmsnorm(xh, H, eps, xh) != 0;
        bad |= orc_router_logits(xh, R, bias, E, H, logits + (size_t)t * E) != 0;
        bad |= orc_softmax_topk(logits + (size_t)t * E, E, K, clamp, ids + (size_t)t * K,
                                w + (size_t)t * K, NULL) != 0;
    }
    free(logits);
    return bad ? -3 : 0;
}

int orc_experts(int T, int E, int H, int FF, int K, const double *xhat,
                const int32_t *ids, const uint8_t *const *blobs, double *o)
{
    if (T <= 0 || E <= 0 || K <= 0 || !xhat || !ids || !blobs || !o)
        return -1;
    for (int s = 0; s < T * K; ++s) {
        int e = ids[s];
        if (e < 0 || e >= E || !blobs[e])
            return -4;
        int rc = orc_expert(blobs[e], xhat + (size_t)(s / K) * H, H, FF, o + (size_t)s * H);
        if (rc)
            return rc;
    }
    return 0;
}

/* zwxr.cn page, routing journey (Combine): the layer output is the routing-
 * weighted sum of the selected experts' outputs. */
int orc_combine(int T, int H, int K, const double *o, const double *w, double *y)
{
    if (T <= 0 || H <= 0 || K <= 0 || !o || !w || !y)
        return -1;
    for (int t = 0; t < T; ++t)
        for (int r = 0; r < H; ++r) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += w[(size_t)t * K + k] * o[((size_t)t * K + k) * H + r];
            y[(size_t)t * H + r] = acc;
        }
    return 0;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
