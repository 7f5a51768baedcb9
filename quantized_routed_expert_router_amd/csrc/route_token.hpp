// route_token.hpp -- one token's routing in one wave, shared by the decode
// top-k (route_decode.hip), the prefill top-k (route.hip) and the one-token
// gate/up launch (experts_decode.hip), so all of them rank alike: the fused
// 512-expert softmax, stable descending order and the first ten heads ("MoE
// 遇上消费级显卡..." (zwxr.cn), the passage following one token through a
// layer).  Device code only.
#pragma once
#include "common.hpp"

namespace strata {

// (p, e) ranks before (q, f): larger probability, or equal and lower id.
__device__ inline bool ranks_before(float p, int e, float q, int f)
{
    return p > q || (p == q && e < f);
}

// Maximum of v over the wave as signed integers, returned uniform.  For the
// bits of floats that are >= 0 or negative (a removed candidate is -1) the
// integer order is the float order, and the integer maximum needs no NaN
// canonicalisation: each step is one v_max_i32 with the DPP operand folded in.
// The block opens with a full window of 5 wait states (the DPP hazards: 2
// after a VALU write of the source, 5 after one of EXEC), as it may be reached
// by a branch whose other path it cannot see.
__device__ inline int wave_max_i(int v)
{
    asm("s_nop 4\n\t"
        "v_max_i32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_i32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_i32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_i32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_i32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_i32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
        "s_nop 1"
        : "+v"(v));
    return __builtin_amdgcn_readlane(v, 63);
}

// Denominator of the renormalised routing weights: the sum of the ten
// selected probabilities, clamped below at 2^-14 (w_k = p_k / den).
__device__ inline float renorm_den(float sel) { return fmaxf(sel, 6.103515625e-05f); }

// The lane's eight raw logits of one token (experts lane + 64 i) and, with a
// bias, its eight bias values (zero without one): loaded apart from the
// routing so that a caller can put other requests in flight between the two.
struct TokLogits {
    float l[8], b[8];
};
__device__ inline TokLogits load_logits(const float *lrow, const float *bias)
{
    const int lane = threadIdx.x & 63;
    TokLogits t;
    if (bias) {   // one uniform branch around all sixteen loads
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            t.l[i] = lrow[lane + 64 * i];
            t.b[i] = bias[lane + 64 * i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            t.l[i] = lrow[lane + 64 * i];
            t.b[i] = 0.f;
        }
    }
    return t;
}

// One token's routing in one wave from its scaled logits l (expert
// lane + 64 i in l[i], bias included): softmax over the 512, then the ten
// (p desc, id asc) heads in order.  Lane k < K gets the k-th id and its p;
// sel (uniform) is the sum of the ten p.  With kmax < K - 1 (uniform) the
// selection stops after head kmax: lanes up to kmax hold the same ids and p
// as a full routing, the others 0, and sel is incomplete.
__device__ inline void route_scaled(float l[8], int &my_id, float &my_p, float &sel,
                                    int kmax = K - 1)
{
    const int lane = threadIdx.x & 63;
    float m = l[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
        m = fmaxf(m, l[i]);
    m = wave_max63(m);
    float p[8], s = 0.f;
    int e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        p[i] = expf(l[i] - m);
        s += p[i];
        e[i] = lane + 64 * i;
    }
    s = wave_sum63(s);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        p[i] = p[i] / s;
    // sort the lane's 8 candidates, best first (19-comparator network)
#define STRATA_CX(i, j)                                                                            \
    {                                                                                              \
        const bool sw = ranks_before(p[j], e[j], p[i], e[i]);                                      \
        const float pi_ = sw ? p[j] : p[i], pj_ = sw ? p[i] : p[j];                                \
        const int ei_ = sw ? e[j] : e[i], ej_ = sw ? e[i] : e[j];                                  \
        p[i] = pi_;                                                                                \
        p[j] = pj_;                                                                                \
        e[i] = ei_;                                                                                \
        e[j] = ej_;                                                                                \
    }
    STRATA_CX(0, 2) STRATA_CX(1, 3) STRATA_CX(4, 6) STRATA_CX(5, 7)
    STRATA_CX(0, 4) STRATA_CX(1, 5) STRATA_CX(2, 6) STRATA_CX(3, 7)
    STRATA_CX(0, 1) STRATA_CX(2, 3) STRATA_CX(4, 5) STRATA_CX(6, 7)
    STRATA_CX(2, 4) STRATA_CX(3, 5)
    STRATA_CX(1, 4) STRATA_CX(3, 6)
    STRATA_CX(1, 2) STRATA_CX(3, 4) STRATA_CX(5, 6)
#undef STRATA_CX
    my_id = 0;
    my_p = 0.f;
    sel = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (k > kmax)
            break;
        // the best head: the largest p, and among equal p the lowest id
        // (the one lane holding the maximum, else a reduction over ids)
        const int hb = __float_as_int(p[0]);
        const int bb = wave_max_i(hb);
        const float bp = __int_as_float(bb);
        const unsigned long long tie = __ballot(hb == bb);
        const int be = __popcll(tie) == 1
                           ? __builtin_amdgcn_readlane(e[0], (int)__builtin_ctzll(tie))
                           : wave_min63(hb == bb ? e[0] : 0x7fffffff);
        const bool pop = e[0] == be;
#pragma unroll
        for (int i = 0; i < 7; ++i) {
            p[i] = pop ? p[i + 1] : p[i];
            e[i] = pop ? e[i + 1] : e[i];
        }
        p[7] = pop ? -1.f : p[7];
        e[7] = pop ? 0x7fffffff : e[7];
        if (lane == k) {
            my_id = be;
            my_p = bp;
        }
        sel += bp;
    }
}

// The routing of logits loaded by load_logits: l = raw * sc (+ bias), heads
// up to kmax (route_scaled).
__device__ inline void route_logits(const TokLogits &t, float sc, bool has_bias, int &my_id,
                                    float &my_p, float &sel, int kmax = K - 1)
{
    float l[8];
    if (has_bias) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            l[i] = t.l[i] * sc + t.b[i];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            l[i] = t.l[i] * sc;
    }
    route_scaled(l, my_id, my_p, sel, kmax);
}

// One token's routing from its raw logits lrow[512]: l = lrow * sc (+ bias).
// The same arithmetic as route_logits; the loads are laid out apart (the
// bias read only when there is one), which the latency of the decode top-k
// kernel is sensitive to.
__device__ inline void route_token(const float *lrow, float sc, const float *bias, int &my_id,
                                   float &my_p, float &sel)
{
    const int lane = threadIdx.x & 63;
    float l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        l[i] = lrow[lane + 64 * i];
    if (bias) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            l[i] = l[i] * sc + bias[lane + 64 * i];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            l[i] = l[i] * sc;
    }
    route_scaled(l, my_id, my_p, sel);
}

} // namespace strata
