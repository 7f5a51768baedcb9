// route.hip -- activation prep and the router: logits = xhat . R^T (+ bias),
// softmax over all 512 experts, stable descending top-10, gather and
// renormalisation with a lower clamp ("MoE 遇上消费级显卡..." (zwxr.cn), the
// passage following one token through a layer: a BF16 GEMV to 512 logits, then
// a fused 512-expert softmax / stable argsort / gather / clamped renorm).
//
// Kernels:
//  prep_kernel    one workgroup per token: optional RMSNorm (eps 1e-6, unit
//                 gain), xhat in fp32 for the router and fp16 xhat in the K
//                 order the prefill MFMA kernels consume.  (Decode-sized T
//                 uses route_decode.hip.)
//  gemm_kernel    64 x 64 fp32 tiles through LDS; each logit is a sequential
//                 k = 0..2559 FMA chain, so identical router rows give
//                 identical logits.
//  topk_kernel    one wave per token: softmax in fp32, ten rounds of a
//                 wave-wide max of p and min of the id among the maxima
//                 (the order p desc, id asc), clamped renorm.
#include "common.hpp"

namespace strata {

// Position pi (0..63) of a block in the prefill K order holds input column
// 16 q + 4 j + s/2 + 8 (s % 2) with pi = 32 j + 8 q + s (see experts_prefill).
__device__ inline int pf_col_of_pos(int pi)
{
    const int j = pi >> 5, q = (pi >> 3) & 3, s = pi & 7;
    return 16 * q + 4 * j + (s >> 1) + 8 * (s & 1);
}

constexpr int PREP_THREADS = 256;

__global__ __launch_bounds__(PREP_THREADS) void prep_kernel(
    const float *__restrict__ x, int rmsnorm, float *__restrict__ xhat,
    __half *__restrict__ xperm)
{
    __shared__ float xs[H];
    __shared__ float wsum[PREP_THREADS / 64];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const float *xt = x + (size_t)t * H;
    float v[H / PREP_THREADS];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < H / PREP_THREADS; ++i) {
        v[i] = xt[tid + PREP_THREADS * i];
        ss = fmaf(v[i], v[i], ss);
    }
    float inv = 1.f;
    if (rmsnorm) {
        ss = wave_sum63(ss);
        if ((tid & 63) == 0)
            wsum[tid >> 6] = ss;
        __syncthreads();
        const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
        inv = 1.f / sqrtf(tot / (float)H + 1e-6f);
    }
#pragma unroll
    for (int i = 0; i < H / PREP_THREADS; ++i) {
        const float h = v[i] * inv;
        xs[tid + PREP_THREADS * i] = h;
        xhat[(size_t)t * H + tid + PREP_THREADS * i] = h;
    }
    __syncthreads();
    if (xperm) {
        for (int pos = tid; pos < H; pos += PREP_THREADS) {
            const int b = pos >> 6;
            xperm[(size_t)t * H + pos] = __float2half_rn(xs[b * QK + pf_col_of_pos(pos & 63)]);
        }
    }
}

// ---------------------------------------------------------------- router GEMM
constexpr int GM_TILE = 64;
constexpr int GM_KC = 32;

__global__ __launch_bounds__(256) void gemm_kernel(
    const float *__restrict__ xhat, int T, const uint16_t *__restrict__ R,
    const float *__restrict__ bias, float *__restrict__ logits)
{
    __shared__ float xs[GM_KC][GM_TILE + 4];
    __shared__ float rs[GM_KC][GM_TILE + 4];
    const int tid = threadIdx.x;
    const int m0 = blockIdx.x * GM_TILE;
    const int n0 = blockIdx.y * GM_TILE;
    const int ty = tid >> 4, tx = tid & 15;
    const int lrow = tid >> 2, lk = (tid & 3) * 8;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < H; k0 += GM_KC) {
        const int m = m0 + lrow;
        float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
        if (m < T) {
            const float4 *src = reinterpret_cast<const float4 *>(xhat + (size_t)m * H + k0 + lk);
            a0 = src[0];
            a1 = src[1];
        }
        const uint4 rq = *reinterpret_cast<const uint4 *>(R + (size_t)(n0 + lrow) * H + k0 + lk);
        __syncthreads();
        xs[lk + 0][lrow] = a0.x;
        xs[lk + 1][lrow] = a0.y;
        xs[lk + 2][lrow] = a0.z;
        xs[lk + 3][lrow] = a0.w;
        xs[lk + 4][lrow] = a1.x;
        xs[lk + 5][lrow] = a1.y;
        xs[lk + 6][lrow] = a1.z;
        xs[lk + 7][lrow] = a1.w;
        const uint32_t u[4] = {rq.x, rq.y, rq.z, rq.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rs[lk + 2 * j][lrow] = bf16_bits_to_float(u[j]);
            rs[lk + 2 * j + 1][lrow] = bf16_bits_to_float(u[j] >> 16);
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < GM_KC; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = xs[kk][ty + 16 * i];
                b[i] = rs[kk][tx + 16 * i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty + 16 * i;
        if (m >= T)
            continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx + 16 * j;
            logits[(size_t)m * E + n] = acc[i][j] + (bias ? bias[n] : 0.f);
        }
    }
}

// ---------------------------------------------------------------- softmax / top-k
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T,
                                                   int32_t *__restrict__ ids,
                                                   float *__restrict__ wout)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T)
        return;
    const float *lt = logits + (size_t)t * E;
    float l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        l[i] = lt[lane + 64 * i];
    float m = l[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
        m = fmaxf(m, l[i]);
    m = wave_max63(m);
    float p[8];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        p[i] = expf(l[i] - m);
        s += p[i];
    }
    s = wave_sum63(s);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        p[i] = p[i] / s;
    unsigned taken = 0;
    int my_id = 0;
    float my_p = 0.f;
    float sel_sum = 0.f;
    for (int k = 0; k < K; ++k) {
        float bp = -1.f;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = lane + 64 * i;
            const bool better = p[i] > bp || (p[i] == bp && e < be);
            if (!((taken >> i) & 1) && better) {
                bp = p[i];
                be = e;
            }
        }
        // the best candidate: the largest p, and among equal p the lowest id
        const float pm = wave_max63(bp);
        be = wave_min63(bp == pm ? be : 0x7fffffff);
        bp = pm;
        if ((be & 63) == lane)
            taken |= 1u << ((be >> 6) & 7);
        if (lane == k) {
            my_id = be;
            my_p = bp;
        }
        sel_sum += bp;
    }
    const float den = fmaxf(sel_sum, 6.103515625e-05f);   // clamp 2^-14
    if (lane < K) {
        ids[(size_t)t * K + lane] = my_id;
        wout[(size_t)t * K + lane] = my_p / den;
    }
}

hipError_t launch_prep(const float *x, int T, int rmsnorm, float *xhat, __half *xperm,
                       hipStream_t st)
{
    hipLaunchKernelGGL(prep_kernel, dim3(T), dim3(PREP_THREADS), 0, st, x, rmsnorm, xhat, xperm);
    return hipGetLastError();
}

hipError_t launch_logits(const float *xhat, int T, const uint16_t *R, const float *bias,
                         float *logits, hipStream_t st)
{
    hipLaunchKernelGGL(gemm_kernel, dim3((T + GM_TILE - 1) / GM_TILE, E / GM_TILE), dim3(256), 0,
                       st, xhat, T, R, bias, logits);
    return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int T, int32_t *ids, float *w, hipStream_t st)
{
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, ids, w);
    return hipGetLastError();
}

} // namespace strata
