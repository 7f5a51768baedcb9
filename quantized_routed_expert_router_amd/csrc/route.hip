// route.hip -- activation prep and the router: logits = xhat . R^T (+ bias),
// softmax over all 512 experts, stable descending top-10, gather and
// renormalisation with a lower clamp ("MoE 遇上消费级显卡..." (zwxr.cn), the
// passage following one token through a layer: a BF16 GEMV to 512 logits, then
// a fused 512-expert softmax / stable argsort / gather / clamped renorm).
//
// Kernels:
//  prep_kernel    one workgroup per token: optional RMSNorm (eps 1e-6, unit
//                 gain), xhat as three bf16 terms for the router and fp16
//                 xhat in the K order the prefill MFMA kernels consume.  (Decode-sized T
//                 uses route_decode.hip.)
//  gemm_kernel    bf16 MFMA over the exact three-term bf16 split of xhat
//                 (fp32-accurate logits); identical router rows give
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

// bf16 bits of v, round to nearest even (finite inputs)
__device__ inline uint16_t bf16_rn_bits(float v)
{
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

__global__ __launch_bounds__(PREP_THREADS) void prep_kernel(
    const float *__restrict__ x, int rmsnorm, uint16_t *__restrict__ xsplit,
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
        const int c = tid + PREP_THREADS * i;
        xs[c] = h;
        // the router's exact three-term bf16 split of xhat
        const uint16_t b1 = bf16_rn_bits(h);
        const float r1 = h - bf16_bits_to_float(b1);   // exact
        const uint16_t b2 = bf16_rn_bits(r1);
        const float r2 = r1 - bf16_bits_to_float(b2);  // exact
        if (xsplit) {
            uint16_t *xo = xsplit + (size_t)t * 3 * H + c;
            xo[0] = b1;
            xo[H] = b2;
            xo[2 * H] = bf16_rn_bits(r2);
        }
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
// logits = xhat . R^T on the bf16 matrix cores.  R is bf16 already; the prep
// kernel splits each fp32 xhat value exactly into three bf16 terms
// x1 + x2 + x3 (x1 = bf16(x), x2 = bf16(x - x1), x3 = bf16(x - x1 - x2):
// together all 24 bits of the fp32 significand), and bf16 x bf16 products are
// exact in the fp32 accumulation, so the logits keep fp32 accuracy.  Every
// logit is the same sequence of MFMAs over K, so identical router rows give
// identical logits.  Workgroup: 16 tokens x 128 experts, wave w owns experts
// 32 w .. 32 w + 31 (two 16-expert subtiles); K in steps of 32, the operands
// of four steps in flight.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
constexpr int GR_M = 16, GR_N = 128, GR_KS = 32, GR_STEPS = H / GR_KS;
static_assert(GR_STEPS % 4 == 0 && E % GR_N == 0, "router GEMM tiling");

struct GrOps {
    uint4 a[3];   // x1, x2, x3: 8 bf16 of row lane % 16 at K 8 (lane / 16) ..
    uint4 b[2];   // 8 bf16 router values per expert subtile
};

__device__ inline void gr_load(GrOps &o, const uint16_t *xa, const uint16_t *rb0, const uint16_t *rb1,
                               int step)
{
#pragma unroll
    for (int j = 0; j < 3; ++j)
        o.a[j] = *reinterpret_cast<const uint4 *>(xa + (size_t)j * H + GR_KS * step);
    o.b[0] = *reinterpret_cast<const uint4 *>(rb0 + GR_KS * step);
    o.b[1] = *reinterpret_cast<const uint4 *>(rb1 + GR_KS * step);
}

__device__ inline void gr_step(const GrOps &o, floatx4 acc[2])
{
    const bf16x8 b0 = __builtin_bit_cast(bf16x8, o.b[0]);
    const bf16x8 b1 = __builtin_bit_cast(bf16x8, o.b[1]);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const bf16x8 xj = __builtin_bit_cast(bf16x8, o.a[j]);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xj, b0, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xj, b1, acc[1], 0, 0, 0);
    }
}

__global__ __launch_bounds__(256) void gemm_kernel(
    const uint16_t *__restrict__ xsplit, int T, const uint16_t *__restrict__ R,
    const float *__restrict__ bias, float *__restrict__ logits)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l = lane & 15, q = lane >> 4;
    const int m0 = blockIdx.x * GR_M;
    const int n0 = blockIdx.y * GR_N + 32 * wave;
    const int m = min(m0 + l, T - 1);   // rows past T compute a copy and are not stored
    const uint16_t *xa = xsplit + (size_t)m * 3 * H + 8 * q;
    const uint16_t *rb0 = R + (size_t)(n0 + l) * H + 8 * q;
    const uint16_t *rb1 = rb0 + (size_t)16 * H;
    floatx4 acc[2] = {(floatx4){0.f, 0.f, 0.f, 0.f}, (floatx4){0.f, 0.f, 0.f, 0.f}};
    GrOps p0, p1, p2, p3;
    gr_load(p0, xa, rb0, rb1, 0);
    gr_load(p1, xa, rb0, rb1, 1);
    gr_load(p2, xa, rb0, rb1, 2);
    gr_load(p3, xa, rb0, rb1, 3);
    // the last four loads re-read the last step (never used), so every
    // iteration issues the same loads
#pragma unroll 1
    for (int s = 0; s < GR_STEPS; s += 4) {
        gr_step(p0, acc);
        gr_load(p0, xa, rb0, rb1, min(s + 4, GR_STEPS - 1));
        gr_step(p1, acc);
        gr_load(p1, xa, rb0, rb1, min(s + 5, GR_STEPS - 1));
        gr_step(p2, acc);
        gr_load(p2, xa, rb0, rb1, min(s + 6, GR_STEPS - 1));
        gr_step(p3, acc);
        gr_load(p3, xa, rb0, rb1, min(s + 7, GR_STEPS - 1));
    }
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        const int n = n0 + 16 * ns + l;
        const float bn = bias ? bias[n] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int mr = m0 + 4 * q + r;
            if (mr < T)
                logits[(size_t)mr * E + n] = acc[ns][r] + bn;
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

hipError_t launch_prep(const float *x, int T, int rmsnorm, uint16_t *xsplit, __half *xperm,
                       hipStream_t st)
{
    hipLaunchKernelGGL(prep_kernel, dim3(T), dim3(PREP_THREADS), 0, st, x, rmsnorm, xsplit, xperm);
    return hipGetLastError();
}

hipError_t launch_logits(const uint16_t *xsplit, int T, const uint16_t *R, const float *bias,
                         float *logits, hipStream_t st)
{
    hipLaunchKernelGGL(gemm_kernel, dim3((T + GR_M - 1) / GR_M, E / GR_N), dim3(256), 0, st,
                       xsplit, T, R, bias, logits);
    return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int T, int32_t *ids, float *w, hipStream_t st)
{
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, ids, w);
    return hipGetLastError();
}

} // namespace strata
