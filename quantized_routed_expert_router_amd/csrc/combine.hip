// combine.hip -- the layer's weighted sum of its experts' outputs,
// y_t = sum_k w[t][k] * out[t*K + k] in routing order ("MoE 遇上消费级显卡..."
// (zwxr.cn), Combine: the inter-layer sync point is one weighted sum), with an
// optional residual add (x += y) for stacked layers.
#include "common.hpp"

namespace strata {

constexpr int CB_THREADS = 256;
constexpr int CB_VEC = 4;

// y (may be NULL) receives the sum; with `residual`, res (may be NULL) gets
// res += sum; a non-residual call stores the sum into y.
__global__ __launch_bounds__(CB_THREADS) void combine_kernel(
    const float *__restrict__ out, const float *__restrict__ w, float *y, float *res,
    int accumulate_y)
{
    const int t = blockIdx.y;
    const int r = (blockIdx.x * CB_THREADS + threadIdx.x) * CB_VEC;
    if (r >= H)
        return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float wk = w[(size_t)t * K + k];
        const float4 o = *reinterpret_cast<const float4 *>(out + ((size_t)t * K + k) * H + r);
        acc.x = fmaf(wk, o.x, acc.x);
        acc.y = fmaf(wk, o.y, acc.y);
        acc.z = fmaf(wk, o.z, acc.z);
        acc.w = fmaf(wk, o.w, acc.w);
    }
    if (y) {
        float4 *yp = reinterpret_cast<float4 *>(y + (size_t)t * H + r);
        if (accumulate_y) {
            float4 v = *yp;
            v.x += acc.x;
            v.y += acc.y;
            v.z += acc.z;
            v.w += acc.w;
            *yp = v;
        } else {
            *yp = acc;
        }
    }
    if (res) {
        float4 *xp = reinterpret_cast<float4 *>(res + (size_t)t * H + r);
        float4 v = *xp;
        v.x += acc.x;
        v.y += acc.y;
        v.z += acc.z;
        v.w += acc.w;
        *xp = v;
    }
}

hipError_t launch_combine(const float *out, const float *w, int T, float *y, float *res,
                          int accumulate_y, hipStream_t st)
{
    const int nb = (H / CB_VEC + CB_THREADS - 1) / CB_THREADS;
    hipLaunchKernelGGL(combine_kernel, dim3(nb, T), dim3(CB_THREADS), 0, st, out, w, y, res,
                       accumulate_y);
    return hipGetLastError();
}

} // namespace strata
