// route_decode.hip -- the router for decode-sized T, in two launches.
//
// "MoE 遇上消费级显卡..." (zwxr.cn), the passage following one token through a
// layer: a BF16 GEMV projects the (normalised) activation onto 512 logits,
// then one fused kernel does the softmax over all experts, the stable
// descending argsort, the gather of the top 10 and the renormalisation with a
// lower clamp.
//
//  rdec_gemv   256 workgroups x 2 waves, one router row per wave: raw logits
//              R . x for every token (the RMSNorm factor is a per-token scalar
//              applied in rdec_topk), plus -- when asked -- the per-token
//              inverse RMS and the 16-bit quantisation of each 64-value block
//              of x for the experts (the RMSNorm factor stays out of the
//              quantisation: it scales the block scale).
//  rdec_topk   one workgroup: wave t takes token t (softmax with DPP
//              reductions, ten rounds of a wave-wide argmax on (p desc, id
//              asc), clamped renorm); then the workgroup groups the T*10 slots
//              by expert (counts, scan, active list, stable ranks).
#include "common.hpp"
#include "quant.hpp"

namespace strata {

constexpr int RG_THREADS = 128;
constexpr int RG_WAVES = RG_THREADS / 64;
constexpr int RG_BLOCKS = E / RG_WAVES;   // 256

// Work records of the decode expert kernels from a grouping (offsets, slots,
// active) that the caller supplies: erec[0] = {na, 0, 0, 0} and, for active
// expert a, erec[1 + a] = {e, beg, n, first slot}, every field clamped into
// range (an expert id outside 0..E-1 or a first slot outside 0..T*K-1 gives an
// empty record).
struct GroupIn {
    const int32_t *offsets, *slots, *active;
    int4 *erec;
};

__device__ inline void build_records(const GroupIn &gi, int T, int tid0, int nthreads)
{
    const int nslot = T * K;
    const int na = min(max(gi.active[0], 0), min(nslot, E));
    for (int i = tid0; i <= na; i += nthreads) {
        if (i == 0) {
            gi.erec[0] = make_int4(na, 0, 0, 0);
            continue;
        }
        const int e = gi.active[i];
        int4 r = make_int4(0, 0, 0, -1);
        if (e >= 0 && e < E) {
            const int beg = min(max(gi.offsets[e], 0), nslot);
            const int n = min(max(gi.offsets[e + 1], beg), nslot) - beg;
            const int s0 = n > 0 ? gi.slots[beg] : -1;
            if (s0 >= 0 && s0 < nslot)
                r = make_int4(e, beg, n, s0);
        }
        gi.erec[i] = r;
    }
}

template <bool GEMV, bool PREP>
__global__ __launch_bounds__(RG_THREADS) void rdec_gemv(const float *__restrict__ x, int T,
                                                        const uint16_t *__restrict__ R,
                                                        float *__restrict__ lraw, XQ xq,
                                                        int rmsnorm, GroupIn gi)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = blockIdx.x * RG_WAVES + wave;   // global wave id 0..511
    if (gi.erec)
        build_records(gi, T, g * 64 + lane, gridDim.x * RG_THREADS);
    if (GEMV) {
        const int e = g;
        const uint4 *row = reinterpret_cast<const uint4 *>(R + (size_t)e * H);
        float rv[40];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const uint4 q = row[lane + 64 * i];
            const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                rv[8 * i + 2 * j] = bf16_bits_to_float(u[j]);
                rv[8 * i + 2 * j + 1] = bf16_bits_to_float(u[j] >> 16);
            }
        }
        for (int t = 0; t < T; ++t) {
            const float4 *xr = reinterpret_cast<const float4 *>(x + (size_t)t * H);
            float4 xa[10];
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                xa[2 * i] = xr[2 * (lane + 64 * i)];
                xa[2 * i + 1] = xr[2 * (lane + 64 * i) + 1];
            }
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                acc = fmaf(rv[8 * i + 0], xa[2 * i].x, acc);
                acc = fmaf(rv[8 * i + 1], xa[2 * i].y, acc);
                acc = fmaf(rv[8 * i + 2], xa[2 * i].z, acc);
                acc = fmaf(rv[8 * i + 3], xa[2 * i].w, acc);
                acc = fmaf(rv[8 * i + 4], xa[2 * i + 1].x, acc);
                acc = fmaf(rv[8 * i + 5], xa[2 * i + 1].y, acc);
                acc = fmaf(rv[8 * i + 6], xa[2 * i + 1].z, acc);
                acc = fmaf(rv[8 * i + 7], xa[2 * i + 1].w, acc);
            }
            acc = wave_sum_dpp(acc);
            if (lane == 0)
                lraw[(size_t)t * E + e] = acc;
        }
    }
    const int nw = gridDim.x * RG_WAVES;
    // inverse RMS of token g (needed by the router and the experts)
    {
        for (int t = g; t < T; t += nw) {
            const float4 *xr = reinterpret_cast<const float4 *>(x + (size_t)t * H);
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 10; ++i) {
                const float4 a = xr[lane + 64 * i];
                ss = fmaf(a.x, a.x, ss);
                ss = fmaf(a.y, a.y, ss);
                ss = fmaf(a.z, a.z, ss);
                ss = fmaf(a.w, a.w, ss);
            }
            ss = wave_sum_dpp(ss);
            if (lane == 0)
                xq.inv_rms[t] = rmsnorm ? 1.f / sqrtf(ss / (float)H + 1e-6f) : 1.f;
        }
    }
    if (PREP) {
        // 16-bit quantisation of the 64-value blocks (token, block) = p
        for (int p = g; p < T * XBLK; p += nw) {
            const int t = p / XBLK, b = p % XBLK;
            const float v = x[(size_t)t * H + b * QK + lane];
            const QuantOut qo = quant_lanes<true>(v);
            const int l16 = lane & 15;
            if (l16 == 12 || l16 == 13)
                store_quarter(xq.dig + (size_t)p * BLK_DWORDS, lane >> 4, l16 - 12, qo.pk);
            if (lane == 0) {
                xq.scale[p] = qo.scale;
                xq.sum[p] = qo.sum;
            }
        }
    }
}

constexpr int RT_THREADS = 1024;

// (p, e) ranks before (q, f): larger probability, or equal and lower id.
__device__ inline bool ranks_before(float p, int e, float q, int f)
{
    return p > q || (p == q && e < f);
}

__global__ __launch_bounds__(RT_THREADS) void rdec_topk(
    const float *__restrict__ lraw, const float *__restrict__ inv_rms, const float *__restrict__ bias,
    int T, int32_t *__restrict__ ids, float *__restrict__ wout, int group,
    int32_t *__restrict__ offsets, int32_t *__restrict__ slots, int32_t *__restrict__ active,
    int4 *__restrict__ erec)
{
    constexpr int NW_SLOT = (DECODE_T_MAX * K + 63) / 64;   // waves holding slots (3)
    __shared__ int sid[NW_SLOT * 64];
    __shared__ int cntw[NW_SLOT][E];
    __shared__ int offl[E];
    __shared__ int first[E];
    __shared__ int wsum[8];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int N = T * K;
    for (int i = tid; i < NW_SLOT * E; i += RT_THREADS)
        (&cntw[0][0])[i] = 0;
    for (int i = tid; i < NW_SLOT * 64; i += RT_THREADS)
        sid[i] = -1;
    __syncthreads();
    if (wave < T) {
        const int t = wave;
        const float sc = inv_rms[t];
        float l[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            l[i] = lraw[(size_t)t * E + lane + 64 * i];
        if (bias) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                l[i] = l[i] * sc + bias[lane + 64 * i];
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                l[i] = l[i] * sc;
        }
        float m = l[0];
#pragma unroll
        for (int i = 1; i < 8; ++i)
            m = fmaxf(m, l[i]);
        m = wave_max_dpp(m);
        float p[8], s = 0.f;
        int e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = expf(l[i] - m);
            s += p[i];
            e[i] = lane + 64 * i;
        }
        s = wave_sum_dpp(s);
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
        int my_id = 0;
        float my_p = 0.f, sel = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float bp = p[0];
            int be = e[0];
            wave_argmax(bp, be);
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
        const float den = fmaxf(sel, 6.103515625e-05f);   // clamp 2^-14
        if (lane < K) {
            ids[(size_t)t * K + lane] = my_id;
            wout[(size_t)t * K + lane] = my_p / den;
            sid[t * K + lane] = my_id;
        }
    }
    if (!group)
        return;
    __syncthreads();
    // Grouping of the N = T*K slots: per-wave counts, scan, active list, and
    // stable ranks from ballots (equal ids inside a 64-slot wave) plus the
    // counts of the earlier waves.
    int my_e = -1;
    if (wave < NW_SLOT) {
        my_e = sid[tid];
        if (my_e >= 0 && my_e < E && tid < N)
            atomicAdd(&cntw[wave][my_e], 1);
        else
            my_e = -1;
    }
    __syncthreads();
    int c = 0, inc = 0;
    if (tid < E) {
#pragma unroll
        for (int w = 0; w < NW_SLOT; ++w)
            c += cntw[w][tid];
        inc = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(inc, d, 64);
            if (lane >= d)
                inc += o;
        }
        if (lane == 63)
            wsum[wave] = inc;
    }
    __syncthreads();
    int off = 0;
    if (tid < E) {
        int base = 0;
        for (int w = 0; w < wave; ++w)
            base += wsum[w];
        off = base + inc - c;
        offsets[tid] = off;
        offl[tid] = off;
        if (tid == E - 1)
            offsets[E] = base + inc;
    }
    __syncthreads();
    int f = 0, finc = 0;
    if (tid < E) {
        f = c > 0;
        finc = f;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(finc, d, 64);
            if (lane >= d)
                finc += o;
        }
        if (lane == 63)
            wsum[wave] = finc;
    }
    __syncthreads();
    int my_a = -1;
    if (tid < E) {
        int base = 0;
        for (int w = 0; w < wave; ++w)
            base += wsum[w];
        if (f) {
            my_a = base + finc - 1;
            active[1 + my_a] = tid;
        }
        if (tid == E - 1) {
            active[0] = base + finc;
            erec[0] = make_int4(base + finc, 0, 0, 0);
        }
    }
    if (wave < NW_SLOT) {
        unsigned long long same = __ballot(my_e >= 0);
#pragma unroll
        for (int bit = 0; bit < 9; ++bit) {
            const unsigned long long bits = __ballot(my_e >= 0 && ((my_e >> bit) & 1));
            same &= ((my_e >> bit) & 1) ? bits : ~bits;
        }
        if (my_e >= 0) {
            int rank = __popcll(same & ((1ull << lane) - 1ull));
            for (int w = 0; w < wave; ++w)
                rank += cntw[w][my_e];
            slots[offl[my_e] + rank] = tid;
            if (rank == 0)
                first[my_e] = tid;
        }
    }
    __syncthreads();
    // work record of each active expert: {e, first grouped slot, count, first slot}
    if (my_a >= 0)
        erec[1 + my_a] = make_int4(tid, off, c, first[tid]);
}

hipError_t launch_route_decode(const float *x, int T, const uint16_t *R, const float *bias,
                               int rmsnorm, float *lraw, XQ xq, bool prep, int32_t *ids,
                               float *w, int group, int32_t *offsets, int32_t *slots,
                               int32_t *active, int4 *erec, hipStream_t st)
{
    const GroupIn none{nullptr, nullptr, nullptr, nullptr};
    if (prep)
        hipLaunchKernelGGL((rdec_gemv<true, true>), dim3(RG_BLOCKS), dim3(RG_THREADS), 0, st, x,
                           T, R, lraw, xq, rmsnorm, none);
    else
        hipLaunchKernelGGL((rdec_gemv<true, false>), dim3(RG_BLOCKS), dim3(RG_THREADS), 0, st, x,
                           T, R, lraw, xq, rmsnorm, none);
    hipLaunchKernelGGL(rdec_topk, dim3(1), dim3(RT_THREADS), 0, st, lraw, xq.inv_rms, bias, T, ids,
                       w, group, offsets, slots, active, erec);
    return hipGetLastError();
}

hipError_t launch_prep_decode(const float *x, int T, int rmsnorm, XQ xq, const int32_t *offsets,
                              const int32_t *slots, const int32_t *active, int4 *erec,
                              hipStream_t st)
{
    const int blocks = min(RG_BLOCKS, (T * XBLK + RG_WAVES - 1) / RG_WAVES);
    const GroupIn gi{offsets, slots, active, erec};
    hipLaunchKernelGGL((rdec_gemv<false, true>), dim3(blocks), dim3(RG_THREADS), 0, st, x, T,
                       (const uint16_t *)nullptr, (float *)nullptr, xq, rmsnorm, gi);
    return hipGetLastError();
}

} // namespace strata
