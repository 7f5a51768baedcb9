// route_decode.hip -- the router for decode-sized T, in two launches.
//
// "MoE 遇上消费级显卡..." (zwxr.cn), the passage following one token through a
// layer: a BF16 GEMV projects the (normalised) activation onto 512 logits,
// then one fused kernel does the softmax over all experts, the stable
// descending argsort, the gather of the top 10 and the renormalisation with a
// lower clamp.
//
//  rdec_gemv   one workgroup of 5 waves per router row: wave w holds the row's
//              elements 512 w .. 512 w + 511 (8 per lane), reads x for up to
//              8 tokens at once and reduces each token's partial dot product
//              with DPP; the 5 partials meet in LDS in a fixed order.  These
//              are the raw logits R . x (the RMSNorm factor is a per-token
//              scalar applied in rdec_topk).  The same launch computes the
//              per-token inverse RMS and, when asked, the 16-bit quantisation
//              of each 64-value block of x for the experts (the RMSNorm factor
//              stays out of the quantisation: it scales the block scale).
//  rdec_topk   one workgroup: wave t takes token t (softmax with DPP
//              reductions, a sorting network on each lane's 8 candidates, then
//              ten rounds of a wave-wide max of p and min of the id among the
//              maxima -- the order (p desc, id asc) -- and the clamped renorm).
//              With a lookahead (the next layer's router, second half of
//              the GEMV grid), waves T .. 2T-1 route the same tokens through
//              it and write the predicted ids.
//              For the layer, wave 0 then groups the T*10 slots by expert
//              with ballots over the bits of the expert ids (stable slot
//              order and one work record per active expert for the experts
//              kernel), and the waves without a token zero the experts
//              kernel's counters.
#include "common.hpp"
#include "quant.hpp"
#include "route_token.hpp"

namespace strata {

constexpr int RG_WAVES = 5;                       // waves per router row
constexpr int RG_THREADS = 64 * RG_WAVES;
constexpr int RG_SPAN = H / RG_WAVES;             // 512 elements per wave
constexpr int RG_TOK = 8;                         // tokens whose x is in flight at once
static_assert(RG_SPAN == 64 * 8, "8 elements per lane");

// Work records of the decode expert kernels from a grouping (offsets, slots,
// active) that the caller supplies: erec[0] = {na, 0, 0, 0} and, for active
// expert a, erec[1 + a] = {e, beg, n, first slot}, every field clamped into
// range (an expert id outside 0..E-1 or a first slot outside 0..T*K-1 gives an
// empty record).
struct GroupIn {
    const int32_t *offsets, *slots, *active;
    int4 *erec;
    int32_t *esync;   // counters of the experts kernel (one per active expert), zeroed here
};

__device__ inline void build_records(const GroupIn &gi, int T, int tid0, int nthreads)
{
    const int nslot = T * K;
    const int na = min(max(gi.active[0], 0), min(nslot, E));
    for (int i = tid0; i < na; i += nthreads)
        gi.esync[1 + SYNC_STRIDE * i] = 0;
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

// With R2 given (lookahead), workgroups E .. 2E-1 compute the raw logits of a
// second router (the next layer's) on the same x into lraw2.
template <bool GEMV, bool PREP>
__global__ __launch_bounds__(RG_THREADS) void rdec_gemv(const float *__restrict__ x, int T,
                                                        const uint16_t *__restrict__ R,
                                                        float *__restrict__ lraw, XQ xq,
                                                        int rmsnorm, GroupIn gi,
                                                        const uint16_t *__restrict__ R2,
                                                        float *__restrict__ lraw2)
{
    __shared__ float part[RG_WAVES][DECODE_T_MAX];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = blockIdx.x * RG_WAVES + wave;   // global wave id
    const int nw = gridDim.x * RG_WAVES;
    if (gi.erec)
        build_records(gi, T, g * 64 + lane, nw * 64);
    if (GEMV) {
        const bool second = blockIdx.x >= E;
        const int e = second ? blockIdx.x - E : blockIdx.x;
        const uint16_t *Rm = second ? R2 : R;
        float *lout = second ? lraw2 : lraw;
        const int k0 = wave * RG_SPAN + 8 * lane;
        const uint4 q = *reinterpret_cast<const uint4 *>(Rm + (size_t)e * H + k0);
        const float r0 = bf16_bits_to_float(q.x), r1 = bf16_bits_to_float(q.x >> 16);
        const float r2 = bf16_bits_to_float(q.y), r3 = bf16_bits_to_float(q.y >> 16);
        const float r4 = bf16_bits_to_float(q.z), r5 = bf16_bits_to_float(q.z >> 16);
        const float r6 = bf16_bits_to_float(q.w), r7 = bf16_bits_to_float(q.w >> 16);
        for (int t0 = 0; t0 < T; t0 += RG_TOK) {
            float4 xa[RG_TOK], xb[RG_TOK];
#pragma unroll
            for (int i = 0; i < RG_TOK; ++i) {
                if (t0 + i < T) {
                    const float4 *xr =
                        reinterpret_cast<const float4 *>(x + (size_t)(t0 + i) * H + k0);
                    xa[i] = xr[0];
                    xb[i] = xr[1];
                }
            }
#pragma unroll
            for (int i = 0; i < RG_TOK; ++i) {
                if (t0 + i < T) {
                    float acc = r0 * xa[i].x;
                    acc = fmaf(r1, xa[i].y, acc);
                    acc = fmaf(r2, xa[i].z, acc);
                    acc = fmaf(r3, xa[i].w, acc);
                    acc = fmaf(r4, xb[i].x, acc);
                    acc = fmaf(r5, xb[i].y, acc);
                    acc = fmaf(r6, xb[i].z, acc);
                    acc = fmaf(r7, xb[i].w, acc);
                    acc = wave_sum63(acc);
                    if (lane == 0)
                        part[wave][t0 + i] = acc;
                }
            }
        }
        __syncthreads();
        if (tid < T)
            lout[(size_t)tid * E + e] =
                (((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid]) + part[4][tid];
    }
    // inverse RMS of token g (needed by the router and the experts)
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
        ss = wave_sum63(ss);
        if (lane == 0)
            xq.inv_rms[t] = rmsnorm ? 1.f / sqrtf(ss / (float)H + 1e-6f) : 1.f;
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
                xq.nsum[p] = -qo.sum;
            }
        }
    }
}

constexpr int RT_THREADS = 64 * DECODE_T_MAX;     // one wave per token

// Workgroup barrier for LDS data only: unlike __syncthreads it does not make
// every wave wait for its outstanding global stores (here the zeroing of the
// experts kernel's counters, which only that later launch reads).
__device__ inline void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Zero the experts kernel's per-call counters: the per-(token, 32 output
// rows) slot counters and the per-active-expert item counters.
__device__ inline void zero_counters(int32_t *cdone, int32_t *esync, int T, int i0, int n)
{
    if (cdone)
        for (int i = i0; i < T * (H / 32); i += n)
            cdone[i] = 0;
    if (esync) {
        const int amax = T * K < E ? T * K : E;
        for (int i = i0; i < amax; i += n)
            esync[1 + SYNC_STRIDE * i] = 0;
    }
}

// Grouping of the N = T * K slots by expert, in one wave: slot s (lane s % 64
// of chunk s / 64) has expert sid[s].  Ten ballots over the bits of a chunk's
// ids (1023 past the end) give every lane the masks of that chunk's slots
// whose expert is below its own (lt) and equal to it (eq), comparing bits
// from the top.  Then, for slot s of expert e:
//   less  = slots of the experts below e       (where e's run starts)
//   rank  = slots of e before s                (stable order)
//   below = active experts below e             (e's record index)
// slots[less + rank] = s, and the first slot of e writes e's record
// {e, less, slots of e, s}; erec[0].x is the number of active experts.
__device__ inline int chunk_expert(const int *sid, int N, int c, int lane)
{
    return 64 * c + lane < N ? sid[64 * c + lane] : 1023;
}

// lt / eq masks of the lane's expert e against the experts m of one chunk.
__device__ inline void compare_chunk(int e, int m, unsigned long long &lt, unsigned long long &eq)
{
    unsigned long long l = 0, q = ~0ull;
#pragma unroll
    for (int b = 9; b >= 0; --b) {
        const unsigned long long bm = __ballot((m >> b) & 1);
        const bool one = (e >> b) & 1;
        l |= one ? (q & ~bm) : 0ull;
        q &= one ? bm : ~bm;
    }
    lt = l;
    eq = q;
}

template <int NC>
__device__ inline void group_slots(const int *sid, int N, int32_t *slots, int4 *erec, int lane)
{
    unsigned long long first[NC], lt0 = 0;
    int less[NC], rank[NC], cnt[NC];
#pragma unroll
    for (int c0 = 0; c0 < NC; ++c0) {
        const int e = chunk_expert(sid, N, c0, lane);
        less[c0] = 0;
        rank[c0] = 0;
        cnt[c0] = 0;
        unsigned long long self = 0;
#pragma unroll 1
        for (int c = 0; c < NC; ++c) {
            unsigned long long lt, eq;
            compare_chunk(e, chunk_expert(sid, N, c, lane), lt, eq);
            less[c0] += __popcll(lt);
            cnt[c0] += __popcll(eq);
            if (c < c0)
                rank[c0] += __popcll(eq);
            if (c == c0)
                self = eq;
            if (NC == 1)
                lt0 = lt;
        }
        rank[c0] += __builtin_amdgcn_mbcnt_hi((uint32_t)(self >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)self, 0));
        first[c0] = __ballot(64 * c0 + lane < N && rank[c0] == 0);
    }
    int na = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c)
        na += __popcll(first[c]);
#pragma unroll
    for (int c0 = 0; c0 < NC; ++c0) {
        const int e = chunk_expert(sid, N, c0, lane);
        int below = 0;
        if (NC == 1) {
            below = __popcll(lt0 & first[0]);
        } else {
#pragma unroll 1
            for (int c = 0; c < NC; ++c) {
                unsigned long long lt, eq;
                compare_chunk(e, chunk_expert(sid, N, c, lane), lt, eq);
                below += __popcll(lt & first[c]);
            }
        }
        const int s = 64 * c0 + lane;
        if (s < N) {
            slots[less[c0] + rank[c0]] = s;
            if (rank[c0] == 0)
                erec[1 + below] = make_int4(e, less[c0], cnt[c0], s);
        }
    }
    if (lane == 0)
        erec[0] = make_int4(na, 0, 0, 0);
}

// With pred given (lookahead, 2T <= 16), waves T .. 2T-1 also route token
// wave - T through the second router's raw logits lraw2 (+ bias2) and write
// its ten ids to pred.
__global__ __launch_bounds__(RT_THREADS) void rdec_topk(
    const float *__restrict__ lraw, const float *__restrict__ inv_rms, const float *__restrict__ bias,
    int T, int32_t *__restrict__ ids, float *__restrict__ wout, int group,
    int32_t *__restrict__ slots, int4 *__restrict__ erec, int32_t *__restrict__ cdone,
    int32_t *__restrict__ esync, const float *__restrict__ lraw2, const float *__restrict__ bias2,
    int32_t *__restrict__ pred)
{
    __shared__ int sid[DECODE_T_MAX * K];   // expert of each slot
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int N = T * K;
    const int busy = pred ? 2 * T : T;   // waves with a token to route
    // Waves without a token zero the counters at once; with every wave busy
    // the token waves do it after reading the logits (one counter orders a
    // wave's loads and stores).
    const bool zero_early = busy < DECODE_T_MAX;
    if (zero_early && wave >= busy)
        zero_counters(cdone, esync, T, tid - 64 * busy, RT_THREADS - 64 * busy);
    if (wave < T) {
        const int t = wave;
        int my_id;
        float my_p, sel;
        route_token(lraw + (size_t)t * E, inv_rms[t], bias, my_id, my_p, sel);
        const float den = renorm_den(sel);
        if (lane < K) {
            ids[(size_t)t * K + lane] = my_id;
            wout[(size_t)t * K + lane] = my_p / den;
            if (group)
                sid[t * K + lane] = my_id;
        }
    } else if (wave < busy) {
        const int t = wave - T;
        int my_id;
        float my_p, sel;
        route_token(lraw2 + (size_t)t * E, inv_rms[t], bias2, my_id, my_p, sel);
        if (lane < K)
            pred[(size_t)t * K + lane] = my_id;
    }
    if (!zero_early)
        zero_counters(cdone, esync, T, tid, RT_THREADS);
    if (!group)
        return;
    lds_barrier();
    if (wave != 0)
        return;
    if (N <= 64)
        group_slots<1>(sid, N, slots, erec, lane);
    else if (N <= 128)
        group_slots<2>(sid, N, slots, erec, lane);
    else
        group_slots<3>(sid, N, slots, erec, lane);
}

hipError_t launch_route_decode(const float *x, int T, const uint16_t *R, const float *bias,
                               int rmsnorm, float *lraw, XQ xq, bool prep, int32_t *ids,
                               float *w, int group, int32_t *slots, int4 *erec, int32_t *cdone,
                               int32_t *esync, const uint16_t *R2, const float *bias2,
                               float *lraw2, int32_t *pred, hipStream_t st)
{
    const GroupIn none{nullptr, nullptr, nullptr, nullptr, nullptr};
    const dim3 grid(R2 ? 2 * E : E);
    if (prep)
        hipLaunchKernelGGL((rdec_gemv<true, true>), grid, dim3(RG_THREADS), 0, st, x, T, R, lraw,
                           xq, rmsnorm, none, R2, lraw2);
    else
        hipLaunchKernelGGL((rdec_gemv<true, false>), grid, dim3(RG_THREADS), 0, st, x, T, R, lraw,
                           xq, rmsnorm, none, R2, lraw2);
    hipLaunchKernelGGL(rdec_topk, dim3(1), dim3(RT_THREADS), 0, st, lraw, xq.inv_rms, bias, T, ids,
                       w, group, slots, erec, cdone, esync, R2 ? lraw2 : nullptr, bias2,
                       R2 ? pred : nullptr);
    return hipGetLastError();
}

// The router GEMV alone (with the 16-bit quantisation of x; with R2, the
// second router's raw logits too): the one-token layer call routes inside its
// gate/up launch.
hipError_t launch_router_gemv(const float *x, int T, const uint16_t *R, int rmsnorm, float *lraw,
                              XQ xq, const uint16_t *R2, float *lraw2, hipStream_t st)
{
    const GroupIn none{nullptr, nullptr, nullptr, nullptr, nullptr};
    hipLaunchKernelGGL((rdec_gemv<true, true>), dim3(R2 ? 2 * E : E), dim3(RG_THREADS), 0, st, x,
                       T, R, lraw, xq, rmsnorm, none, R2, lraw2);
    return hipGetLastError();
}

hipError_t launch_prep_decode(const float *x, int T, int rmsnorm, XQ xq, const int32_t *offsets,
                              const int32_t *slots, const int32_t *active, int4 *erec,
                              int32_t *esync, hipStream_t st)
{
    const int blocks = (T * XBLK + RG_WAVES - 1) / RG_WAVES;
    const GroupIn gi{offsets, slots, active, erec, esync};
    hipLaunchKernelGGL((rdec_gemv<false, true>), dim3(blocks), dim3(RG_THREADS), 0, st, x, T,
                       (const uint16_t *)nullptr, (float *)nullptr, xq, rmsnorm, gi,
                       (const uint16_t *)nullptr, (float *)nullptr);
    return hipGetLastError();
}

} // namespace strata
