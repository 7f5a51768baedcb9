// group.hip -- token -> expert grouping and the prefill work list.
//
// Collecting the tokens of a chunk per expert lets one read of an expert's
// weights serve all of them (the momoyeyu.github.io Strata explainer, section
// 提示词处理: four tokens of one expert read its weights once, W X with
// X = [x1..x4]); for a verify window it is the dedup of routed ids ("Strata in
// the source...", section "The plan: three destinations per expert").
//
// group_kernel (decode-sized T) is one 1024-thread workgroup: per-wave histograms in LDS
// (integer atomics, so the counts are exact), an exclusive scan to offsets, the
// ascending active-expert list, then a stable scatter in which each wave walks
// its contiguous slice of slots in order and ranks equal experts inside a
// 64-slot step with ballots.  Every output is a pure function of ids.
#include "common.hpp"

namespace strata {

constexpr int GR_THREADS = 1024;
constexpr int GR_WAVES = GR_THREADS / 64;
constexpr int GR_BATCH = 24;  // 64-slot steps whose ids are loaded together

__device__ inline int block_exclusive_scan_512(int v, int tid, int *tmp, int *total)
{
    // tid < 512 contribute v; returns the exclusive prefix for tid < 512.
    // tmp holds 8 wave sums.  Called by all threads of the block.
    const int lane = tid & 63, wave = tid >> 6;
    int inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d, 64);
        if (lane >= d)
            inc += o;
    }
    if (tid < 512 && lane == 63)
        tmp[wave] = inc;
    __syncthreads();
    int base = 0;
    if (tid < 512)
        for (int w = 0; w < wave; ++w)
            base += tmp[w];
    if (tid == 0) {
        int s = 0;
        for (int w = 0; w < 8; ++w)
            s += tmp[w];
        *total = s;
    }
    __syncthreads();
    return base + inc - v;
}

__global__ __launch_bounds__(GR_THREADS) void group_kernel(const int32_t *__restrict__ ids,
                                                           int T, int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ slots,
                                                           int32_t *__restrict__ active)
{
    __shared__ int hist[GR_WAVES][E];
    __shared__ int tmp[8];
    __shared__ int tot;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int N = T * K;
    const int S = (N + GR_WAVES - 1) / GR_WAVES;   // slots per wave
    const int beg = min(wave * S, N), end = min(beg + S, N);

    for (int i = tid; i < GR_WAVES * E; i += GR_THREADS)
        (&hist[0][0])[i] = 0;
    // The ids are read GR_BATCH 64-slot steps at a time, so their loads
    // overlap; when a wave's slice fits one batch (T <= 2457), the ids stay in
    // registers for the scatter too.
    const int steps = (S + 63) / 64;
    int ev[GR_BATCH];
#pragma unroll
    for (int j = 0; j < GR_BATCH; ++j) {
        const int i = beg + j * 64 + lane;
        ev[j] = i < end ? ids[i] : -1;
    }
    __syncthreads();
    for (int it0 = 0; it0 < steps; it0 += GR_BATCH) {
        if (it0 > 0) {
#pragma unroll
            for (int j = 0; j < GR_BATCH; ++j) {
                const int i = beg + (it0 + j) * 64 + lane;
                ev[j] = i < end ? ids[i] : -1;
            }
        }
#pragma unroll
        for (int j = 0; j < GR_BATCH; ++j)
            if (ev[j] >= 0 && ev[j] < E)
                atomicAdd(&hist[wave][ev[j]], 1);
    }
    __syncthreads();
    // Per expert: each wave's start within the expert, and the expert total.
    int count = 0;
    if (tid < E) {
        int run = 0;
        for (int w = 0; w < GR_WAVES; ++w) {
            const int c = hist[w][tid];
            hist[w][tid] = run;
            run += c;
        }
        count = run;
    }
    const int off = block_exclusive_scan_512(count, tid, tmp, &tot);
    if (tid < E) {
        offsets[tid] = off;
        for (int w = 0; w < GR_WAVES; ++w)
            hist[w][tid] += off;   // now the wave's cursor for expert tid
    }
    if (tid == 0)
        offsets[E] = tot;
    const int flag = (tid < E && count > 0) ? 1 : 0;
    const int pos = block_exclusive_scan_512(flag, tid, tmp, &tot);
    if (flag)
        active[1 + pos] = tid;
    if (tid == 0)
        active[0] = tot;
    __syncthreads();

    // Stable scatter: each wave walks its slice in order; a wave's cursors
    // (hist[wave]) are its own, and LDS keeps one wave's accesses in order.
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    for (int it0 = 0; it0 < steps; it0 += GR_BATCH) {
        if (steps > GR_BATCH) {
#pragma unroll
            for (int j = 0; j < GR_BATCH; ++j) {
                const int i = beg + (it0 + j) * 64 + lane;
                ev[j] = i < end ? ids[i] : -1;
            }
        }
#pragma unroll
        for (int j = 0; j < GR_BATCH; ++j) {
            const int i = beg + (it0 + j) * 64 + lane;
            const int e = (ev[j] >= 0 && ev[j] < E) ? ev[j] : -1;
            unsigned long long same = __ballot(e >= 0);
            if (e < 0)
                same = 0;
#pragma unroll
            for (int b = 0; b < 9; ++b) {
                const unsigned long long bits = __ballot(e >= 0 && ((e >> b) & 1));
                same &= ((e >> b) & 1) ? bits : ~bits;
            }
            if (e >= 0) {
                const int rank = __popcll(same & lt_mask);
                const int cur = hist[wave][e];
                slots[cur + rank] = i;
                if ((same >> lane) == 1ull)   // highest lane of its group
                    hist[wave][e] = cur + __popcll(same);
            }
        }
    }
}

// The same grouping over many workgroups, for prefill-sized T (bitwise the
// same outputs): 1024-slot blocks count their experts in LDS
// (group_count_kernel), then place their slots stably (group_place_kernel).
constexpr int GS_BATCH = 40;    // per-block counts one scan thread loads at once (T = 2048: one round)

__global__ __launch_bounds__(GB_SLOTS) void group_count_kernel(const int32_t *__restrict__ ids,
                                                               int N, int32_t *__restrict__ gcount)
{
    __shared__ int hist[E];
    const int tid = threadIdx.x, b = blockIdx.x;
    for (int i = tid; i < E; i += GB_SLOTS)
        hist[i] = 0;
    __syncthreads();
    const int s = b * GB_SLOTS + tid;
    const int e = s < N ? ids[s] : -1;
    if (e >= 0 && e < E)
        atomicAdd(&hist[e], 1);
    __syncthreads();
    for (int i = tid; i < E; i += GB_SLOTS)
        gcount[(size_t)b * E + i] = hist[i];
}

// The blocks place their slots stably.  Each block first works out from the
// per-block counts (threads e < E, one expert each) its own start inside
// every expert's run and the expert totals, whose exclusive scan gives the
// offsets -- every block does the same sums, so no separate scan launch is
// needed; block 0 also writes the offsets, the active list and, with mlist
// given, the prefill work list (expert e's chunks sit at the exclusive scan
// of the chunk counts, which in ascending e is the active order).  Then each
// slot's rank among equal experts inside its wave comes from ballots over the
// id bits, plus the earlier waves' counts of that expert.
__global__ __launch_bounds__(GB_SLOTS) void group_place_kernel(
    const int32_t *__restrict__ ids, int N, int nb, const int32_t *__restrict__ gcount,
    int32_t *__restrict__ offsets, int32_t *__restrict__ active, int max_items,
    int32_t *__restrict__ mlist, int32_t *__restrict__ nitems, int32_t *__restrict__ slots)
{
    __shared__ int wc[GB_SLOTS / 64][E];   // per-wave counts of each expert
    __shared__ int start[E];               // this block's first grouped position in expert e
    __shared__ int tmp[8];
    __shared__ int tot;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, b = blockIdx.x;
    for (int i = tid; i < (GB_SLOTS / 64) * E; i += GB_SLOTS)
        (&wc[0][0])[i] = 0;
    int pre = 0, all = 0;   // expert tid's slots in the blocks before b, and in all
    if (tid < E) {
        for (int b0 = 0; b0 < nb; b0 += GS_BATCH) {   // GS_BATCH counts in flight
            int c[GS_BATCH];
#pragma unroll
            for (int j = 0; j < GS_BATCH; ++j)
                c[j] = b0 + j < nb ? gcount[(size_t)(b0 + j) * E + tid] : 0;
#pragma unroll
            for (int j = 0; j < GS_BATCH; ++j) {
                pre += b0 + j < b ? c[j] : 0;
                all += c[j];
            }
        }
    }
    const int off = block_exclusive_scan_512(all, tid, tmp, &tot);
    if (tid < E)
        start[tid] = off + pre;
    if (b == 0) {   // uniform per block
        if (tid < E)
            offsets[tid] = off;
        if (tid == 0)
            offsets[E] = tot;
        const int flag = tid < E && all > 0 ? 1 : 0;
        const int pos = block_exclusive_scan_512(flag, tid, tmp, &tot);
        if (flag)
            active[1 + pos] = tid;
        if (tid == 0)
            active[0] = tot;
        if (mlist) {
            const int nch = tid < E ? (all + PF_M - 1) / PF_M : 0;
            const int base = block_exclusive_scan_512(nch, tid, tmp, &tot);
            for (int c = 0; c < nch; ++c) {
                const int it = base + c;
                if (it < max_items)
                    reinterpret_cast<int4 *>(mlist)[it] =
                        make_int4(tid, off + c * PF_M, min(PF_M, all - c * PF_M), 0);
            }
            if (tid == 0)
                nitems[0] = min(tot, max_items);
        }
    }
    const int s = b * GB_SLOTS + tid;
    const int v = s < N ? ids[s] : -1;
    const int e = (v >= 0 && v < E) ? v : -1;
    unsigned long long same = __ballot(e >= 0);
    if (e < 0)
        same = 0;
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {
        const unsigned long long bits = __ballot(e >= 0 && ((e >> bit) & 1));
        same &= ((e >> bit) & 1) ? bits : ~bits;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    __syncthreads();   // the counts are zero; start is written
    if (e >= 0 && rank == 0)   // the first lane of each group records the group's size
        wc[wave][e] = __popcll(same);
    __syncthreads();
    if (e >= 0) {
        int before = rank;
        for (int w = 0; w < wave; ++w)
            before += wc[w][e];
        slots[start[e] + before] = s;
    }
}

// Prefill work list from a caller's grouping: one record {e, gp0, rows} per
// (active expert, 64-row chunk), in active order; offsets are clamped to the
// slots as the grouping allows (an active entry out of range adds nothing);
// nitems[0] = item count.
__global__ __launch_bounds__(512) void plan_kernel(const int32_t *__restrict__ offsets,
                                                   const int32_t *__restrict__ active,
                                                   int max_items, int nslot,
                                                   int32_t *__restrict__ mlist,
                                                   int32_t *__restrict__ nitems)
{
    __shared__ int tmp[8];
    __shared__ int tot;
    const int tid = threadIdx.x;
    const int na = active[0];
    int nch = 0, e = 0, beg = 0, n = 0;
    if (tid < na) {
        e = active[1 + tid];
        if (e >= 0 && e < E) {
            beg = min(max(offsets[e], 0), nslot);
            n = min(max(offsets[e + 1], beg), nslot) - beg;
            nch = (n + PF_M - 1) / PF_M;
        }
    }
    const int base = block_exclusive_scan_512(nch, tid, tmp, &tot);
    for (int c = 0; c < nch; ++c) {
        const int it = base + c;
        if (it < max_items)
            reinterpret_cast<int4 *>(mlist)[it] = make_int4(e, beg + c * PF_M, min(PF_M, n - c * PF_M), 0);
    }
    if (tid == 0)
        nitems[0] = min(tot, max_items);
}

hipError_t launch_group(const int32_t *ids, int T, int32_t *offsets, int32_t *slots,
                        int32_t *active, int32_t *gcount, int max_items, int32_t *mlist,
                        int32_t *nitems, hipStream_t st)
{
    if (is_decode(T) || !gcount) {
        hipLaunchKernelGGL(group_kernel, dim3(1), dim3(GR_THREADS), 0, st, ids, T, offsets, slots,
                           active);
        return hipGetLastError();
    }
    const int N = T * K, nb = (N + GB_SLOTS - 1) / GB_SLOTS;
    hipLaunchKernelGGL(group_count_kernel, dim3(nb), dim3(GB_SLOTS), 0, st, ids, N, gcount);
    hipLaunchKernelGGL(group_place_kernel, dim3(nb), dim3(GB_SLOTS), 0, st, ids, N, nb,
                       (const int32_t *)gcount, offsets, active, max_items, mlist, nitems, slots);
    return hipGetLastError();
}

hipError_t launch_plan(const int32_t *offsets, const int32_t *active, int max_items, int T,
                       int32_t *mlist, int32_t *nitems, hipStream_t st)
{
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(512), 0, st, offsets, active, max_items, T * K,
                       mlist, nitems);
    return hipGetLastError();
}

} // namespace strata
