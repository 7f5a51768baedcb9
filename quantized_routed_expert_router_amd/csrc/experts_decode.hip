// experts_decode.hip -- SwiGLU experts for decode-sized T (verify windows).
//
// The expert FFN of every routed (token, expert) pair: g = W_g x, u = W_u x,
// h = silu(g) * u, o = W_d h, on Q2_0 weights ("Strata in the source...",
// section "The byte budget, in code": gate, up and down of 2,560 x 640 in
// 18-byte blocks).  Tokens are grouped per expert first, so each active
// expert's blob is read once per call however many tokens of the window chose
// it (the window dedup of section "The plan: three destinations per expert").
//
// Both kernels are HBM streams over small work items with the next item's
// bytes prefetched into registers while the current one is computed:
//  dec_gateup  item = (active expert, 16-row FF slice): 16 gate rows and the
//              same 16 up rows (23 KB) staged in LDS; 320 threads = 5 waves,
//              wave w owns block columns 8w..8w+7 for 8 rows per pass; a
//              block is 32 v_dot8_i32_i4 against the token's 16-bit
//              activations; rows are reduced with DPP in fixed order, then
//              h = silu(g) * u is quantised per 16 values for the down pass.
//  dec_down    item = (active expert, 32 output rows): 320 threads = 32 rows
//              x 10 block columns; writes the unweighted output per slot.
// Workgroups take contiguous item ranges, so consecutive items of one
// workgroup belong to the same expert.  Every reduction has a fixed order:
// results are bitwise reproducible and independent of the other tokens.
#include "common.hpp"
#include "quant.hpp"

namespace strata {

constexpr int DG_THREADS = 320;
constexpr int DG_SLICE = 16;                       // FF rows per item
constexpr int DG_SLICES = FF / DG_SLICE;           // 40
constexpr int DG_ROWS = 2 * DG_SLICE;              // 16 gate + 16 up rows
constexpr int DG_BYTES = DG_ROWS * ROW_G;          // 23,040
constexpr int DG_CHUNKS = DG_BYTES / 16;           // 1,440
constexpr int DG_LOADS = (DG_CHUNKS + DG_THREADS - 1) / DG_THREADS;   // 5

struct ExpertRange {
    int ok, e, beg, ntok;
};

__device__ inline ExpertRange expert_of(int a, const int32_t *offsets, const int32_t *active,
                                        int nslot)
{
    ExpertRange r{0, 0, 0, 0};
    const int e = active[1 + a];
    if (e < 0 || e >= E)
        return r;
    r.ok = 1;
    r.e = e;
    r.beg = min(max(offsets[e], 0), nslot);
    r.ntok = min(max(offsets[e + 1], r.beg), nslot) - r.beg;
    return r;
}

// Item range [lo, hi) of workgroup b out of G over n items.
__device__ inline void item_range(int n, int b, int G, int &lo, int &hi)
{
    lo = (int)(((long long)n * b) / G);
    hi = (int)(((long long)n * (b + 1)) / G);
}

__global__ __launch_bounds__(DG_THREADS) void dec_gateup(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ slots, const int32_t *__restrict__ active, XQ xq, HQ hq, int T)
{
    __shared__ __attribute__((aligned(16))) uint8_t wlds[DG_BYTES];
    __shared__ float red[5][DG_ROWS];
    __shared__ float gu[DG_ROWS];

    const int nslot = T * K;
    const int na = min(max(active[0], 0), min(nslot, E));
    int lo, hi;
    item_range(na * DG_SLICES, blockIdx.x, gridDim.x, lo, hi);
    if (lo >= hi)
        return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c = 8 * wave + (lane & 7);   // block column
    const int r = lane >> 3;               // row within a pass
    const BlockCol bc = block_col(c);

    // The next item's bytes are held in p0..p4 (registers) from the moment the
    // current item is in LDS until the top of the next iteration.
    static_assert(DG_LOADS == 5 && DG_CHUNKS > 4 * DG_THREADS, "five loads per thread");
    uint4 p0, p1, p2, p3, p4 = make_uint4(0, 0, 0, 0);
    const bool has4 = tid + 4 * DG_THREADS < DG_CHUNKS;
#define STRATA_DG_LD(P, I) P = (tid + DG_THREADS * (I)) < DG_CHUNKS / 2 ? g_[tid + DG_THREADS * (I)] \
                                : u_[tid + DG_THREADS * (I) - DG_CHUNKS / 2];
#define STRATA_DG_FETCH(ITEM)                                                                      \
    {                                                                                              \
        const int a_ = (ITEM) / DG_SLICES, s_ = (ITEM) % DG_SLICES;                                \
        int e_ = active[1 + a_];                                                                   \
        e_ = (e_ < 0 || e_ >= E) ? 0 : e_;                                                         \
        const uint8_t *blob_ = blobs + (size_t)e_ * BLOB + (size_t)s_ * DG_SLICE * ROW_G;          \
        const uint4 *g_ = reinterpret_cast<const uint4 *>(blob_);                                  \
        const uint4 *u_ = reinterpret_cast<const uint4 *>(blob_ + MAT);                            \
        STRATA_DG_LD(p0, 0)                                                                        \
        STRATA_DG_LD(p1, 1)                                                                        \
        STRATA_DG_LD(p2, 2)                                                                        \
        STRATA_DG_LD(p3, 3)                                                                        \
        if (has4)                                                                                  \
            STRATA_DG_LD(p4, 4)                                                                    \
    }
    int cache_a = -1, slot0 = -1, d_tok = -1, qs = 0;
    ExpertRange er{0, 0, 0, 0};
    uint32_t D[BLK_DWORDS];
    float sx = 0.f;
    STRATA_DG_FETCH(lo)
    for (int item = lo; item < hi; ++item) {
        __syncthreads();   // the previous item's LDS readers are done
        uint4 *dst = reinterpret_cast<uint4 *>(wlds);
        dst[tid] = p0;
        dst[tid + DG_THREADS] = p1;
        dst[tid + 2 * DG_THREADS] = p2;
        dst[tid + 3 * DG_THREADS] = p3;
        if (has4)
            dst[tid + 4 * DG_THREADS] = p4;
        __syncthreads();
        if (item + 1 < hi)
            STRATA_DG_FETCH(item + 1)   // in flight while this item is computed

        const int a = item / DG_SLICES, s = item % DG_SLICES;
        if (a != cache_a) {   // a new expert: its slot range (kept while it lasts)
            er = expert_of(a, offsets, active, nslot);
            cache_a = a;
            slot0 = er.ok && er.ntok > 0 ? slots[er.beg] : -1;
        }
        for (int ti = 0; er.ok && ti < er.ntok; ++ti) {
            const int slot = ti == 0 ? slot0 : slots[er.beg + ti];
            if (slot < 0 || slot >= nslot)
                continue;   // only a corrupt grouping gets here; uniform per block
            const int t = slot / K;
            if (t != d_tok) {   // the token's activation block c, kept across items
                const uint4 *dsrc = reinterpret_cast<const uint4 *>(
                    xq.dig + ((size_t)t * XBLK + c) * BLK_DWORDS);
#pragma unroll
                for (int i = 0; i < BLK_DWORDS / 4; ++i) {
                    const uint4 v = dsrc[i];
                    D[4 * i] = v.x;
                    D[4 * i + 1] = v.y;
                    D[4 * i + 2] = v.z;
                    D[4 * i + 3] = v.w;
                }
                sx = xq.scale[(size_t)t * XBLK + c] * xq.inv_rms[t];
                qs = xq.sum[(size_t)t * XBLK + c];
                d_tok = t;
            }
#pragma unroll
            for (int pass = 0; pass < DG_ROWS / 8; ++pass) {
                const int R = pass * 8 + r;
                uint32_t w[4];
                float d;
                lds_block(wlds + R * ROW_G, bc, w, d);
                const float part = (d * sx) * (float)block_dot64(w, D, qs);
                const float rs = sum8(part);
                if ((lane & 7) == 0)
                    red[wave][R] = rs;
            }
            __syncthreads();
            if (tid < DG_ROWS)
                gu[tid] = (((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid]) + red[4][tid];
            __syncthreads();
            if (wave == 0) {
                // lanes 0..15: h_j = silu(g_j) * u_j for j = 16 s + lane
                const int j = lane & 15;
                const float g = gu[j], u = gu[DG_SLICE + j];
                const float h = lane < 16 ? g / (1.f + expf(-g)) * u : 0.f;
                const QuantOut qo = quant_lanes<false>(h);
                const size_t seg = (size_t)slot * HSEG16 + s;
                if (lane == 12 || lane == 13) {
                    uint32_t *o = hq.dig + seg * SEG16_DWORDS + (lane - 12) * 4;
                    o[0] = qo.pk[0];
                    o[1] = qo.pk[1];
                    o[2] = qo.pk[2];
                    o[3] = qo.pk[3];
                }
                if (lane == 0) {
                    hq.scale[seg] = qo.scale;
                    hq.sum[seg] = qo.sum;
                }
            }
        }
    }
#undef STRATA_DG_FETCH
#undef STRATA_DG_LD
}

constexpr int DD_THREADS = 320;
constexpr int DD_ROWS = 32;
constexpr int DD_CHUNKS_PER_E = H / DD_ROWS;       // 80
constexpr int DD_BYTES = DD_ROWS * ROW_D;          // 5,760
constexpr int DD_CH16 = DD_BYTES / 16;             // 360
constexpr int DD_LOADS = 2;

__global__ __launch_bounds__(DD_THREADS) void dec_down(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ slots, const int32_t *__restrict__ active, HQ hq,
    float *__restrict__ out, int T)
{
    __shared__ __attribute__((aligned(16))) uint8_t wlds[DD_BYTES];
    __shared__ float red[DD_ROWS][NB_D + 1];

    const int nslot = T * K;
    const int na = min(max(active[0], 0), min(nslot, E));
    int lo, hi;
    item_range(na * DD_CHUNKS_PER_E, blockIdx.x, gridDim.x, lo, hi);
    if (lo >= hi)
        return;
    const int tid = threadIdx.x;
    const int r = tid / NB_D, c = tid % NB_D;
    const BlockCol bc = block_col(c);

    static_assert(DD_LOADS == 2 && DD_CH16 > DD_THREADS, "two loads per thread");
    uint4 p0, p1 = make_uint4(0, 0, 0, 0);
    const bool has1 = tid + DD_THREADS < DD_CH16;
#define STRATA_DD_FETCH(ITEM)                                                                      \
    {                                                                                              \
        const int a_ = (ITEM) / DD_CHUNKS_PER_E, ch_ = (ITEM) % DD_CHUNKS_PER_E;                   \
        int e_ = active[1 + a_];                                                                   \
        e_ = (e_ < 0 || e_ >= E) ? 0 : e_;                                                         \
        const uint4 *src_ = reinterpret_cast<const uint4 *>(                                       \
            blobs + (size_t)e_ * BLOB + 2 * MAT + (size_t)ch_ * DD_ROWS * ROW_D);                 \
        p0 = src_[tid];                                                                            \
        if (has1)                                                                                  \
            p1 = src_[tid + DD_THREADS];                                                           \
    }
    int cache_a = -1, slot0 = -1, d_slot = -1;
    ExpertRange er{0, 0, 0, 0};
    uint32_t D[BLK_DWORDS];
    float sh[4] = {0.f, 0.f, 0.f, 0.f};
    int qs[4] = {0, 0, 0, 0};
    STRATA_DD_FETCH(lo)
    for (int item = lo; item < hi; ++item) {
        __syncthreads();
        uint4 *dst = reinterpret_cast<uint4 *>(wlds);
        dst[tid] = p0;
        if (has1)
            dst[tid + DD_THREADS] = p1;
        __syncthreads();
        if (item + 1 < hi)
            STRATA_DD_FETCH(item + 1)

        const int a = item / DD_CHUNKS_PER_E, ch = item % DD_CHUNKS_PER_E;
        if (a != cache_a) {
            er = expert_of(a, offsets, active, nslot);
            cache_a = a;
            slot0 = er.ok && er.ntok > 0 ? slots[er.beg] : -1;
        }
        for (int ti = 0; er.ok && ti < er.ntok; ++ti) {
            const int slot = ti == 0 ? slot0 : slots[er.beg + ti];
            if (slot < 0 || slot >= nslot)
                continue;
            if (slot != d_slot) {   // the slot's h block c, kept across items
                const size_t seg0 = (size_t)slot * HSEG16 + 4 * c;
                const uint4 *dsrc = reinterpret_cast<const uint4 *>(hq.dig + seg0 * SEG16_DWORDS);
#pragma unroll
                for (int i = 0; i < BLK_DWORDS / 4; ++i) {
                    const uint4 v = dsrc[i];
                    D[4 * i] = v.x;
                    D[4 * i + 1] = v.y;
                    D[4 * i + 2] = v.z;
                    D[4 * i + 3] = v.w;
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    sh[k] = hq.scale[seg0 + k];
                    qs[k] = hq.sum[seg0 + k];
                }
                d_slot = slot;
            }
            uint32_t w[4];
            float d;
            lds_block(wlds + r * ROW_D, bc, w, d);
            red[r][c] = d * block_dot16x4(w, D, sh, qs);
            __syncthreads();
            if (tid < DD_ROWS) {
                float acc = 0.f;
#pragma unroll
                for (int cc = 0; cc < NB_D; ++cc)
                    acc += red[tid][cc];
                out[(size_t)slot * H + ch * DD_ROWS + tid] = acc;
            }
            __syncthreads();
        }
    }
#undef STRATA_DD_FETCH
}

hipError_t launch_decode_experts(const uint8_t *blobs, const int32_t *offsets,
                                 const int32_t *slots, const int32_t *active, XQ xq, HQ hq,
                                 float *out, int T, int n_cu, hipStream_t st)
{
    const int amax = T * K < E ? T * K : E;
    const int g1 = min(amax * DG_SLICES, 3 * n_cu);
    const int g2 = min(amax * DD_CHUNKS_PER_E, 4 * n_cu);
    hipLaunchKernelGGL(dec_gateup, dim3(g1), dim3(DG_THREADS), 0, st, blobs, offsets, slots,
                       active, xq, hq, T);
    hipLaunchKernelGGL(dec_down, dim3(g2), dim3(DD_THREADS), 0, st, blobs, offsets, slots, active,
                       hq, out, T);
    return hipGetLastError();
}

} // namespace strata
