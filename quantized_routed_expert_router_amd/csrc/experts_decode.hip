// experts_decode.hip -- SwiGLU experts for decode-sized T (verify windows).
//
// The expert FFN of every routed (token, expert) pair: g = W_g x, u = W_u x,
// h = silu(g) * u, o = W_d h, on Q2_0 weights ("Strata in the source...",
// section "The byte budget, in code": gate, up, down of 2,560 x 640 in 18-byte
// blocks).  Tokens are grouped per expert first, so every active expert's
// blob is read once per call however many tokens of the window chose it
// (the window dedup of section "The plan: three destinations per expert").
//
// Two kernels, both HBM-bound streams of the routed blobs:
//  dec_gateup  one workgroup per (active expert, 32-row FF slice): stages the
//              slice's 32 gate rows and 32 up rows (46 KB) in LDS with
//              coalesced 16-byte loads, then 320 threads = 8 rows x 40 block
//              columns dot them against the token's 16-bit activations with
//              v_dot8_i32_i4, reduce per row, apply SiLU and quantise the 32
//              h values of the slice as one segment.
//  dec_down    one workgroup per (active expert, 64 output rows): stages the
//              rows (11.5 KB), 320 threads = 32 rows x 10 block columns, and
//              writes the unweighted expert output per slot.
// Every reduction runs in a fixed order, so results are bitwise reproducible
// and a token's output does not depend on the other tokens of the window.
#include "common.hpp"
#include "quant.hpp"

namespace strata {

constexpr int DG_THREADS = 320;
constexpr int DG_ROWS = 64;                    // 32 gate + 32 up rows per slice
constexpr int DG_SLICES = FF / SEG;            // 20
constexpr int DG_LDS_W = DG_ROWS * ROW_G;      // 46,080 bytes

__global__ __launch_bounds__(DG_THREADS) void dec_gateup(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ slots, const int32_t *__restrict__ active, ActQ xq, ActQ hq,
    int T)
{
    __shared__ __attribute__((aligned(16))) uint8_t wlds[DG_LDS_W];
    __shared__ float red[DG_ROWS][NB_G + 1];
    __shared__ float gu[DG_ROWS];

    const int slice = blockIdx.x;
    const int a = blockIdx.y;
    if (a >= active[0])
        return;
    const int e = active[1 + a];
    if (e < 0 || e >= E)
        return;
    const int nslot = T * K;
    const int beg = min(max(offsets[e], 0), nslot);
    const int ntok = min(max(offsets[e + 1], beg), nslot) - beg;
    const int tid = threadIdx.x;
    const int j0 = slice * SEG;

    // Stage gate rows j0..j0+31 then up rows j0..j0+31 (two contiguous runs).
    const uint8_t *blob = blobs + (size_t)e * BLOB;
    const uint4 *g_src = reinterpret_cast<const uint4 *>(blob + (size_t)j0 * ROW_G);
    const uint4 *u_src = reinterpret_cast<const uint4 *>(blob + MAT + (size_t)j0 * ROW_G);
    constexpr int HALF16 = SEG * ROW_G / 16;   // 1,440 chunks per run
    uint4 *dst = reinterpret_cast<uint4 *>(wlds);
    uint4 tmp[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) {
        const int ch = tid + DG_THREADS * i;   // 0 .. 2,879
        tmp[i] = ch < HALF16 ? g_src[ch] : u_src[ch - HALF16];
    }
#pragma unroll
    for (int i = 0; i < 9; ++i)
        dst[tid + DG_THREADS * i] = tmp[i];
    __syncthreads();

    const int r = tid / NB_G;      // 0..7
    const int c = tid % NB_G;      // block column 0..39
    const BlockCol bc = block_col(c);
    const int wave = tid >> 6, lane = tid & 63;

    for (int ti = 0; ti < ntok; ++ti) {
        const int s = slots[beg + ti];
        if (s < 0 || s >= nslot)
            continue;   // only a corrupt grouping gets here; uniform per block
        const int t = s / K;
        // The token's activation block c = segments 2c and 2c+1.
        uint32_t D[32];
        const uint4 *dsrc = reinterpret_cast<const uint4 *>(
            xq.dig + ((size_t)t * XSEG + 2 * c) * SEG_DWORDS);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint4 v = dsrc[i];
            D[4 * i] = v.x;
            D[4 * i + 1] = v.y;
            D[4 * i + 2] = v.z;
            D[4 * i + 3] = v.w;
        }
        const float s0 = xq.scale[(size_t)t * XSEG + 2 * c];
        const float s1 = xq.scale[(size_t)t * XSEG + 2 * c + 1];
        const int q0 = xq.sum[(size_t)t * XSEG + 2 * c];
        const int q1 = xq.sum[(size_t)t * XSEG + 2 * c + 1];
#pragma unroll 2
        for (int rt = 0; rt < DG_ROWS / 8; ++rt) {
            const int R = rt * 8 + r;
            uint32_t w[4];
            float d;
            lds_block(wlds + R * ROW_G, bc, w, d);
            red[R][c] = block_partial(w, d, D, s0, s1, q0, q1);
        }
        __syncthreads();
        if (tid < DG_ROWS) {
            float acc = 0.f;
#pragma unroll 8
            for (int cc = 0; cc < NB_G; ++cc)
                acc += red[tid][cc];
            gu[tid] = acc;
        }
        __syncthreads();
        if (wave == 0) {
            // Lanes 0..31: h_j = silu(g_j) * u_j for j = j0 + lane; the other
            // half-wave quantises a dummy segment so every lane takes part.
            const int l32 = lane & 31;
            float h = 0.f;
            if (lane < 32) {
                const float g = gu[l32];
                const float u = gu[SEG + l32];
                h = g / (1.f + expf(-g)) * u;
            }
            const size_t seg = (size_t)s * HSEG + slice;
            quant_seg32(h, l32, lane < 32, hq.dig + seg * SEG_DWORDS, hq.scale + seg,
                        hq.sum + seg);
        }
        // red and gu are rewritten by the next token only after every thread
        // has passed this barrier.
        __syncthreads();
    }
}

constexpr int DD_THREADS = 320;
constexpr int DD_ROWS = 64;
constexpr int DD_CHUNKS = H / DD_ROWS;         // 40
constexpr int DD_LDS_W = DD_ROWS * ROW_D;      // 11,520 bytes

__global__ __launch_bounds__(DD_THREADS) void dec_down(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ slots, const int32_t *__restrict__ active, ActQ hq,
    float *__restrict__ out, int T)
{
    __shared__ __attribute__((aligned(16))) uint8_t wlds[DD_LDS_W];
    __shared__ float red[DD_ROWS][NB_D + 1];

    const int chunk = blockIdx.x;
    const int a = blockIdx.y;
    if (a >= active[0])
        return;
    const int e = active[1 + a];
    if (e < 0 || e >= E)
        return;
    const int nslot = T * K;
    const int beg = min(max(offsets[e], 0), nslot);
    const int ntok = min(max(offsets[e + 1], beg), nslot) - beg;
    const int tid = threadIdx.x;
    const int r0 = chunk * DD_ROWS;

    const uint4 *src = reinterpret_cast<const uint4 *>(blobs + (size_t)e * BLOB + 2 * MAT +
                                                       (size_t)r0 * ROW_D);
    constexpr int N16 = DD_LDS_W / 16;          // 720 chunks = 2 x 320 + 80
    static_assert(N16 > 2 * DD_THREADS && N16 <= 3 * DD_THREADS, "staging split");
    uint4 *dst = reinterpret_cast<uint4 *>(wlds);
    const bool third = tid + 2 * DD_THREADS < N16;
    const uint4 v0 = src[tid];
    const uint4 v1 = src[tid + DD_THREADS];
    const uint4 v2 = third ? src[tid + 2 * DD_THREADS] : make_uint4(0, 0, 0, 0);
    dst[tid] = v0;
    dst[tid + DD_THREADS] = v1;
    if (third)
        dst[tid + 2 * DD_THREADS] = v2;
    __syncthreads();

    const int r = tid / NB_D;      // 0..31
    const int c = tid % NB_D;      // 0..9
    const BlockCol bc = block_col(c);

    for (int ti = 0; ti < ntok; ++ti) {
        const int s = slots[beg + ti];
        if (s < 0 || s >= nslot)
            continue;
        uint32_t D[32];
        const uint4 *dsrc = reinterpret_cast<const uint4 *>(
            hq.dig + ((size_t)s * HSEG + 2 * c) * SEG_DWORDS);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint4 v = dsrc[i];
            D[4 * i] = v.x;
            D[4 * i + 1] = v.y;
            D[4 * i + 2] = v.z;
            D[4 * i + 3] = v.w;
        }
        const size_t sg = (size_t)s * HSEG + 2 * c;
        const float s0 = hq.scale[sg], s1 = hq.scale[sg + 1];
        const int q0 = hq.sum[sg], q1 = hq.sum[sg + 1];
#pragma unroll
        for (int rt = 0; rt < DD_ROWS / 32; ++rt) {
            const int R = rt * 32 + r;
            uint32_t w[4];
            float d;
            lds_block(wlds + R * ROW_D, bc, w, d);
            red[R][c] = block_partial(w, d, D, s0, s1, q0, q1);
        }
        __syncthreads();
        if (tid < DD_ROWS) {
            float acc = 0.f;
#pragma unroll
            for (int cc = 0; cc < NB_D; ++cc)
                acc += red[tid][cc];
            out[(size_t)s * H + r0 + tid] = acc;
        }
        __syncthreads();
    }
}

// Launchers (arguments validated by the caller).
hipError_t launch_decode_experts(const uint8_t *blobs, const int32_t *offsets,
                                 const int32_t *slots, const int32_t *active, ActQ xq, ActQ hq,
                                 float *out, int T, hipStream_t st)
{
    const int amax = T * K < E ? T * K : E;
    hipLaunchKernelGGL(dec_gateup, dim3(DG_SLICES, amax), dim3(DG_THREADS), 0, st, blobs,
                       offsets, slots, active, xq, hq, T);
    hipLaunchKernelGGL(dec_down, dim3(DD_CHUNKS, amax), dim3(DD_THREADS), 0, st, blobs, offsets,
                       slots, active, hq, out, T);
    return hipGetLastError();
}

} // namespace strata
