// experts_prefill_i8.hip -- the integer variant of the prefill experts
// (STRATA_INT8): 2-bit codes times int8 activations on the gfx950 int8
// matrix cores, the arithmetic of the pages' CPU kernel ("Strata in the
// source...", section "The CPU kernels": codes against int8 activations with
// the code offset removed by a correction term, and h requantised before
// down) moved onto v_mfma_i32_16x16x64_i8.
//
// Activations (x for gate/up, h for down) are int8 per 64-value block: for
// block b of a row, s = max |v| / 127 and q = rint(v / s), with
// n = -(sum of q over the block) stored beside.  Weights enter as their raw
// codes c in 0..3.  One MFMA multiplies a whole Q2_0 block (K = 64) of 16
// rows by 16 columns, starting from C = n, so its int32 result is
// sum (c - 1) q exactly; the block's contribution d * s * that is added in
// fp32.  Per block and 16 x 16 tile that is one MFMA and twelve VALU ops,
// against two fp16 MFMAs and shared dequantisation in experts_prefill.hip.
//
// K order inside a block: lane group g (= lane / 16) of an MFMA fragment
// holds K positions 16 g .. 16 g + 15.  For the weights, those are code dword
// g of the block split into four bytes-of-codes dwords v_k = (w >> 2k) &
// 0x03030303, whose byte i holds code 16 g + 4 i + k; so fragment byte p is
// code 16 g + 4 (p % 4) + p / 4, and the activations are stored in the same
// order (position 16 g + p holds value 16 g + 4 (p % 4) + p / 4).
//
// Kernels:
//  prep_i8_kernel  one workgroup per token: optional RMSNorm, int8 blocks.
//  pq_gateup       (active expert, 64-token chunk) x 64 FF rows: gate and up
//                  (wave w: rows 16 w .. 16 w + 15 of each), K in groups of
//                  four blocks staged in LDS (activations as stored; weights
//                  as 16 aligned code bytes and an fp32 scale per block);
//                  epilogue h = silu(g) u, requantised to int8 over the
//                  64 FF rows (one h block).
//  pq_down         (active expert, 64-token chunk) x 128 output rows, K = 640
//                  in two groups of five blocks; per-slot fp32 rows out.
// Every sum has a fixed order, so results are bitwise reproducible and do not
// depend on the other tokens of the call.
#include "common.hpp"
#include <hip/hip_ext.h>

namespace strata {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int PQ_THREADS = 256;
constexpr int PQ_NT_G = 64;                       // FF rows per gate/up work item
constexpr int PQ_NTILES_G = FF / PQ_NT_G;         // 10 (= the h blocks of a slot)
constexpr int PQ_NT_D = 128;                      // output rows per down work item
constexpr int PQ_NTILES_D = H / PQ_NT_D;          // 20
constexpr int PQ_GB = 4;                          // blocks per gate/up K group
constexpr int PQ_GG = NB_G / PQ_GB;               // 10 groups
constexpr int PQ_DB = 5;                          // blocks per down K group
constexpr int PQ_DG = NB_D / PQ_DB;               // 2 groups
static_assert(PQ_GG * PQ_GB == NB_G && PQ_DG * PQ_DB == NB_D, "whole groups");

// Position of value e (0..63) of a block in the stored order.
__host__ __device__ constexpr int pq_pos(int e)
{
    return 16 * (e >> 4) + 4 * (e & 3) + ((e >> 2) & 3);
}

// ------------------------------------------------------------------ activations
// x8 [T][H] int8 (stored order), xs [T][40] block scales, xn [T][40] -(sum q).
__global__ __launch_bounds__(PQ_THREADS) void prep_i8_kernel(const float *__restrict__ x,
                                                             int rmsnorm, int8_t *__restrict__ x8,
                                                             float *__restrict__ xs,
                                                             int32_t *__restrict__ xn)
{
    __shared__ float wsum[PQ_THREADS / 64];
    const int t = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const float *xt = x + (size_t)t * H;
    float inv = 1.f;
    if (rmsnorm) {
        float ss = 0.f;
        for (int i = tid; i < H; i += PQ_THREADS)
            ss = fmaf(xt[i], xt[i], ss);
        ss = wave_sum63(ss);
        if (lane == 0)
            wsum[wave] = ss;
        __syncthreads();
        const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
        inv = 1.f / sqrtf(tot / (float)H + 1e-6f);
    }
    for (int b = wave; b < NB_G; b += PQ_THREADS / 64) {
        const float v = xt[QK * b + lane] * inv;
        const float m = wave_max63(fabsf(v));
        const float r = m > 0.f ? 127.f / m : 0.f;
        const int q = max(-127, min(127, (int)rintf(v * r)));
        const int sq = (int)wave_sum63((float)q);   // |sum| <= 8128: exact in fp32
        x8[(size_t)t * H + QK * b + pq_pos(lane)] = (int8_t)q;
        if (lane == 0) {
            xs[(size_t)t * NB_G + b] = m / 127.f;
            xn[(size_t)t * NB_G + b] = -sq;
        }
    }
}

// ------------------------------------------------------------------ shared pieces
struct PqItem {
    int ok, e, gp0, rows;
};

// Work item `item` from the planner's record (as the fp16 kernels read it).
__device__ inline PqItem pq_item(int item, const int32_t *mlist, const int32_t *nitems, int T)
{
    PqItem it{0, 0, 0, 0};
    const int4 r = reinterpret_cast<const int4 *>(mlist)[item];   // padded: always in bounds
    if (item >= nitems[0] || !pf_rec_ok(r.x, r.y, r.z, T))
        return it;
    it.ok = 1;
    it.e = r.x;
    it.gp0 = r.y;
    it.rows = r.z;
    return it;
}

// The 16 code bytes and the scale of the 18-byte block at byte offset `off`
// of `base` (which is 4-byte aligned): loaded as the five dwords from the one
// at or below the block's start.
__device__ inline void pq_block(const uint8_t *base, uint32_t off, uint4 &codes, float &d)
{
    const uint32_t *p = reinterpret_cast<const uint32_t *>(base + (off & ~3u));
    const uint32_t w0 = p[0], w1 = p[1], w2 = p[2], w3 = p[3], w4 = p[4];
    if (off & 2u) {   // the block starts 2 bytes into w0
        d = half_bits_to_float(w0 >> 16);
        codes = make_uint4(w1, w2, w3, w4);
    } else {
        d = half_bits_to_float(w0);
        const uint32_t sel = 0x05040302u;
        codes = make_uint4(__builtin_amdgcn_perm(w1, w0, sel), __builtin_amdgcn_perm(w2, w1, sel),
                           __builtin_amdgcn_perm(w3, w2, sel), __builtin_amdgcn_perm(w4, w3, sel));
    }
}

// The B fragment of code dword w: v_k = (w >> 2k) & 0x03030303.
__device__ inline i32x4 pq_codes(uint32_t w)
{
    return (i32x4){(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u),
                   (int)((w >> 4) & 0x03030303u), (int)((w >> 6) & 0x03030303u)};
}

// acc += d s (float)P for the four rows of a lane in a tile.
__device__ inline void pq_accum(f32x4 &acc, i32x4 P, float d, f32x4 s)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc[i] = fmaf((float)P[i], d * s[i], acc[i]);
}

__device__ inline float pq_silu_mul(float g, float u)
{
    return g * u / (1.f + expf(-g));
}

// ------------------------------------------------------------------ gate / up
// LDS of one K group: activations [64 rows][68 dwords] (256 bytes used, the
// pad spreads rows over banks), weight codes [128 rows][17 dwords] (16 used),
// weight scales [128][4], activation scales and -(sum q) [4][64].
constexpr int PQ_AS = 68;
constexpr int PQ_BS = PQ_GB * 4 + 1;
struct PqGLds {
    uint32_t a[PF_M * PQ_AS];
    uint32_t bc[2 * PQ_NT_G * PQ_BS];
    float bd[2 * PQ_NT_G * PQ_GB];
    float xs[PQ_GB * PF_M];
    int32_t xn[PQ_GB * PF_M];
    int32_t tok[PF_M];
    float hmax[PQ_THREADS / 64][PF_M];
    int32_t hsum[PQ_THREADS / 64][PF_M];
};

template <int MS>
__device__ inline void pq_gateup_group(const PqGLds &L, int wave, int q, int n, f32x4 acc[2][4])
{
#pragma unroll
    for (int j = 0; j < PQ_GB; ++j) {
        i32x4 bf[2];
        float d[2];
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const int row = PQ_NT_G * ns + 16 * wave + n;   // gate rows, then up rows
            bf[ns] = pq_codes(L.bc[row * PQ_BS + 4 * j + q]);
            d[ns] = L.bd[row * PQ_GB + j];
        }
#pragma unroll
        for (int mi = 0; mi < MS; ++mi) {
            const i32x4 af = *reinterpret_cast<const i32x4 *>(&L.a[(16 * mi + n) * PQ_AS + 16 * j + 4 * q]);
            const i32x4 c0 = *reinterpret_cast<const i32x4 *>(&L.xn[j * PF_M + 16 * mi + 4 * q]);
            const f32x4 s = *reinterpret_cast<const f32x4 *>(&L.xs[j * PF_M + 16 * mi + 4 * q]);
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const i32x4 P = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[ns], c0, 0, 0, 0);
                pq_accum(acc[ns][mi], P, d[ns], s);
            }
        }
    }
}

__global__ __launch_bounds__(PQ_THREADS) void pq_gateup(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ slots,
    const int32_t *__restrict__ mlist, const int32_t *__restrict__ nitems,
    const int8_t *__restrict__ x8, const float *__restrict__ xs8, const int32_t *__restrict__ xn8,
    int8_t *__restrict__ h8, float *__restrict__ hs8, int32_t *__restrict__ hn8, int T)
{
    __shared__ __attribute__((aligned(16))) PqGLds L;
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int item = 8 * (idx / PQ_NTILES_G) + xcd;
    const int nt = idx % PQ_NTILES_G;
    const PqItem it = pq_item(item, mlist, nitems, T);
    if (!it.ok)
        return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = lane >> 4, n = lane & 15;
    if (tid < PF_M) {   // the token of each item row (rows past the end: the first row's)
        const int sl = slots[it.gp0 + (tid < it.rows ? tid : 0)];
        L.tok[tid] = (sl >= 0 && sl < T * K) ? sl / K : 0;
    }
    __syncthreads();
    const uint8_t *blob = blobs + (size_t)it.e * BLOB;
    f32x4 acc[2][4];
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            acc[ns][mi] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int ms = (it.rows + 15) >> 4;
    for (int g = 0; g < PQ_GG; ++g) {
        // activations: 64 rows x 256 bytes, four 16-byte chunks per thread
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + PQ_THREADS * i, m = c >> 4, k16 = c & 15;
            const uint4 v = *reinterpret_cast<const uint4 *>(x8 + (size_t)L.tok[m] * H +
                                                             PQ_GB * QK * g + 16 * k16);
            *reinterpret_cast<uint4 *>(&L.a[m * PQ_AS + 4 * k16]) = v;
        }
        // weights: 128 rows x 4 blocks, two (row, block) pairs per thread
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = tid + PQ_THREADS * i, row = p >> 2, j = p & 3;
            const uint32_t ffrow = nt * PQ_NT_G + (row & (PQ_NT_G - 1));
            const uint32_t off = (row >= PQ_NT_G ? (uint32_t)MAT : 0u) + ffrow * ROW_G +
                                 BB * (PQ_GB * g + j);
            uint4 cw;
            float d;
            pq_block(blob, off, cw, d);
            uint32_t *dst = &L.bc[row * PQ_BS + 4 * j];
            dst[0] = cw.x;
            dst[1] = cw.y;
            dst[2] = cw.z;
            dst[3] = cw.w;
            L.bd[row * PQ_GB + j] = d;
        }
        {   // activation scales and -(sum q): thread = (block j, row m)
            const int j = tid >> 6, m = tid & 63;
            const size_t src = (size_t)L.tok[m] * NB_G + PQ_GB * g + j;
            L.xs[j * PF_M + m] = xs8[src];
            L.xn[j * PF_M + m] = xn8[src];
        }
        __syncthreads();
        switch (ms) {
        case 1:
            pq_gateup_group<1>(L, wave, q, n, acc);
            break;
        case 2:
            pq_gateup_group<2>(L, wave, q, n, acc);
            break;
        case 3:
            pq_gateup_group<3>(L, wave, q, n, acc);
            break;
        default:
            pq_gateup_group<4>(L, wave, q, n, acc);
            break;
        }
        __syncthreads();
    }
    // Epilogue: h = silu(g) u for FF column 16 wave + n of the item's h block
    // nt, rows m = 16 mi + 4 q + i; requantised over the block's 64 columns.
    float h[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            h[mi][i] = pq_silu_mul(acc[0][mi][i], acc[1][mi][i]);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float m16 = max16(fabsf(h[mi][i]));   // over the wave's 16 columns
            if (n == 0)
                L.hmax[wave][16 * mi + 4 * q + i] = m16;
        }
    __syncthreads();
    int qh[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * mi + 4 * q + i;
            const float mx = fmaxf(fmaxf(L.hmax[0][m], L.hmax[1][m]), fmaxf(L.hmax[2][m], L.hmax[3][m]));
            const float r = mx > 0.f ? 127.f / mx : 0.f;
            qh[mi][i] = max(-127, min(127, (int)rintf(h[mi][i] * r)));
            const int s16 = isum16(qh[mi][i]);
            if (n == 0)
                L.hsum[wave][m] = s16;
        }
    __syncthreads();
    const int col = pq_pos(16 * wave + n);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * mi + 4 * q + i;
            if (m < it.rows) {
                const size_t gp = (size_t)(it.gp0 + m);
                h8[gp * FF + PQ_NT_G * nt + col] = (int8_t)qh[mi][i];
                if (wave == 0 && n == 0) {
                    const float mx = fmaxf(fmaxf(L.hmax[0][m], L.hmax[1][m]),
                                           fmaxf(L.hmax[2][m], L.hmax[3][m]));
                    hs8[gp * PQ_NTILES_G + nt] = mx / 127.f;
                    hn8[gp * PQ_NTILES_G + nt] =
                        -((L.hsum[0][m] + L.hsum[1][m]) + (L.hsum[2][m] + L.hsum[3][m]));
                }
            }
        }
}

// ----------------------------------------------------------------------- down
constexpr int PQ_DAS = PQ_DB * 16 + 4;            // 84 dwords per activation row (80 used)
constexpr int PQ_DBS = PQ_DB * 4 + 1;             // 21 dwords per weight row (20 used)
struct PqDLds {
    uint32_t a[PF_M * PQ_DAS];
    uint32_t bc[PQ_NT_D * PQ_DBS];
    float bd[PQ_NT_D * PQ_DB];
    float hs[PQ_DB * PF_M];
    int32_t hn[PQ_DB * PF_M];
};

template <int MS>
__device__ inline void pq_down_group(const PqDLds &L, int wave, int q, int n, f32x4 acc[2][4])
{
#pragma unroll
    for (int j = 0; j < PQ_DB; ++j) {
        i32x4 bf[2];
        float d[2];
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const int row = 32 * wave + 16 * ns + n;
            bf[ns] = pq_codes(L.bc[row * PQ_DBS + 4 * j + q]);
            d[ns] = L.bd[row * PQ_DB + j];
        }
#pragma unroll
        for (int mi = 0; mi < MS; ++mi) {
            const i32x4 af = *reinterpret_cast<const i32x4 *>(&L.a[(16 * mi + n) * PQ_DAS + 16 * j + 4 * q]);
            const i32x4 c0 = *reinterpret_cast<const i32x4 *>(&L.hn[j * PF_M + 16 * mi + 4 * q]);
            const f32x4 s = *reinterpret_cast<const f32x4 *>(&L.hs[j * PF_M + 16 * mi + 4 * q]);
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const i32x4 P = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[ns], c0, 0, 0, 0);
                pq_accum(acc[ns][mi], P, d[ns], s);
            }
        }
    }
}

__global__ __launch_bounds__(PQ_THREADS) void pq_down(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ slots,
    const int32_t *__restrict__ mlist, const int32_t *__restrict__ nitems,
    const int8_t *__restrict__ h8, const float *__restrict__ hs8, const int32_t *__restrict__ hn8,
    float *__restrict__ out, int T)
{
    __shared__ __attribute__((aligned(16))) PqDLds L;
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int item = 8 * (idx / PQ_NTILES_D) + xcd;
    const int nt = idx % PQ_NTILES_D;
    const PqItem it = pq_item(item, mlist, nitems, T);
    if (!it.ok)
        return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = lane >> 4, n = lane & 15;
    const uint8_t *dmat = blobs + (size_t)it.e * BLOB + 2 * MAT;
    f32x4 acc[2][4];
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            acc[ns][mi] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int ms = (it.rows + 15) >> 4;
    for (int g = 0; g < PQ_DG; ++g) {
        // h rows (grouped order; rows past the end read the first row): 64 x
        // 320 bytes, five 16-byte chunks per thread
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int c = tid + PQ_THREADS * i, m = c / 20, k16 = c % 20;
            const int gp = it.gp0 + (m < it.rows ? m : 0);
            const uint4 v = *reinterpret_cast<const uint4 *>(h8 + (size_t)gp * FF + PQ_DB * QK * g +
                                                             16 * k16);
            *reinterpret_cast<uint4 *>(&L.a[m * PQ_DAS + 4 * k16]) = v;
        }
        // down rows: 128 x 5 blocks, (row, block) pairs p = tid + 256 i < 640
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int p = tid + PQ_THREADS * i;
            if (p < PQ_NT_D * PQ_DB) {
                const int row = p / PQ_DB, j = p % PQ_DB;
                const uint32_t off = (uint32_t)(nt * PQ_NT_D + row) * ROW_D + BB * (PQ_DB * g + j);
                uint4 cw;
                float d;
                pq_block(dmat, off, cw, d);
                uint32_t *dst = &L.bc[row * PQ_DBS + 4 * j];
                dst[0] = cw.x;
                dst[1] = cw.y;
                dst[2] = cw.z;
                dst[3] = cw.w;
                L.bd[row * PQ_DB + j] = d;
            }
        }
        // h scales and -(sum q): (block j, row m) pairs, 320 of them
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = tid + PQ_THREADS * i;
            if (p < PQ_DB * PF_M) {
                const int j = p / PF_M, m = p % PF_M;
                const int gp = it.gp0 + (m < it.rows ? m : 0);
                L.hs[j * PF_M + m] = hs8[(size_t)gp * PQ_NTILES_G + PQ_DB * g + j];
                L.hn[j * PF_M + m] = hn8[(size_t)gp * PQ_NTILES_G + PQ_DB * g + j];
            }
        }
        __syncthreads();
        switch (ms) {
        case 1:
            pq_down_group<1>(L, wave, q, n, acc);
            break;
        case 2:
            pq_down_group<2>(L, wave, q, n, acc);
            break;
        case 3:
            pq_down_group<3>(L, wave, q, n, acc);
            break;
        default:
            pq_down_group<4>(L, wave, q, n, acc);
            break;
        }
        __syncthreads();
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * mi + 4 * q + i;
            if (m < it.rows) {
                const int s = slots[it.gp0 + m];
                if (s >= 0 && s < T * K) {
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns)
                        out[(size_t)s * H + nt * PQ_NT_D + 32 * wave + 16 * ns + n] = acc[ns][mi][i];
                }
            }
        }
}

hipError_t launch_prep_i8(const float *x, int T, int rmsnorm, int8_t *x8, float *xs, int32_t *xn,
                          hipStream_t st)
{
    hipLaunchKernelGGL(prep_i8_kernel, dim3(T), dim3(PQ_THREADS), 0, st, x, rmsnorm, x8, xs, xn);
    return hipGetLastError();
}

hipError_t launch_prefill_experts_i8(const uint8_t *blobs, const int32_t *offsets,
                                     const int32_t *slots, const int32_t *active,
                                     const int32_t *mlist, const int32_t *nitems, int max_items,
                                     const int8_t *x8, const float *xs8, const int32_t *xn8,
                                     int8_t *h8, float *hs8, int32_t *hn8, float *out, int T,
                                     hipEvent_t ev0, hipEvent_t ev1, hipStream_t st)
{
    const int groups = (max_items + 7) / 8;
    const dim3 grid_g(8 * PQ_NTILES_G * groups), block(PQ_THREADS);
    if (ev0) {   // timed launch: the events carry the dispatch's own start and end
        void *args[] = {&blobs, &slots, &mlist, &nitems, &x8, &xs8, &xn8, &h8, &hs8, &hn8, &T};
        const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(&pq_gateup), grid_g,
                                                block, args, 0, st, ev0, ev1, 0);
        if (e != hipSuccess)
            return e;
    } else {
        hipLaunchKernelGGL(pq_gateup, grid_g, block, 0, st, blobs, slots, mlist, nitems, x8, xs8,
                           xn8, h8, hs8, hn8, T);
    }
    hipLaunchKernelGGL(pq_down, dim3(8 * PQ_NTILES_D * groups), block, 0, st, blobs, slots,
                       mlist, nitems, h8, hs8, hn8, out, T);
    return hipGetLastError();
}

} // namespace strata
