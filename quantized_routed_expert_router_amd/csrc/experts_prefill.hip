// experts_prefill.hip -- SwiGLU experts for prefill chunks as grouped GEMMs on
// the gfx950 matrix cores.
//
// Grouping a chunk's tokens per expert turns each expert into a dense
// contraction X_e W^T with about T*10/512 token rows (the momoyeyu.github.io
// Strata explainer, section 提示词处理: one weight read serves every grouped
// token; the fused kernel dequantises next to the matrix math so no dequantised
// weights are written back).  Weights arrive as Q2_0 blocks ("Strata in the
// source...", "The byte budget, in code"); each weight (c - 1) * d is formed
// exactly in fp16 in registers -- (c - 1) is a small integer and d an fp16, so
// the product is exact -- and fed to v_mfma_f32_16x16x32_f16 against fp16
// activations with fp32 accumulation.
//
// Dequantisation: a code dword w holds codes 0..15 of a quarter block at bits
// 2i..2i+1.  For position p <= 4 the mask (w & 0x00030003 << 2p) OR an fp16
// exponent pattern gives, in each 16-bit half, the exact fp16 value M_p + c
// (M_p = 2^(10-2p)) for codes p and p + 8; positions 5..7 use w >> 10.  One
// packed subtract of M_p + 1 and one packed multiply by d finish two weights.
// So a lane's 16 weights cost 25 VALU ops, once per 64-token M-chunk.
//
// K order inside a 64-block: MFMA step j (0, 1) and lane group q (= lane/16)
// cover positions pi = 32 j + 8 q + s (s = 0..7), which carry input column
// 16 q + 4 j + s/2 + 8 (s % 2).  Activations are stored in that order once
// (prep kernel for x, the gate/up epilogue for h), so every A fragment is one
// 16-byte LDS read.
//
// Work items: (active expert, 64-token chunk) x N-tile.  gate/up tiles hold
// 128 FF rows of gate and the same 128 rows of up, so SiLU(g) * u happens in
// registers; down tiles hold 256 output rows.  The N-tiles of one item are
// placed on one XCD (blockIdx % 8), so its gathered rows stay in that L2.
#include "common.hpp"
#include <hip/hip_ext.h>

namespace strata {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int PF_THREADS = 256;
constexpr int XA_STRIDE = 72;                  // halfs per staged row (144 B, conflict-free)

__device__ inline uint32_t as_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }
__device__ inline half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// Eight fp16 pairs (exact (c - 1) * d) from one code dword; pair p holds codes
// p (low half) and p + 8 (high half).
__device__ inline void dequant_dword(uint32_t w, uint32_t dbits, uint32_t out[8])
{
    const half2v d2 = as_h2(dbits | (dbits << 16));
    const uint32_t w10 = w >> 10;
    const uint32_t src[8] = {w, w, w, w, w, w10, w10, w10};
    const int pos[8] = {0, 1, 2, 3, 4, 0, 1, 2};
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int q = pos[p];
        const uint32_t mag = (uint32_t)(25 - 2 * q) << 10;
        const uint32_t u = (src[p] & (0x00030003u << (2 * q))) | (mag | (mag << 16));
        const _Float16 m1 = (_Float16)(float)((1 << (10 - 2 * q)) + 1);
        const half2v cm1 = as_h2(u) - (half2v){m1, m1};
        out[p] = as_u32(cm1 * d2);
    }
}

// K-order position of input column c (0..63) inside its block.
__device__ inline int pf_pos_of_col(int c)
{
    const int q = c >> 4, r16 = c & 15;
    const int p = r16 & 7, hb = r16 >> 3;
    return 32 * (p >> 2) + 8 * q + 2 * (p & 3) + hb;
}

// One (item, N-tile) of a grouped GEMM: acc[ns][mi] += A(64 x K) W(K x 64)
// for the wave's four 16-column subtiles.  rowp[ns] points at this lane's
// weight row for subtile ns; NBLK blocks of ROWB-byte rows along K.
template <int NBLK>
__device__ inline void pf_mainloop(const uint8_t *const rowp[4], const __half *arow,
                                   bool arow_ok, int n_msub, __half *xa, floatx4 acc[4][4])
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int q = lane >> 4;
    const int am = tid >> 2, apart = tid & 3;   // staging: row am, 16 halfs at 16*apart
    for (int b = 0; b < NBLK; ++b) {
        // Weights for this block: scale and this lane's code dword per subtile.
        uint32_t dbits[4], wc[4];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
            const uint16_t *p16 = reinterpret_cast<const uint16_t *>(rowp[ns] + BB * b);
            dbits[ns] = p16[0];
            wc[ns] = (uint32_t)p16[1 + 2 * q] | ((uint32_t)p16[2 + 2 * q] << 16);
        }
        // Activations for this block: 64 rows x 64 halfs.
        uint4 av0 = make_uint4(0, 0, 0, 0), av1 = av0;
        if (arow_ok) {
            const uint4 *src = reinterpret_cast<const uint4 *>(arow + QK * b + 16 * apart);
            av0 = src[0];
            av1 = src[1];
        }
        __syncthreads();
        uint4 *dst = reinterpret_cast<uint4 *>(xa + am * XA_STRIDE + 16 * apart);
        dst[0] = av0;
        dst[1] = av1;
        __syncthreads();
        half8 bf[4][2];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
            uint32_t pr[8];
            dequant_dword(wc[ns], dbits[ns], pr);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint4 v = make_uint4(pr[4 * j], pr[4 * j + 1], pr[4 * j + 2], pr[4 * j + 3]);
                bf[ns][j] = __builtin_bit_cast(half8, v);
            }
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi >= n_msub)
                break;
            const __half *ap = xa + (16 * mi + (lane & 15)) * XA_STRIDE + 8 * q;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const half8 af = *reinterpret_cast<const half8 *>(ap + 32 * j);
#pragma unroll
                for (int ns = 0; ns < 4; ++ns)
                    acc[ns][mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[ns][j],
                                                                          acc[ns][mi], 0, 0, 0);
            }
        }
    }
}

struct PfItem {
    int ok, e, gp0, rows;
};

__device__ inline PfItem pf_item(int item, const int32_t *mlist, const int32_t *nitems,
                                 const int32_t *offsets, const int32_t *active, int T)
{
    PfItem it{0, 0, 0, 0};
    if (item >= nitems[0])
        return it;
    const int a = mlist[2 * item], m0 = mlist[2 * item + 1];
    if (a < 0 || a >= active[0])
        return it;
    const int e = active[1 + a];
    if (e < 0 || e >= E)
        return it;
    const int nslot = T * K;
    const int beg = min(max(offsets[e], 0), nslot);
    const int end = min(max(offsets[e + 1], beg), nslot);
    const int rows = min(PF_M, end - beg - m0);
    if (rows <= 0)
        return it;
    it.ok = 1;
    it.e = e;
    it.gp0 = beg + m0;
    it.rows = rows;
    return it;
}

__global__ __launch_bounds__(PF_THREADS) void pf_gateup(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ slots, const int32_t *__restrict__ active,
    const int32_t *__restrict__ mlist, const int32_t *__restrict__ nitems,
    const __half *__restrict__ xperm, __half *__restrict__ hperm, int T)
{
    __shared__ __attribute__((aligned(16))) __half xa[PF_M * XA_STRIDE];
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int item = 8 * (idx / PF_NTILES_G) + xcd;
    const int nt = idx % PF_NTILES_G;
    const PfItem it = pf_item(item, mlist, nitems, offsets, active, T);
    if (!it.ok)
        return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int jw = nt * PF_NT_G + 32 * wave;   // this wave's first FF row
    const uint8_t *blob = blobs + (size_t)it.e * BLOB;
    const uint8_t *rowp[4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
        rowp[ns] = blob + (ns >= 2 ? MAT : 0) + (size_t)(jw + 16 * (ns & 1) + (lane & 15)) * ROW_G;
    // Staged activation row of this thread.
    const int am = tid >> 2;
    const bool aok = am < it.rows;
    int at = 0;
    if (aok) {
        const int s = slots[it.gp0 + am];
        at = (s >= 0 && s < T * K) ? s / K : 0;
    }
    const __half *arow = xperm + (size_t)at * H;
    const int n_msub = (it.rows + 15) >> 4;
    floatx4 acc[4][4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            acc[ns][mi] = (floatx4){0.f, 0.f, 0.f, 0.f};
    pf_mainloop<NB_G>(rowp, arow, aok, n_msub, xa, acc);
    // Epilogue: h = silu(g) * u for FF rows jw + 16 h2 + lane%16.
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        const int j = jw + 16 * h2 + (lane & 15);
        const int col = QK * (j >> 6) + pf_pos_of_col(j & 63);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * mi + 4 * (lane >> 4) + r;
                if (m < it.rows) {
                    const float g = acc[h2][mi][r];
                    const float u = acc[2 + h2][mi][r];
                    const float h = g / (1.f + expf(-g)) * u;
                    hperm[(size_t)(it.gp0 + m) * FF + col] = __float2half_rn(h);
                }
            }
        }
    }
}

__global__ __launch_bounds__(PF_THREADS) void pf_down(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ slots, const int32_t *__restrict__ active,
    const int32_t *__restrict__ mlist, const int32_t *__restrict__ nitems,
    const __half *__restrict__ hperm, float *__restrict__ out, int T)
{
    __shared__ __attribute__((aligned(16))) __half xa[PF_M * XA_STRIDE];
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int item = 8 * (idx / PF_NTILES_D) + xcd;
    const int nt = idx % PF_NTILES_D;
    const PfItem it = pf_item(item, mlist, nitems, offsets, active, T);
    if (!it.ok)
        return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rw = nt * PF_NT_D + 64 * wave;   // this wave's first output row
    const uint8_t *dmat = blobs + (size_t)it.e * BLOB + 2 * MAT;
    const uint8_t *rowp[4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
        rowp[ns] = dmat + (size_t)(rw + 16 * ns + (lane & 15)) * ROW_D;
    const int am = tid >> 2;
    const bool aok = am < it.rows;
    const __half *arow = hperm + (size_t)(it.gp0 + (aok ? am : 0)) * FF;
    const int n_msub = (it.rows + 15) >> 4;
    floatx4 acc[4][4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            acc[ns][mi] = (floatx4){0.f, 0.f, 0.f, 0.f};
    pf_mainloop<NB_D>(rowp, arow, aok, n_msub, xa, acc);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * mi + 4 * (lane >> 4) + r;
            if (m < it.rows) {
                const int s = slots[it.gp0 + m];
                if (s >= 0 && s < T * K) {
#pragma unroll
                    for (int ns = 0; ns < 4; ++ns)
                        out[(size_t)s * H + rw + 16 * ns + (lane & 15)] = acc[ns][mi][r];
                }
            }
        }
    }
}

hipError_t launch_prefill_experts(const uint8_t *blobs, const int32_t *offsets,
                                  const int32_t *slots, const int32_t *active,
                                  const int32_t *mlist, const int32_t *nitems, int max_items,
                                  const __half *xperm, __half *hperm, float *out, int T,
                                  hipEvent_t ev0, hipEvent_t ev1, hipStream_t st)
{
    const int groups = (max_items + 7) / 8;
    const dim3 grid_g(8 * PF_NTILES_G * groups), block(PF_THREADS);
    if (ev0) {   // timed launch: the events carry the dispatch's own start and end
        void *args[] = {&blobs, &offsets, &slots, &active, &mlist, &nitems, &xperm, &hperm, &T};
        const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(&pf_gateup), grid_g,
                                                block, args, 0, st, ev0, ev1, 0);
        if (e != hipSuccess)
            return e;
    } else {
        hipLaunchKernelGGL(pf_gateup, grid_g, block, 0, st, blobs, offsets, slots, active, mlist,
                           nitems, xperm, hperm, T);
    }
    hipLaunchKernelGGL(pf_down, dim3(8 * PF_NTILES_D * groups), dim3(PF_THREADS), 0, st, blobs,
                       offsets, slots, active, mlist, nitems, hperm, out, T);
    return hipGetLastError();
}

} // namespace strata
