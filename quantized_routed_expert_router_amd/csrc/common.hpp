// common.hpp -- internal constants, workspace layout and device helpers of the
// routed-expert MoE library (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stddef.h>
#include <stdint.h>

#include "strata_moe.h"

namespace strata {

constexpr int H = STRATA_MOE_H;
constexpr int FF = STRATA_MOE_FF;
constexpr int E = STRATA_MOE_E;
constexpr int K = STRATA_MOE_K;
constexpr int QK = STRATA_MOE_QK;
constexpr int BB = STRATA_MOE_BB;
constexpr size_t BLOB = STRATA_MOE_BLOB;
constexpr int T_MAX = STRATA_MOE_T_MAX;

constexpr int NB_G = H / QK;                   // 40 blocks per gate/up row
constexpr int NB_D = FF / QK;                  // 10 blocks per down row
constexpr int ROW_G = NB_G * BB;               // 720 bytes per gate/up row
constexpr int ROW_D = NB_D * BB;               // 180 bytes per down row
constexpr size_t MAT = (size_t)FF * ROW_G;     // 460,800 bytes per matrix
static_assert(3 * MAT == BLOB, "blob = gate + up + down");
static_assert((size_t)H * ROW_D == MAT, "down matrix size");

// Decode path: T up to this many tokens runs the dot-product kernels.
constexpr int DECODE_T_MAX = 16;

// 16-bit activation quantisation for the decode kernels: per 32-value segment
// a scale s = max|v| / QMAX and integers q = rint(v / s), |q| <= QMAX, stored
// as four signed base-16 digits packed for v_dot8_i32_i4 (see quant.hpp).
constexpr int SEG = 32;
constexpr int QMAX = 30000;
constexpr int SEG_DWORDS = 16;                 // 32 values x 4 digits x 4 bits
constexpr int XSEG = H / SEG;                  // 80 segments per token
constexpr int HSEG = FF / SEG;                 // 20 segments per slot

// Prefill path tiles.
constexpr int PF_M = 64;                       // tokens per M-chunk
constexpr int PF_NT_G = 128;                   // FF rows per gate/up work item
constexpr int PF_NT_D = 256;                   // output rows per down work item
constexpr int PF_NTILES_G = FF / PF_NT_G;      // 5
constexpr int PF_NTILES_D = H / PF_NT_D;       // 10

// Workspace regions (byte offsets, 256-aligned) for a call with T tokens.
struct Ws {
    size_t xhat;       // f32 [T][H]
    size_t xq_dig;     // u32 [Td][XSEG][16]
    size_t xq_scale;   // f32 [Td][XSEG]
    size_t xq_sum;     // i32 [Td][XSEG]
    size_t xperm;      // f16 [Tp][H]
    size_t logits;     // f32 [T][E]
    size_t offsets;    // i32 [E+1]
    size_t slots;      // i32 [T*K]
    size_t active;     // i32 [1+E]
    size_t ids;        // i32 [T*K]
    size_t w;          // f32 [T*K]
    size_t mlist;      // i32 [2][max items]
    size_t nitems;     // i32 [4]
    size_t hq_dig;     // u32 [Td*K][HSEG][16]
    size_t hq_scale;   // f32 [Td*K][HSEG]
    size_t hq_sum;     // i32 [Td*K][HSEG]
    size_t hperm;      // f16 [Tp*K][FF] (grouped order)
    size_t out;        // f32 [T*K][H]
    size_t total;
    int max_items;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline bool is_decode(int T) { return T <= DECODE_T_MAX; }

inline int pf_max_items(int T) { return E + (T * K + PF_M - 1) / PF_M; }

inline Ws ws_layout(int T)
{
    Ws L{};
    size_t o = 0;
    const size_t Td = is_decode(T) ? (size_t)T : 0;
    const size_t Tp = is_decode(T) ? 0 : (size_t)T;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    L.xhat = take((size_t)T * H * 4);
    L.xq_dig = take(Td * XSEG * SEG_DWORDS * 4);
    L.xq_scale = take(Td * XSEG * 4);
    L.xq_sum = take(Td * XSEG * 4);
    L.xperm = take(Tp * H * 2);
    L.logits = take((size_t)T * E * 4);
    L.offsets = take((E + 1) * 4);
    L.slots = take((size_t)T * K * 4);
    L.active = take((1 + E) * 4);
    L.ids = take((size_t)T * K * 4);
    L.w = take((size_t)T * K * 4);
    L.max_items = pf_max_items(T);
    L.mlist = take((size_t)2 * L.max_items * 4);
    L.nitems = take(16);
    L.hq_dig = take(Td * K * HSEG * SEG_DWORDS * 4);
    L.hq_scale = take(Td * K * HSEG * 4);
    L.hq_sum = take(Td * K * HSEG * 4);
    L.hperm = take(Tp * K * FF * 2);
    L.out = take((size_t)T * K * H * 4);
    L.total = o;
    return L;
}

// Quantised activations (decode path): one vector = nseg segments.
struct ActQ {
    uint32_t *dig;  // [vec][nseg][16]
    float *scale;   // [vec][nseg]
    int32_t *sum;   // [vec][nseg]
};

// ---------------------------------------------------------------- device helpers
__device__ inline float half_bits_to_float(uint32_t bits)
{
    return __half2float(__ushort_as_half((unsigned short)(bits & 0xffff)));
}

__device__ inline float bf16_bits_to_float(uint32_t bits)
{
    return __uint_as_float((bits & 0xffff) << 16);
}

// Sum over the 64 lanes of a wave with a fixed butterfly (same tree for every
// wave, so equal inputs give equal bits).
__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

__device__ inline float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

} // namespace strata
