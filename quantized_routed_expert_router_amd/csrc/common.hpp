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
// Decode experts kernel: the counter of active expert a (finished gate/up
// items) is sync[1 + SYNC_STRIDE * a], one 128-byte line per counter.
constexpr int SYNC_STRIDE = 32;

// Prefill path tiles.
constexpr int PF_M = 64;                       // tokens per M-chunk
constexpr int PF_NT_G = 128;                   // FF rows per gate/up work item
constexpr int PF_NT_D = 256;                   // output rows per down work item
constexpr int PF_NTILES_G = FF / PF_NT_G;      // 5
constexpr int PF_NTILES_D = H / PF_NT_D;       // 10

// Workspace regions (byte offsets, 256-aligned) for a call with T tokens;
// Td = T on the decode path (T <= DECODE_T_MAX) else 0, Tp the converse.
struct Ws {
    size_t xsplit;     // bf16 [Tp][3][H]    router input (prefill): x = x1 + x2 + x3 exactly
    size_t xperm;      // f16 [Tp][H]        MFMA-ordered activations (prefill)
    size_t logits;     // f32 [T][E]         logits (prefill) / raw logits (decode)
    size_t inv_rms;    // f32 [Td]
    size_t xq_dig;     // u32 [Td][40][32]   16-bit x, one 64-block per block column
    size_t xq_scale;   // f32 [Td][40]
    size_t xq_sum;     // i32 [Td][40]
    size_t offsets;    // i32 [E+1]
    size_t slots;      // i32 [T*K]
    size_t active;     // i32 [1+E]
    size_t erec;       // i32x4 [1+E]        decode work records (header + one per active expert)
    size_t ids;        // i32 [T*K]
    size_t w;          // f32 [T*K]
    size_t mlist;      // i32 [2][max items]
    size_t nitems;     // i32 [4]
    size_t hq_dig;     // u32 [Td*K][10][32] 16-bit h per 16 values (64-value blocks)
    size_t hq_scale;   // f32 [Td*K][40]
    size_t hq_sum;     // i32 [Td*K][40]
    size_t hperm;      // f16 [Tp*K][FF]     (grouped order)
    size_t out;        // f32 [T*K][H]
    size_t cdone;      // i32 [Td][H/32]      decode layer: finished slots per (token, 32 rows)
    size_t esync;      // i32 [1+32E]        decode experts: finished gate/up items per active expert (128-B apart)
    size_t gcount;     // i32 [ceil(Tp*K/256)][E] prefill grouping: per-block expert counts / starts
    size_t lraw2;      // f32 [Td][E]        lookahead: the next layer's raw logits
    size_t pred;       // i32 [Td*K]         lookahead: the next layer's predicted ids
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
    const size_t nb = H / QK, ns = FF / 16;
    L.xsplit = take(Tp * 3 * H * 2);
    L.xperm = take(Tp * H * 2);
    L.logits = take((size_t)T * E * 4);
    L.inv_rms = take(Td * 4);
    L.xq_dig = take(Td * nb * 32 * 4);
    L.xq_scale = take(Td * nb * 4);
    L.xq_sum = take(Td * nb * 4);
    L.offsets = take((E + 1) * 4);
    L.slots = take((size_t)T * K * 4);
    L.active = take((1 + E) * 4);
    L.erec = take(Td ? (size_t)(1 + E) * 16 : 0);
    L.ids = take((size_t)T * K * 4);
    L.w = take((size_t)T * K * 4);
    L.max_items = pf_max_items(T);
    L.mlist = take((size_t)2 * L.max_items * 4);
    L.nitems = take(16);
    L.hq_dig = take(Td * K * (FF / QK) * 32 * 4);
    L.hq_scale = take(Td * K * ns * 4);
    L.hq_sum = take(Td * K * ns * 4);
    L.hperm = take(Tp * K * FF * 2);
    L.out = take((size_t)T * K * H * 4);
    L.cdone = take(Td * (H / 32) * 4);
    L.esync = take(Td ? (size_t)(1 + 32 * E) * 4 : 0);
    L.gcount = take((Tp * K + 255) / 256 * E * 4);
    L.lraw2 = take(Td * E * 4);
    L.pred = take(Td * K * 4);
    L.total = o;
    return L;
}

// ---------------------------------------------------------------- device helpers
__device__ inline float half_bits_to_float(uint32_t bits)
{
    return __half2float(__ushort_as_half((unsigned short)(bits & 0xffff)));
}

__device__ inline float bf16_bits_to_float(uint32_t bits)
{
    return __uint_as_float((bits & 0xffff) << 16);
}

// ---------------------------------------------------------------- DPP lane exchange
// dpp_ctrl encodings (GCN/CDNA): quad_perm 0x00-0xFF, row_shr:n 0x110+n,
// row_mirror 0x140, row_half_mirror 0x141.  Lanes without a source get `old`.
template <int CTRL> __device__ inline int dpp_i(int v, int old = 0)
{
    return __builtin_amdgcn_update_dpp(old, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ inline float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_HMIRROR = 0x141;  // lane i <- 7 - i within each 8
constexpr int DPP_MIRROR = 0x140;   // lane i <- 15 - i within each 16
constexpr int DPP_SHR4 = 0x114;
constexpr int DPP_SHR8 = 0x118;

// Sum / max over each group of 8 lanes; every lane of the group gets the
// result, lanes of one group all computing it in the same order.
__device__ inline float sum8(float v)
{
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    return v + dpp_f<DPP_HMIRROR>(v);
}
__device__ inline float sum16(float v) { v = sum8(v); return v + dpp_f<DPP_MIRROR>(v); }
__device__ inline float max16(float v)
{
    v = fmaxf(v, dpp_f<DPP_XOR1>(v));
    v = fmaxf(v, dpp_f<DPP_XOR2>(v));
    v = fmaxf(v, dpp_f<DPP_HMIRROR>(v));
    return fmaxf(v, dpp_f<DPP_MIRROR>(v));
}
__device__ inline int isum16(int v)
{
    v += dpp_i<DPP_XOR1>(v);
    v += dpp_i<DPP_XOR2>(v);
    v += dpp_i<DPP_HMIRROR>(v);
    return v + dpp_i<DPP_MIRROR>(v);
}
// Whole-wave reductions in six DPP steps (quad xor 1, xor 2, half mirror,
// mirror, then the gfx9 row broadcasts of lanes 15 and 31 into the next rows):
// lane 63 ends with the result, which v_readlane hands to every lane.  The
// order of the operations is fixed, so equal inputs give equal bits.
template <int CTRL, int ROWS> __device__ inline float dppf_rows(float v, float old)
{
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS> __device__ inline int dppi_rows(int v, int old)
{
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
constexpr int DPP_BCAST15 = 0x142;
constexpr int DPP_BCAST31 = 0x143;

__device__ inline float wave_sum63(float v)
{
    v += dppf_rows<DPP_XOR1, 0xF>(v, 0.f);
    v += dppf_rows<DPP_XOR2, 0xF>(v, 0.f);
    v += dppf_rows<DPP_HMIRROR, 0xF>(v, 0.f);
    v += dppf_rows<DPP_MIRROR, 0xF>(v, 0.f);
    v += dppf_rows<DPP_BCAST15, 0xA>(v, 0.f);
    v += dppf_rows<DPP_BCAST31, 0xC>(v, 0.f);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ inline float wave_max63(float v)
{
    v = fmaxf(v, dppf_rows<DPP_XOR1, 0xF>(v, v));
    v = fmaxf(v, dppf_rows<DPP_XOR2, 0xF>(v, v));
    v = fmaxf(v, dppf_rows<DPP_HMIRROR, 0xF>(v, v));
    v = fmaxf(v, dppf_rows<DPP_MIRROR, 0xF>(v, v));
    v = fmaxf(v, dppf_rows<DPP_BCAST15, 0xA>(v, v));
    v = fmaxf(v, dppf_rows<DPP_BCAST31, 0xC>(v, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ inline int wave_min63(int v)
{
    v = min(v, dppi_rows<DPP_XOR1, 0xF>(v, v));
    v = min(v, dppi_rows<DPP_XOR2, 0xF>(v, v));
    v = min(v, dppi_rows<DPP_HMIRROR, 0xF>(v, v));
    v = min(v, dppi_rows<DPP_MIRROR, 0xF>(v, v));
    v = min(v, dppi_rows<DPP_BCAST15, 0xA>(v, v));
    v = min(v, dppi_rows<DPP_BCAST31, 0xC>(v, v));
    return __builtin_amdgcn_readlane(v, 63);
}
// Inclusive prefix sum over the 64 lanes (row shifts 1, 2, 3, 4, 8, then the
// row broadcasts), and the exclusive one.
__device__ inline int wave_incl_scan(int v)
{
    const int v0 = v;
    v += __builtin_amdgcn_update_dpp(0, v0, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v0, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v0, 0x113, 0xF, 0xF, true);   // row_shr:3
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xE, false);   // row_shr:4, banks 1-3
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xC, false);   // row_shr:8, banks 2-3
    v += __builtin_amdgcn_update_dpp(0, v, DPP_BCAST15, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, DPP_BCAST31, 0xC, 0xF, false);
    return v;
}

} // namespace strata
