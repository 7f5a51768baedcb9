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
constexpr int GB_SLOTS = 1024;                 // slots per block of the prefill grouping
constexpr int PF_M = 64;                       // tokens per M-chunk
constexpr int PF_NT_G = 128;                   // FF rows per gate/up work item
constexpr int PF_NT_D = 256;                   // output rows per down work item
constexpr int PF_NTILES_G = FF / PF_NT_G;      // 5
constexpr int PF_NTILES_D = H / PF_NT_D;       // 10

// Layer calls for T <= ROUTED_T_MAX route every token in the gate/up launch
// (400 workgroups per token) instead of a top-k launch (measured faster up to
// three tokens).
constexpr int ROUTED_T_MAX = 3;

constexpr bool is_decode(int T) { return T <= DECODE_T_MAX; }

constexpr int pf_max_items(int T) { return E + (T * K + PF_M - 1) / PF_M; }
// A prefill work item, as the planners write it (four int32 per item):
// rows gp0 .. gp0 + rows - 1 of the grouped order, all routed to expert e,
// 1 <= rows <= PF_M.  The work list holds PF_LIST_PAD records more than items
// so that every workgroup of a grid rounded up to the 8 XCDs can load its
// record before it knows whether the record is in use.
constexpr int PF_LIST_PAD = 8;
__host__ __device__ inline bool pf_rec_ok(int e, int gp0, int rows, int T)
{
    return e >= 0 && e < E && rows > 0 && rows <= PF_M && gp0 >= 0 && gp0 <= T * K - rows;
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
