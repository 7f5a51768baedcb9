// quant.hpp -- 16-bit activation quantisation and the Q2_0 block dot product
// on v_dot8_i32_i4, for the decode kernels.
//
// A segment of n activations v (n = 64 for x, one per Q2_0 block column; n =
// 16 for h) gets a scale s = max|v| / QMAX and integers q = rint(v / s) with
// |q| <= QMAX = 30000, written as q = n0 + 16 n1 + 256 n2 + 4096 n3 with
// balanced signed base-16 digits n_i in [-8, 7].  Digit i of 16 consecutive
// values (a "quarter": codes 16k..16k+15 of a block) is stored in two dwords
// of 8 nibbles: dword (par, i) holds in nibble m the digit of value 2m + par.
// That is how the 2-bit codes fall out of one code dword w: (w & 0x33333333)
// has code 2m in nibble m, ((w >> 2) & 0x33333333) code 2m + 1.  So the sum of
// code * q over a block is 32 v_dot8 instructions, exact in int32 (digit plane
// i accumulated apart and weighted by 16^i at the end, or -- for a single
// quarter -- planes 3, 2, 1, 0 in turn with a shift by 4 between them),
// and the sum of (code - 1) * q = that - sum q removes the code offset of the
// Q2_0 table {0,1,2,3} -> {-1,0,1,2} ("Strata in the source...", section "The
// CPU kernels"); the segment stores -sum q for that last add.
//
// Layout of one quantised block of 64 values (32 dwords).  Logical dword
// j = 8k + 4 par + i (quarter k, parity par, digit i) is stored at position
// 2 (j mod 16) + j / 16: lane l of a 16-lane row loads the pair (j = l,
// j = 16 + l) with one 8-byte load, and the decode kernels hand dword j to all
// 16 lanes of the row with a DPP row broadcast (row_newbcast) folded into the
// v_dot8 itself, so the activations never pass through scalar registers or LDS.
#pragma once
#include "common.hpp"

namespace strata {

constexpr int QMAX = 30000;
constexpr int XBLK = H / QK;          // 40 activation blocks per token
constexpr int BLK_DWORDS = 32;        // 64 values x 4 digits x 4 bits
constexpr int HSEG16 = FF / 16;       // 40 h segments of 16 per slot
constexpr int HBLK = FF / QK;         // 10 h blocks of 64 per slot

// Storage position of logical dword j of a quantised block.
__host__ __device__ constexpr int dig_pos(int j) { return 2 * (j & 15) + (j >> 4); }

// Quantised activations of the decode path.
struct XQ {
    uint32_t *dig;     // [T][XBLK][32]  one 64-value block per Q2_0 block column
    float *scale;      // [T][XBLK]      scale of raw x; the RMSNorm factor is apart
    int32_t *nsum;     // [T][XBLK]      -(sum of q over the block)
    float *inv_rms;    // [T]            1 / sqrt(mean(x^2) + 1e-6), or 1 without RMSNorm
};
// h per 16 values; the digits of four consecutive segments form one 64-value
// block in the layout above, so dig is [T*K][HBLK][32].
struct HQ {
    uint32_t *dig;     // [T*K][HBLK][32]
    float *scale;      // [T*K][HSEG16]
    int32_t *nsum;     // [T*K][HSEG16]  -(sum of q over the segment)
};

// Quantise the value v of each lane, with the scale taken over each 16-lane
// row (nrows_per_seg = 1) or over the whole wave (nrows_per_seg = 4).  Returns
// q; packs the digits so that, in each row, lane 12 holds dwords (par 0, i) and
// lane 13 holds (par 1, i) for i = 0..3 in pk[i].  Every lane must call.
struct QuantOut {
    float scale;      // s (uniform over the segment)
    int sum;          // sum of q over the segment (valid in every lane)
    uint32_t pk[4];   // packed digits (valid in lanes 12 and 13 of each row)
};

template <bool WHOLE_WAVE> __device__ inline QuantOut quant_lanes(float v)
{
    QuantOut o;
    float m = max16(fabsf(v));
    if (WHOLE_WAVE) {
        const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0));
        const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16));
        const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32));
        const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48));
        m = fmaxf(fmaxf(a, b), fmaxf(c, d));
    }
    const float inv = m > 0.f ? (float)QMAX / m : 0.f;
    int q = (int)rintf(v * inv);
    q = q > QMAX ? QMAX : (q < -QMAX ? -QMAX : q);
    int s = isum16(q);
    if (WHOLE_WAVE) {
        s = __builtin_amdgcn_readlane(s, 0) + __builtin_amdgcn_readlane(s, 16) +
            __builtin_amdgcn_readlane(s, 32) + __builtin_amdgcn_readlane(s, 48);
    }
    o.scale = m / (float)QMAX;
    o.sum = s;
    const int mpos = (__lane_id() & 15) >> 1;
    int r = q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = ((r + 8) & 15) - 8;
        r = (r - n) >> 4;
        int val = (n & 15) << (4 * mpos);
        val |= dpp_i<DPP_XOR2>(val);
        val |= dpp_i<DPP_SHR4>(val);
        val |= dpp_i<DPP_SHR8>(val);
        o.pk[i] = (uint32_t)val;
    }
    return o;
}

// Store the packed digits of quarter k (0..3) of a block at blk (32 dwords):
// called by lanes 12 (par 0) and 13 (par 1) of a row.
__device__ inline void store_quarter(uint32_t *blk, int k, int par, const uint32_t pk[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        blk[dig_pos(8 * k + 4 * par + i)] = pk[i];
}

// acc += dot8(dword N of the row's broadcast register D, E): v_dot8c with the
// activation operand taken by row_newbcast:N from lane N of each 16-lane row.
#define STRATA_DOT8_BCAST(ACC, D, E, N)                                                            \
    asm("v_dot8c_i32_i4_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"                 \
        : "+v"(ACC)                                                                                \
        : "v"(D), "v"(E), "i"(N))

// Digit plane I (0..3) of one 16-value quarter against its two code
// registers E0 (even codes) and E1 (odd codes): quarter k takes logical dwords
// 8k + I (par 0) and 8k + 4 + I (par 1), from register DX (k < 2) or DY.
#define STRATA_QPLANE(A, DR, E0, E1, KH, I)                                                        \
    STRATA_DOT8_BCAST(A, DR, E0, 8 * (KH) + (I));                                                  \
    STRATA_DOT8_BCAST(A, DR, E1, 8 * (KH) + 4 + (I))

// The 16 code dwords of a block (W0..W3) split into even/odd code registers.
struct Codes {
    int e0[4], e1[4];
};
__device__ inline Codes split_codes(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3)
{
    Codes c;
    const uint32_t w[4] = {w0, w1, w2, w3};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        c.e0[k] = (int)(w[k] & 0x33333333u);
        c.e1[k] = (int)((w[k] >> 2) & 0x33333333u);
    }
    return c;
}

// Sum over a 64-value block of code * q plus A0: one accumulator per digit
// plane, so that consecutive v_dot8 never wait on each other's result.
__device__ inline int block_codes_dot(const Codes &c, uint32_t DX, uint32_t DY, int A0)
{
    int a0 = A0, a1 = 0, a2 = 0, a3 = 0;
#define STRATA_BQUARTER(DR, K, KH)                                                                 \
    STRATA_DOT8_BCAST(a0, DR, c.e0[K], 8 * (KH) + 0);                                              \
    STRATA_DOT8_BCAST(a1, DR, c.e0[K], 8 * (KH) + 1);                                              \
    STRATA_DOT8_BCAST(a2, DR, c.e0[K], 8 * (KH) + 2);                                              \
    STRATA_DOT8_BCAST(a3, DR, c.e0[K], 8 * (KH) + 3);                                              \
    STRATA_DOT8_BCAST(a0, DR, c.e1[K], 8 * (KH) + 4);                                              \
    STRATA_DOT8_BCAST(a1, DR, c.e1[K], 8 * (KH) + 5);                                              \
    STRATA_DOT8_BCAST(a2, DR, c.e1[K], 8 * (KH) + 6);                                              \
    STRATA_DOT8_BCAST(a3, DR, c.e1[K], 8 * (KH) + 7)
    STRATA_BQUARTER(DX, 0, 0);
    STRATA_BQUARTER(DX, 1, 1);
    STRATA_BQUARTER(DY, 2, 0);
    STRATA_BQUARTER(DY, 3, 1);
#undef STRATA_BQUARTER
    return a0 + (a1 << 4) + (a2 << 8) + (a3 << 12);
}

// The four 16-value quarters of a block, each summed apart (code * q), the
// four chains interleaved so that consecutive v_dot8 do not depend on each
// other; each chain takes digit planes 3, 2, 1, 0 with a shift by 4 between.
struct Quad {
    int q[4];
};
__device__ inline Quad quarters_codes_dot(const Codes &c, uint32_t DX, uint32_t DY)
{
    int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
#define STRATA_QPLANES(I)                                                                          \
    STRATA_DOT8_BCAST(a0, DX, c.e0[0], 0 + (I));                                                   \
    STRATA_DOT8_BCAST(a1, DX, c.e0[1], 8 + (I));                                                   \
    STRATA_DOT8_BCAST(a2, DY, c.e0[2], 0 + (I));                                                   \
    STRATA_DOT8_BCAST(a3, DY, c.e0[3], 8 + (I));                                                   \
    STRATA_DOT8_BCAST(a0, DX, c.e1[0], 4 + (I));                                                   \
    STRATA_DOT8_BCAST(a1, DX, c.e1[1], 12 + (I));                                                  \
    STRATA_DOT8_BCAST(a2, DY, c.e1[2], 4 + (I));                                                   \
    STRATA_DOT8_BCAST(a3, DY, c.e1[3], 12 + (I))
    STRATA_QPLANES(3);
    a0 <<= 4; a1 <<= 4; a2 <<= 4; a3 <<= 4;
    STRATA_QPLANES(2);
    a0 <<= 4; a1 <<= 4; a2 <<= 4; a3 <<= 4;
    STRATA_QPLANES(1);
    a0 <<= 4; a1 <<= 4; a2 <<= 4; a3 <<= 4;
    STRATA_QPLANES(0);
#undef STRATA_QPLANES
    Quad r;
    r.q[0] = a0;
    r.q[1] = a1;
    r.q[2] = a2;
    r.q[3] = a3;
    return r;
}

// Lane N of the caller's 16-lane row, as seen by every lane of the row.
template <int N> __device__ inline int row_bcast_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, 0x150 + N, 0xF, 0xF, false);
}
template <int N> __device__ inline float row_bcast_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xF, 0xF, false));
}

} // namespace strata
