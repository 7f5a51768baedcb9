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
// code * q over a quarter is 8 v_dot8 instructions, exact in int32, and the sum
// of (code - 1) * q = that - sum q removes the code offset of the Q2_0 table
// {0,1,2,3} -> {-1,0,1,2} ("Strata in the source...", section "The CPU kernels").
//
// Layout of one quantised block of 64 values: 32 dwords [quarter k][par][i].
#pragma once
#include "common.hpp"

namespace strata {

constexpr int QMAX = 30000;
constexpr int XBLK = H / QK;          // 40 activation blocks per token
constexpr int BLK_DWORDS = 32;        // 64 values x 4 digits x 4 bits
constexpr int HSEG16 = FF / 16;       // 40 h segments of 16 per slot
constexpr int SEG16_DWORDS = 8;

// Quantised activations of the decode path.
struct XQ {
    uint32_t *dig;     // [T][XBLK][32]  one 64-value block per Q2_0 block column
    float *scale;      // [T][XBLK]      scale of raw x; the RMSNorm factor is apart
    int32_t *sum;      // [T][XBLK]
    float *inv_rms;    // [T]            1 / sqrt(mean(x^2) + 1e-6), or 1 without RMSNorm
};
struct HQ {
    uint32_t *dig;     // [T*K][HSEG16][8]
    float *scale;      // [T*K][HSEG16]
    int32_t *sum;      // [T*K][HSEG16]
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

// sum over one quarter (16 codes in w) of code * q, digits D[par][i].
__device__ inline void quarter_dot(uint32_t w, const uint32_t *D, int &a0, int &a1, int &a2,
                                   int &a3)
{
    const int e0 = (int)(w & 0x33333333u);
    const int e1 = (int)((w >> 2) & 0x33333333u);
    a0 = __builtin_amdgcn_sdot8(e0, (int)D[0], a0, false);
    a1 = __builtin_amdgcn_sdot8(e0, (int)D[1], a1, false);
    a2 = __builtin_amdgcn_sdot8(e0, (int)D[2], a2, false);
    a3 = __builtin_amdgcn_sdot8(e0, (int)D[3], a3, false);
    a0 = __builtin_amdgcn_sdot8(e1, (int)D[4], a0, false);
    a1 = __builtin_amdgcn_sdot8(e1, (int)D[5], a1, false);
    a2 = __builtin_amdgcn_sdot8(e1, (int)D[6], a2, false);
    a3 = __builtin_amdgcn_sdot8(e1, (int)D[7], a3, false);
}

__device__ inline int digits_combine(int a0, int a1, int a2, int a3)
{
    return a0 + 16 * a1 + 256 * a2 + 4096 * a3;
}

// sum over a whole 64-block of (code - 1) * q with one scale for the block.
__device__ inline int block_dot64(const uint32_t w[4], const uint32_t D[32], int qsum)
{
    int a0 = -qsum, a1 = 0, a2 = 0, a3 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        quarter_dot(w[k], D + 8 * k, a0, a1, a2, a3);
    return digits_combine(a0, a1, a2, a3);
}

// The same block against four 16-value segments with their own scales:
// returns sum_k s_k * sum_quarter_k (code - 1) * q in fp32.
__device__ inline float block_dot16x4(const uint32_t w[4], const uint32_t D[32], const float s[4],
                                      const int qsum[4])
{
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int a0 = -qsum[k], a1 = 0, a2 = 0, a3 = 0;
        quarter_dot(w[k], D + 8 * k, a0, a1, a2, a3);
        acc = fmaf(s[k], (float)digits_combine(a0, a1, a2, a3), acc);
    }
    return acc;
}

// Per-lane constants to read block column c of a row staged in LDS: the 5
// dwords at byte offset st = 18c - 2(c & 1) (4-aligned) hold the whole block;
// for even c the scale is their bytes 0-1 and the codes bytes 2..17, for odd c
// the scale is bytes 2-3 and the codes bytes 4..19.
struct BlockCol {
    int st;         // byte offset of the 5-dword window within the row
    uint32_t sel;   // v_perm selector assembling a code dword from 2 window dwords
    uint32_t sh;    // bit offset of the scale inside window dword 0
};

__device__ inline BlockCol block_col(int c)
{
    BlockCol b;
    const int odd = c & 1;
    b.st = 18 * c - 2 * odd;
    b.sel = odd ? 0x07060504u : 0x05040302u;
    b.sh = odd ? 16u : 0u;
    return b;
}

// Read one block from an LDS row: the four code dwords and the fp32 scale.
__device__ inline void lds_block(const uint8_t *row, const BlockCol &bc, uint32_t w[4], float &d)
{
    const uint32_t *p = reinterpret_cast<const uint32_t *>(row + bc.st);
    const uint32_t v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3], v4 = p[4];
    w[0] = __builtin_amdgcn_perm(v1, v0, bc.sel);
    w[1] = __builtin_amdgcn_perm(v2, v1, bc.sel);
    w[2] = __builtin_amdgcn_perm(v3, v2, bc.sel);
    w[3] = __builtin_amdgcn_perm(v4, v3, bc.sel);
    d = half_bits_to_float(__builtin_amdgcn_ubfe(v0, bc.sh, 16));
}

} // namespace strata
