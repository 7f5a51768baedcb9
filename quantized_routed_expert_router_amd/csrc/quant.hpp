// quant.hpp -- 16-bit segment quantisation of activations and the Q2_0 block
// dot product on v_dot8_i32_i4, for the decode kernels.
//
// A segment is 32 consecutive activations v.  With s = max|v| / QMAX and
// q = rint(v / s) (|q| <= QMAX = 30000), q = n0 + 16 n1 + 256 n2 + 4096 n3 with
// balanced signed base-16 digits n_i in [-8, 7].  Digit i of the 32 values is
// stored as 4 dwords of 8 nibbles: dword (kk, par) holds, in nibble m, the
// digit of value 16 kk + 2 m + par.  That matches how the 2-bit codes of a
// block fall out of one code dword w (codes 16 kk .. 16 kk + 15 of the
// segment): (w & 0x33333333) has code 2m in nibble m, ((w >> 2) & 0x33333333)
// code 2m + 1.  So sum_i code_i * q_i is 32 v_dot8 instructions per 64-weight
// block, all exact in int32, and sum_i (code_i - 1) * q_i = that - sum_i q_i
// (the offset of the code table {0,1,2,3} -> {-1,0,1,2} of the Q2_0 format,
// "Strata in the source...", section "The CPU kernels").
#pragma once
#include "common.hpp"

namespace strata {

// Quantise one segment held by the 32 lanes of a half-wave (lane32 = lane & 31;
// both halves of a wave may quantise different segments at once, and every
// lane of the wave must call).  If `store`, lanes with lane32 in {0, 1, 16, 17}
// write the 16 digit dwords and lane32 == 0 the scale and the integer sum.
__device__ inline void quant_seg32(float v, int lane32, bool store, uint32_t *dig,
                                   float *scale, int32_t *sum)
{
    float m = fabsf(v);
#pragma unroll
    for (int x = 16; x >= 1; x >>= 1)
        m = fmaxf(m, __shfl_xor(m, x, 64));
    float inv = m > 0.f ? (float)QMAX / m : 0.f;
    int q = (int)rintf(v * inv);
    q = q > QMAX ? QMAX : (q < -QMAX ? -QMAX : q);
    int s = q;
#pragma unroll
    for (int x = 16; x >= 1; x >>= 1)
        s += __shfl_xor(s, x, 64);
    const int mpos = (lane32 & 15) >> 1;
    const int kk = lane32 >> 4;
    const int par = lane32 & 1;
    int r = q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int n = ((r + 8) & 15) - 8;
        r = (r - n) >> 4;
        uint32_t val = (uint32_t)(n & 15) << (4 * mpos);
        val |= __shfl_xor(val, 2, 64);
        val |= __shfl_xor(val, 4, 64);
        val |= __shfl_xor(val, 8, 64);
        if (store && mpos == 0)
            dig[kk * 8 + par * 4 + i] = val;
    }
    if (store && lane32 == 0) {
        *scale = m / (float)QMAX;
        *sum = s;
    }
}

// sum over one segment of (code - 1) * q: wa, wb are the segment's two code
// dwords, D its 16 digit dwords, qsum the segment's sum of q.
__device__ inline int seg_dot(uint32_t wa, uint32_t wb, const uint32_t *D, int qsum)
{
    int a0 = -qsum, a1 = 0, a2 = 0, a3 = 0;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const uint32_t w = kk ? wb : wa;
        const uint32_t e0 = w & 0x33333333u;
        const uint32_t e1 = (w >> 2) & 0x33333333u;
        const uint32_t *d = D + kk * 8;
        a0 = __builtin_amdgcn_sdot8((int)e0, (int)d[0], a0, false);
        a1 = __builtin_amdgcn_sdot8((int)e0, (int)d[1], a1, false);
        a2 = __builtin_amdgcn_sdot8((int)e0, (int)d[2], a2, false);
        a3 = __builtin_amdgcn_sdot8((int)e0, (int)d[3], a3, false);
        a0 = __builtin_amdgcn_sdot8((int)e1, (int)d[4], a0, false);
        a1 = __builtin_amdgcn_sdot8((int)e1, (int)d[5], a1, false);
        a2 = __builtin_amdgcn_sdot8((int)e1, (int)d[6], a2, false);
        a3 = __builtin_amdgcn_sdot8((int)e1, (int)d[7], a3, false);
    }
    return a0 + 16 * a1 + 256 * a2 + 4096 * a3;
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
    uint32_t v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3], v4 = p[4];
    w[0] = __builtin_amdgcn_perm(v1, v0, bc.sel);
    w[1] = __builtin_amdgcn_perm(v2, v1, bc.sel);
    w[2] = __builtin_amdgcn_perm(v3, v2, bc.sel);
    w[3] = __builtin_amdgcn_perm(v4, v3, bc.sel);
    d = half_bits_to_float(__builtin_amdgcn_ubfe(v0, bc.sh, 16));
}

// Partial dot of one 64-weight block with a quantised 64-value activation
// block (two segments): returns d * (s0 * S0 + s1 * S1) in fp32.
__device__ inline float block_partial(const uint32_t w[4], float d, const uint32_t D[32],
                                      float s0, float s1, int q0, int q1)
{
    const int S0 = seg_dot(w[0], w[1], D, q0);
    const int S1 = seg_dot(w[2], w[3], D + 16, q1);
    return fmaf(d * s1, (float)S1, (d * s0) * (float)S0);
}

} // namespace strata
