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
// K order: activations are stored once in the order the MFMA fragments take
// them, so every A fragment is one 16-byte LDS read.  For down (h, written by
// the gate/up epilogue), inside a 64-block: MFMA step j (0, 1) and lane group
// q (= lane/16) cover positions pi = 32 j + 8 q + s (s = 0..7), which carry
// input column 16 q + 4 j + s/2 + 8 (s % 2).  For gate/up (x, written by the
// prep kernel) the order runs over groups of four blocks (see the gate/up
// loop below).
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

// Four fp16 pairs (exact (c - 1) * d) from one code dword w and the scale
// pair d2 = (d, d): pair t of half HF is pair p = 4 HF + t of the dword, which
// holds codes p (low half) and p + 8 (high half).
template <int HF>
__device__ inline void dequant_half(uint32_t w, uint32_t d2bits, uint32_t out[4])
{
    const half2v d2 = as_h2(d2bits);
    const uint32_t w10 = w >> 10;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int p = 4 * HF + t;
        const uint32_t src = p < 5 ? w : w10;
        const int q = p < 5 ? p : p - 5;
        const uint32_t mag = (uint32_t)(25 - 2 * q) << 10;
        // (src & mask) | exponent pattern in one v_and_or_b32 (the compiler
        // would spend an AND and an OR with literal operands)
        uint32_t u;
        asm("v_and_or_b32 %0, %1, %2, %3"
            : "=v"(u)
            : "v"(src), "s"(0x00030003u << (2 * q)), "v"(mag | (mag << 16)));
        const _Float16 m1 = (_Float16)(float)((1 << (10 - 2 * q)) + 1);
        const half2v cm1 = as_h2(u) - (half2v){m1, m1};
        out[t] = as_u32(cm1 * d2);
    }
}

// All eight pairs of a code dword; dbits is the scale's fp16 bit pattern.
__device__ inline void dequant_dword(uint32_t w, uint32_t dbits, uint32_t out[8])
{
    const uint32_t d2 = dbits | (dbits << 16);
    dequant_half<0>(w, d2, out);
    dequant_half<1>(w, d2, out + 4);
}

// K-order position of input column c (0..63) inside its block.
__device__ inline int pf_pos_of_col(int c)
{
    const int q = c >> 4, r16 = c & 15;
    const int p = r16 & 7, hb = r16 >> 3;
    return 32 * (p >> 2) + 8 * q + 2 * (p & 3) + hb;
}

// Down: software pipeline of one (item, N-tile), fed by direct global->LDS
// loads (global_load_lds: the data never passes through registers).
//  - Activations (h): one block (64 rows x 64 halfs, 8 KB) per K-step in a
//    ring of four LDS buffers, requested three blocks ahead.  Rows are packed
//    at 128 bytes; the 16-byte chunk c of row m sits at position c ^ (m & 7),
//    so the MFMA fragment reads of 16 rows hit distinct banks without padding.
//  - Weights: the tile's down rows are contiguous in memory and all 10 blocks
//    (46,080 bytes) arrive at once, 16 bytes a lane.
// Every LDS read of a block and its wait are one asm statement, and the
// vector-memory waits are explicit counts that follow from the fixed issue
// order (derived at each wait below); one barrier per block.
constexpr int PF_ROWS = 256;                            // weight rows per WG
constexpr int PF_ABYTES = PF_M * QK * 2;                // 8,192 bytes per activation block
constexpr int PF_NABUF = 4;                             // activation ring
constexpr int PF_DB = PF_ROWS * ROW_D;                  // 46,080 bytes of down rows
constexpr int PF_DCH = PF_DB / 16 / 4;                 // 720 16-byte chunks per wave
constexpr int PF_DNB = (PF_DCH + 63) / 64;              // 12 dwordx4 loads per wave
constexpr int PF_LDS_D = PF_NABUF * PF_ABYTES + PF_DB;           // 78,848
static_assert(PF_DCH * 16 * 4 == PF_DB, "load split");
static_assert(PF_THREADS == 256, "four waves");

// Gate/up: K is walked in groups of four blocks (256 input columns).  In
// group g the lanes of quarter q (= lane / 16) own block 4 g + q of their
// weight row whole, loaded straight into registers -- the weights of a wave
// serve no other wave, so they skip the LDS: 16 + 4 bytes from the dword at
// or below the block's start (an 18-byte block starts 0 or 2 bytes into that
// dword, the same for every lane of a quarter), then byte permutes pick out
// the scale pair and the four code dwords.  MFMA step j (0..7) of a group
// uses code dword j / 2, codes 4 (j % 2) + s / 2 + 8 (s % 2) along its
// fragment (s = 0..7), i.e. input column
// 64 (4 g + q) + 16 (j / 2) + 4 (j % 2) + s / 2 + 8 (s % 2); the prep kernel
// stores the activations in that order, as 16-byte chunk 8 q + j of each
// 512-byte group.
// Activations: one group (64 rows x 512 bytes) per LDS buffer, two buffers,
// filled by direct global->LDS loads one group ahead, and read by all four
// waves.  A 1 KB request fills 8 rows (row group r = row / 8) x 8 chunks of
// one octet; inside the row group chunk c sits at position c ^ (r & 1), so
// the two row groups of a 16-row fragment read fall on different banks.
// One barrier per group.
constexpr int PG_BLK = 4;                               // blocks per K group
constexpr int PG_NG = NB_G / PG_BLK;                    // 10 groups
constexpr int PG_GBYTES = PG_BLK * QK * 2;              // 512 bytes of a row per group
constexpr int PG_ABYTES = PF_M * PG_GBYTES;             // 32,768 bytes per activation group
constexpr int PF_LDS_G = 2 * PG_ABYTES;                 // 65,536
static_assert(PG_NG * PG_BLK == NB_G, "whole groups");
static_assert(BB + 2 <= 20 && PG_BLK * BB * (PG_NG - 1) + 3 * BB - 2 + 20 == ROW_G,
              "20 loaded bytes hold a block; those of a row's last block end at the row's end");

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ inline uint32_t lds_addr(uint8_t *p)
{
    return (uint32_t)(uintptr_t)(lds_u8 *)p;
}

// Activation requests of block b for this wave: two 16-byte chunks per lane
// (rows 16 w + 8 h + lane / 8, position lane % 8).
struct PfAct {
    const __half *row[2];   // this lane's two rows (valid memory for every lane)
    int chunk;              // global 16-byte chunk for this lane's position
    __device__ void request(uint8_t *abuf, int b) const
    {
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
        for (int h = 0; h < 2; ++h)
            __builtin_amdgcn_global_load_lds(row[h] + QK * b + 8 * chunk,
                                             abuf + (128 * w + 64 * h) * 16, 16, 0, 0);
    }
};

// The LDS reads of one block: the 4 activation subtiles x 2 K-halves and, for
// each of the 4 weight subtiles, its scale and this lane's code dword.
// AOFF: activation buffer offset; BOFF: this block's offset in the weight
// rows; NS1..NS3: offsets of weight subtiles 1..3 from subtile 0.
struct PfVals {
    half8 af[4][2];
    uint32_t dbits[4], wc[4];
};

// Issues the reads without waiting for them: the values are not to be used
// before pf_reads_done on the same PfVals (which is what orders them).  Only
// the MS activation subtiles that hold item rows are read.
template <int AOFF, int BOFF, int NS1, int NS2, int NS3, int MS>
__device__ inline void pf_reads_issue(uint32_t a0, uint32_t a1, uint32_t bs, uint32_t bc, PfVals &v)
{
#define STRATA_PF_AREAD(MI)                                                                        \
    asm volatile("ds_read_b128 %0, %2 offset:%4\n\t"                                             \
                 "ds_read_b128 %1, %3 offset:%4"                                                   \
                 : "=&v"(v.af[MI][0]), "=&v"(v.af[MI][1])                                          \
                 : "v"(a0), "v"(a1), "i"(AOFF + 2048 * (MI))                                       \
                 : "memory")
    STRATA_PF_AREAD(0);
    if constexpr (MS > 1)
        STRATA_PF_AREAD(1);
    if constexpr (MS > 2)
        STRATA_PF_AREAD(2);
    if constexpr (MS > 3)
        STRATA_PF_AREAD(3);
#undef STRATA_PF_AREAD
    asm volatile("ds_read_u16 %0, %8 offset:%10\n\t"
                 "ds_read_b32 %4, %9 offset:%10\n\t"
                 "ds_read_u16 %1, %8 offset:%11\n\t"
                 "ds_read_b32 %5, %9 offset:%11\n\t"
                 "ds_read_u16 %2, %8 offset:%12\n\t"
                 "ds_read_b32 %6, %9 offset:%12\n\t"
                 "ds_read_u16 %3, %8 offset:%13\n\t"
                 "ds_read_b32 %7, %9 offset:%13"
                 : "=&v"(v.dbits[0]), "=&v"(v.dbits[1]), "=&v"(v.dbits[2]), "=&v"(v.dbits[3]),
                   "=&v"(v.wc[0]), "=&v"(v.wc[1]), "=&v"(v.wc[2]), "=&v"(v.wc[3])
                 : "v"(bs), "v"(bc), "i"(BOFF), "i"(BOFF + NS1), "i"(BOFF + NS2),
                   "i"(BOFF + NS3)
                 : "memory");
}

// Waits for the reads of v: from here on the compiler sees their values.
__device__ inline void pf_reads_done(PfVals &v)
{
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v.af[0][0]), "+v"(v.af[0][1]), "+v"(v.af[1][0]), "+v"(v.af[1][1]),
                   "+v"(v.af[2][0]), "+v"(v.af[2][1]), "+v"(v.af[3][0]), "+v"(v.af[3][1]),
                   "+v"(v.dbits[0]), "+v"(v.dbits[1]), "+v"(v.dbits[2]), "+v"(v.dbits[3]),
                   "+v"(v.wc[0]), "+v"(v.wc[1]), "+v"(v.wc[2]), "+v"(v.wc[3])
                 :
                 : "memory");
}

// acc[ns][mi] += A(64 x 64) W(64 x 64) from the values read for one block:
// the four weight subtiles are dequantised first, then the 32 MFMAs run in
// an order where one accumulator recurs only every 16 instructions.
template <int MS>
__device__ inline void pf_math(const PfVals &v, floatx4 acc[4][4])
{
    const auto &af = v.af;
    const auto &dbits = v.dbits;
    const auto &wc = v.wc;
    half8 bf[4][2];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
        uint32_t pr[8];
        dequant_dword(wc[ns], dbits[ns], pr);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bf[ns][j] = __builtin_bit_cast(
                half8, make_uint4(pr[4 * j], pr[4 * j + 1], pr[4 * j + 2], pr[4 * j + 3]));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
#pragma unroll
            for (int mi = 0; mi < MS; ++mi)   // only the 16-row groups holding item rows
                acc[ns][mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mi][j], bf[ns][j], acc[ns][mi],
                                                                      0, 0, 0);
#ifdef PF_INTERLEAVE
    // scheduler hint: one MFMA, then up to three VALU, repeated
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
#endif
}

template <int N> __device__ inline void vm_wait()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// Per-lane LDS read addresses of the activation fragments (K-halves j = 0, 1)
// of row 16 mi + lane % 16, position (lane / 16 + 4 j) ^ (lane % 8).
__device__ inline void pf_act_read_addrs(uint32_t abase, uint32_t &a0, uint32_t &a1)
{
    const int lane = threadIdx.x & 63, q = lane >> 4;
    a0 = abase + (lane & 15) * 128 + 16 * (q ^ (lane & 7));
    a1 = abase + (lane & 15) * 128 + 16 * ((q + 4) ^ (lane & 7));
}

// Activation requests of gate/up group g for this wave: 8 requests of 1 KB,
// request i filling row group 2 w + i / 4, chunk octet i % 4.
struct PgAct {
    const uint8_t *row[2];   // rows 16 w + 8 h + lane % 8 (valid memory for every lane)
    uint32_t coff[2];        // byte offset of this lane's chunk in the octet, h = 0, 1
    __device__ void request(uint8_t *abuf, int g) const
    {
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds(row[i >> 2] + PG_GBYTES * g + 128 * (i & 3) + coff[i >> 2],
                                             abuf + (8 * w + i) * 1024, 16, 0, 0);
    }
};

// One group's weight bytes for the wave's four 16-row subtiles.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
struct PgW {
    u32x4 lo[4];
    uint32_t hi[4];
};

// Waits for all of this wave's loads; the compiler then sees r as ready (its
// own wait for them would otherwise also wait for the loads issued since).
__device__ inline void pg_wait_all(PgW &r)
{
    u32x4 a = r.lo[0], b = r.lo[1], c = r.lo[2], d = r.lo[3];
    uint32_t e = r.hi[0], f = r.hi[1], g = r.hi[2], h = r.hi[3];
    asm volatile("s_waitcnt vmcnt(0)"
                 : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h)
                 :
                 : "memory");
    r.lo[0] = a, r.lo[1] = b, r.lo[2] = c, r.lo[3] = d;
    r.hi[0] = e, r.hi[1] = f, r.hi[2] = g, r.hi[3] = h;
}

__device__ inline void pg_wload(const uint8_t *blob, const uint32_t woff[4], int g, PgW &r)
{
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
        const uint8_t *p = blob + woff[ns] + PG_BLK * BB * g;
        r.lo[ns] = *reinterpret_cast<const u32x4 *>(p);
        r.hi[ns] = *reinterpret_cast<const uint32_t *>(p + 16);
    }
}

// LDS reads of the MS activation fragments of one MFMA step (without waiting);
// 16-row group mi is two row groups, 8 KB, further on.
template <int OFF, int MS>
__device__ inline void pg_aread(uint32_t a, half8 af[4])
{
#define STRATA_PG_AREAD(MI)                                                                        \
    asm volatile("ds_read_b128 %0, %1 offset:%2"                                                   \
                 : "=&v"(af[MI])                                                                   \
                 : "v"(a), "i"(OFF + 8192 * (MI))                                                  \
                 : "memory")
    STRATA_PG_AREAD(0);
    if constexpr (MS > 1)
        STRATA_PG_AREAD(1);
    if constexpr (MS > 2)
        STRATA_PG_AREAD(2);
    if constexpr (MS > 3)
        STRATA_PG_AREAD(3);
#undef STRATA_PG_AREAD
}

// Waits for pg_aread: from here on the compiler sees the values.
template <int MS>
__device__ inline void pg_await(half8 af[4])
{
    if constexpr (MS == 1)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(af[0]) : : "memory");
    else if constexpr (MS == 2)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(af[0]), "+v"(af[1]) : : "memory");
    else if constexpr (MS == 3)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]) : : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3])
                     :
                     : "memory");
}

// MFMA step J of a group: issue the reads of step J + 1, dequantise this
// step's four weight fragments, issue its 4 x MS MFMAs, wait for the reads.
template <int BUF, int MS, int J>
__device__ inline void pg_step(uint32_t ae, uint32_t ao, const uint32_t d2[4], const uint32_t cw[4][4],
                               half8 af[2][4], floatx4 acc[4][4])
{
    if constexpr (J < 7)
        pg_aread<BUF * PG_ABYTES + 128 * (J + 1), MS>(((J + 1) & 1) ? ao : ae, af[(J + 1) & 1]);
    uint32_t pr[4][4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
        dequant_half<J & 1>(cw[ns][J >> 1], d2[ns], pr[ns]);
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
        const half8 bf = __builtin_bit_cast(half8, make_uint4(pr[ns][0], pr[ns][1], pr[ns][2], pr[ns][3]));
#pragma unroll
        for (int mi = 0; mi < MS; ++mi)   // only the 16-row groups holding item rows
            acc[ns][mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[J & 1][mi], bf, acc[ns][mi], 0, 0, 0);
    }
    if constexpr (J < 7)
        pg_await<MS>(af[(J + 1) & 1]);
}

// acc[ns][mi] += the products of one group: the scale pairs and code dwords
// are picked out of the loaded bytes, then each of the 8 MFMA steps reads its
// activation fragments (the next step's reads run during this step's math),
// dequantises its four weight fragments and issues 4 x MS MFMAs.
// ae / ao: this lane's fragment read address for even / odd steps.
template <int BUF, int MS>
__device__ inline void pg_group(uint32_t ae, uint32_t ao, const PgW &wr, uint32_t sel_c,
                                uint32_t sel_d, floatx4 acc[4][4])
{
    uint32_t d2[4], cw[4][4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
        const uint32_t L[5] = {wr.lo[ns].x, wr.lo[ns].y, wr.lo[ns].z, wr.lo[ns].w, wr.hi[ns]};
        d2[ns] = __builtin_amdgcn_perm(L[0], L[0], sel_d);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            cw[ns][i] = __builtin_amdgcn_perm(L[i + 1], L[i], sel_c);
    }
    half8 af[2][4];
    pg_aread<BUF * PG_ABYTES, MS>(ae, af[0]);
    pg_await<MS>(af[0]);
    pg_step<BUF, MS, 0>(ae, ao, d2, cw, af, acc);
    pg_step<BUF, MS, 1>(ae, ao, d2, cw, af, acc);
    pg_step<BUF, MS, 2>(ae, ao, d2, cw, af, acc);
    pg_step<BUF, MS, 3>(ae, ao, d2, cw, af, acc);
    pg_step<BUF, MS, 4>(ae, ao, d2, cw, af, acc);
    pg_step<BUF, MS, 5>(ae, ao, d2, cw, af, acc);
    pg_step<BUF, MS, 6>(ae, ao, d2, cw, af, acc);
    pg_step<BUF, MS, 7>(ae, ao, d2, cw, af, acc);
}

// Gate/up K loop over the 10 groups: group g computes from LDS buffer g % 2
// and register set g % 2.  At the top of each group the wave waits for all
// its requests (the group's activations and weights, issued one group
// earlier) and passes the barrier (every wave's share has landed; every wave
// is done reading the other buffer), then requests group g + 1 into the
// other buffer and register set and computes group g.
template <int MS>
__device__ inline void pg_gateup_loop(const uint8_t *blob, const uint32_t woff[4], const PgAct &act,
                                      uint8_t *lds, uint32_t ae, uint32_t ao, uint32_t sel_c,
                                      uint32_t sel_d, floatx4 acc[4][4])
{
    PgW w0, w1;
    act.request(lds, 0);
    pg_wload(blob, woff, 0, w0);
#pragma unroll 1
    for (int g = 0; g < PG_NG; g += 2) {
        pg_wait_all(w0);
        __builtin_amdgcn_s_barrier();
        act.request(lds + PG_ABYTES, g + 1);
        pg_wload(blob, woff, g + 1, w1);
        pg_group<0, MS>(ae, ao, w0, sel_c, sel_d, acc);
        pg_wait_all(w1);
        __builtin_amdgcn_s_barrier();
        if (g + 2 < PG_NG) {
            act.request(lds, g + 2);
            pg_wload(blob, woff, g + 2, w0);
        }
        pg_group<1, MS>(ae, ao, w1, sel_c, sel_d, acc);
    }
}

// Down K loop: 10 blocks; all weights requested first, then A0 .. A3.
// Iteration b: wait for A(b+1) (younger: A(b+2), A(b+3): 4), barrier, request
// A(b+4) into block b's buffer, issue the reads of block b+1, compute block b.
template <int MS>
__device__ inline void pf_down_loop(const uint8_t *wsrc, const PfAct &act, uint8_t *lds,
                                    uint32_t bs, uint32_t bc, floatx4 acc[4][4])
{
    uint8_t *const wbuf = lds + PF_NABUF * PF_ABYTES;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // the 46,080 contiguous bytes of the tile, 16 bytes a lane (the last
    // request of a wave has 16 lanes)
#pragma unroll
    for (int h = 0; h < PF_DNB; ++h)
        if (64 * h + lane < PF_DCH)
            __builtin_amdgcn_global_load_lds(wsrc + 16 * (PF_DCH * w + 64 * h + lane),
                                             wbuf + (PF_DCH * w + 64 * h) * 16, 16, 0, 0);
    uint32_t a0, a1;
    pf_act_read_addrs(lds_addr(lds), a0, a1);
    act.request(lds, 0);
    act.request(lds + PF_ABYTES, 1);
    act.request(lds + 2 * PF_ABYTES, 2);
    act.request(lds + 3 * PF_ABYTES, 3);
    constexpr int NS1 = 16 * ROW_D, NS2 = 32 * ROW_D, NS3 = 48 * ROW_D;
    vm_wait<6>();   // the weights and A0: younger A1, A2, A3
    __builtin_amdgcn_s_barrier();
    PfVals cur, nxt;
    pf_reads_issue<0, 0, NS1, NS2, NS3, MS>(a0, a1, bs, bc, cur);
    pf_reads_done(cur);
#define STRATA_PF_DSTEP(B)                                                                         \
    {                                                                                              \
        vm_wait<4>();                                                                              \
        __builtin_amdgcn_s_barrier();                                                              \
        act.request(lds + ((B) & 3) * PF_ABYTES, (B) + 4 < NB_D ? (B) + 4 : NB_D - 1);             \
        pf_reads_issue<(((B) + 1) & 3) * PF_ABYTES, BB * ((B) + 1 < NB_D ? (B) + 1 : NB_D - 1),    \
                       NS1, NS2, NS3, MS>(a0, a1, bs, bc, nxt);                                        \
        pf_math<MS>(cur, acc);                                                                     \
        pf_reads_done(nxt);                                                                        \
        cur = nxt;                                                                                 \
    }
    STRATA_PF_DSTEP(0)
    STRATA_PF_DSTEP(1)
    STRATA_PF_DSTEP(2)
    STRATA_PF_DSTEP(3)
    STRATA_PF_DSTEP(4)
    STRATA_PF_DSTEP(5)
    STRATA_PF_DSTEP(6)
    STRATA_PF_DSTEP(7)
    STRATA_PF_DSTEP(8)
    STRATA_PF_DSTEP(9)
#undef STRATA_PF_DSTEP
    vm_wait<0>();
}

// silu(g) * u = g u / (1 + e^-g) with the hardware exp2 and reciprocal (each
// within about 1 ulp in fp32, far inside the fp16 rounding h gets next; for
// g << 0, e^-g overflows to inf and the reciprocal gives 0).
__device__ inline float pf_silu_mul(float g, float u)
{
    const float e = __builtin_amdgcn_exp2f(-1.44269504088896341f * g);
    return g * u * __builtin_amdgcn_rcpf(1.f + e);
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

__global__ __launch_bounds__(PF_THREADS, 2) void pf_gateup(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ slots, const int32_t *__restrict__ active,
    const int32_t *__restrict__ mlist, const int32_t *__restrict__ nitems,
    const __half *__restrict__ xperm, __half *__restrict__ hperm, int T)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[PF_LDS_G];
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int item = 8 * (idx / PF_NTILES_G) + xcd;
    const int nt = idx % PF_NTILES_G;
    const PfItem it = pf_item(item, mlist, nitems, offsets, active, T);
    if (!it.ok)
        return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int jw = nt * PF_NT_G + 32 * wave;   // this wave's first FF row
    const uint8_t *blob = blobs + (size_t)it.e * BLOB;
    // Activation rows this lane requests (rows past the item's end read its
    // first row; their results are never stored): rows 16 w + 8 h + lane % 8,
    // chunk (lane / 8) ^ h of each octet.
    PgAct act;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 16 * wave + 8 * h + (lane & 7);
        const int sl = slots[it.gp0 + (r < it.rows ? r : 0)];
        const int t = (sl >= 0 && sl < T * K) ? sl / K : 0;
        act.row[h] = reinterpret_cast<const uint8_t *>(xperm + (size_t)t * H);
        act.coff[h] = 16 * ((lane >> 3) ^ h);
    }
    // Weight bytes: subtile ns is gate (ns < 2) or up rows jw + 16 (ns % 2) +
    // lane % 16; quarter q loads from the dword at or below block q's start.
    const int q = lane >> 4, odd = q & 1;
    uint32_t woff[4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
        woff[ns] = (uint32_t)((ns >= 2 ? MAT : 0) + (size_t)(jw + 16 * (ns & 1) + (lane & 15)) * ROW_G +
                              BB * q - 2 * odd);
    const uint32_t sel_c = odd ? 0x07060504u : 0x05040302u;   // code dword i: bytes 2..5 or 4..7 of L[i], L[i+1]
    const uint32_t sel_d = odd ? 0x03020302u : 0x01000100u;   // (d, d) from bytes 0, 1 or 2, 3 of L[0]
    // Fragment reads: row 16 mi + lane % 16 (row group 2 mi + b), chunk 8 q + j at
    // position 8 q + (j ^ b) of the row group.
    const int b = (lane >> 3) & 1;
    const uint32_t abase = lds_addr(lds) + (32 * b + 8 * q) * 128 + 16 * (lane & 7);
    const uint32_t ae = abase + 128 * b, ao = abase - 128 * b;
    floatx4 acc[4][4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            acc[ns][mi] = (floatx4){0.f, 0.f, 0.f, 0.f};
    // one straight-line loop per number of 16-row groups holding item rows
    switch ((it.rows + 15) >> 4) {
    case 1:
        pg_gateup_loop<1>(blob, woff, act, lds, ae, ao, sel_c, sel_d, acc);
        break;
    case 2:
        pg_gateup_loop<2>(blob, woff, act, lds, ae, ao, sel_c, sel_d, acc);
        break;
    case 3:
        pg_gateup_loop<3>(blob, woff, act, lds, ae, ao, sel_c, sel_d, acc);
        break;
    default:
        pg_gateup_loop<4>(blob, woff, act, lds, ae, ao, sel_c, sel_d, acc);
        break;
    }
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
                    const float h = pf_silu_mul(g, u);
                    hperm[(size_t)(it.gp0 + m) * FF + col] = __float2half_rn(h);
                }
            }
        }
    }
}

__global__ __launch_bounds__(PF_THREADS, 2) void pf_down(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ slots, const int32_t *__restrict__ active,
    const int32_t *__restrict__ mlist, const int32_t *__restrict__ nitems,
    const __half *__restrict__ hperm, float *__restrict__ out, int T)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[PF_LDS_D];
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int item = 8 * (idx / PF_NTILES_D) + xcd;
    const int nt = idx % PF_NTILES_D;
    const PfItem it = pf_item(item, mlist, nitems, offsets, active, T);
    if (!it.ok)
        return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rw = nt * PF_NT_D + 64 * wave;   // this wave's first output row
    PfAct act;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 16 * wave + 8 * h + (lane >> 3);
        act.row[h] = hperm + (size_t)(it.gp0 + (r < it.rows ? r : 0)) * FF;
    }
    act.chunk = (lane & 7) ^ (lane >> 3);
    const uint8_t *wsrc = blobs + (size_t)it.e * BLOB + 2 * MAT + (size_t)nt * PF_DB;
    const uint32_t bs = lds_addr(lds + PF_NABUF * PF_ABYTES) + (64 * wave + (lane & 15)) * ROW_D;
    const uint32_t bc = bs + 2 + 4 * (lane >> 4);
    floatx4 acc[4][4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            acc[ns][mi] = (floatx4){0.f, 0.f, 0.f, 0.f};
    switch ((it.rows + 15) >> 4) {
    case 1:
        pf_down_loop<1>(wsrc, act, lds, bs, bc, acc);
        break;
    case 2:
        pf_down_loop<2>(wsrc, act, lds, bs, bc, acc);
        break;
    case 3:
        pf_down_loop<3>(wsrc, act, lds, bs, bc, acc);
        break;
    default:
        pf_down_loop<4>(wsrc, act, lds, bs, bc, acc);
        break;
    }
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
