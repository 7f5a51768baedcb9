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
// filled by direct global->LDS loads one group ahead, and read by every wave
// of the workgroup.  A 1 KB request fills 8 rows (row group r = row / 8) x 8 chunks of
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

// Activation requests of a group for a wave of a four-wave workgroup (the
// down kernel's groups 0 and 1): 8 requests of 1 KB,
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

// One group's weight bytes for the wave's NS 16-row subtiles.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <int NS> struct PgWn {
    u32x4 lo[NS];
    uint32_t hi[NS];
};
using PgW = PgWn<4>;

// Waits for all of this wave's loads; the compiler then sees r as ready (its
// own wait for them would otherwise also wait for the loads issued since).
template <int NS> __device__ inline void pg_wait_all(PgWn<NS> &r)
{
    static_assert(NS == 2 || NS == 4, "two or four subtiles");
    if constexpr (NS == 4) {
        u32x4 a = r.lo[0], b = r.lo[1], c = r.lo[2], d = r.lo[3];
        uint32_t e = r.hi[0], f = r.hi[1], g = r.hi[2], h = r.hi[3];
        asm volatile("s_waitcnt vmcnt(0)"
                     : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h)
                     :
                     : "memory");
        r.lo[0] = a, r.lo[1] = b, r.lo[2] = c, r.lo[3] = d;
        r.hi[0] = e, r.hi[1] = f, r.hi[2] = g, r.hi[3] = h;
    } else {
        u32x4 a = r.lo[0], b = r.lo[1];
        uint32_t e = r.hi[0], f = r.hi[1];
        asm volatile("s_waitcnt vmcnt(0)" : "+v"(a), "+v"(b), "+v"(e), "+v"(f) : : "memory");
        r.lo[0] = a, r.lo[1] = b;
        r.hi[0] = e, r.hi[1] = f;
    }
}

template <int NS>
__device__ inline void pg_wload(const uint8_t *blob, const uint32_t woff[NS], int g, PgWn<NS> &r)
{
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
        const uint8_t *p = blob + woff[ns] + PG_BLK * BB * g;
        r.lo[ns] = *reinterpret_cast<const u32x4 *>(p);
        r.hi[ns] = *reinterpret_cast<const uint32_t *>(p + 16);
    }
}

// LDS reads of the MS activation fragments of one MFMA step (without waiting);
// 16-row group mi is two row groups, MSTR bytes, further on.
template <int OFF, int MSTR, int MS>
__device__ inline void pg_aread(uint32_t a, half8 af[4])
{
#define STRATA_PG_AREAD(MI)                                                                        \
    asm volatile("ds_read_b128 %0, %1 offset:%2"                                                   \
                 : "=&v"(af[MI])                                                                   \
                 : "v"(a), "i"(OFF + MSTR * (MI))                                                  \
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

// MFMA step J of a group of NSTEP steps whose fragments start at LDS offset
// AOFF (16-row groups MSTR bytes apart): issue the reads of step J + 1,
// dequantise this step's four weight fragments, issue its 4 x MS MFMAs, wait
// for the reads.
template <int AOFF, int MSTR, int NSTEP, int MS, int J, int NS = 4>
__device__ inline void pg_step(uint32_t ae, uint32_t ao, const uint32_t d2[NS],
                               const uint32_t cw[NS][4], half8 af[2][4], floatx4 acc[NS][4])
{
    if constexpr (J + 1 < NSTEP)
        pg_aread<AOFF + 128 * (J + 1), MSTR, MS>(((J + 1) & 1) ? ao : ae, af[(J + 1) & 1]);
    uint32_t pr[NS][4];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
        dequant_half<J & 1>(cw[ns][J >> 1], d2[ns], pr[ns]);
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
        const half8 bf = __builtin_bit_cast(half8, make_uint4(pr[ns][0], pr[ns][1], pr[ns][2], pr[ns][3]));
#pragma unroll
        for (int mi = 0; mi < MS; ++mi)   // only the 16-row groups holding item rows
            acc[ns][mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[J & 1][mi], bf, acc[ns][mi], 0, 0, 0);
    }
    if constexpr (J + 1 < NSTEP)
        pg_await<MS>(af[(J + 1) & 1]);
}

// The scale pairs and code dwords of one group, picked out of its loaded
// bytes (sel_d, sel_c: the byte selections for this lane's block offset).
template <int NS>
__device__ inline void pg_extract(const PgWn<NS> &wr, uint32_t sel_c, uint32_t sel_d, uint32_t d2[NS],
                                  uint32_t cw[NS][4])
{
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
        const uint32_t L[5] = {wr.lo[ns].x, wr.lo[ns].y, wr.lo[ns].z, wr.lo[ns].w, wr.hi[ns]};
        d2[ns] = __builtin_amdgcn_perm(L[0], L[0], sel_d);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            cw[ns][i] = __builtin_amdgcn_perm(L[i + 1], L[i], sel_c);
    }
}

// acc[ns][mi] += the products of one group: the scale pairs and code dwords
// are picked out of the loaded bytes, then each of the 8 MFMA steps reads its
// activation fragments (the next step's reads run during this step's math),
// dequantises its four weight fragments and issues 4 x MS MFMAs.
// ae / ao: this lane's fragment read address for even / odd steps.
template <int BUF, int MS, int NS = 4>
__device__ inline void pg_group(uint32_t ae, uint32_t ao, const PgWn<NS> &wr, uint32_t sel_c,
                                uint32_t sel_d, floatx4 acc[NS][4])
{
    uint32_t d2[NS], cw[NS][4];
    pg_extract(wr, sel_c, sel_d, d2, cw);
    constexpr int A0 = BUF * PG_ABYTES;
    half8 af[2][4];
    pg_aread<A0, 8192, MS>(ae, af[0]);
    pg_await<MS>(af[0]);
    pg_step<A0, 8192, 8, MS, 0, NS>(ae, ao, d2, cw, af, acc);
    pg_step<A0, 8192, 8, MS, 1, NS>(ae, ao, d2, cw, af, acc);
    pg_step<A0, 8192, 8, MS, 2, NS>(ae, ao, d2, cw, af, acc);
    pg_step<A0, 8192, 8, MS, 3, NS>(ae, ao, d2, cw, af, acc);
    pg_step<A0, 8192, 8, MS, 4, NS>(ae, ao, d2, cw, af, acc);
    pg_step<A0, 8192, 8, MS, 5, NS>(ae, ao, d2, cw, af, acc);
    pg_step<A0, 8192, 8, MS, 6, NS>(ae, ao, d2, cw, af, acc);
    pg_step<A0, 8192, 8, MS, 7, NS>(ae, ao, d2, cw, af, acc);
}

// Gate/up K loop over the 10 groups: group g computes from LDS buffer g % 2
// and register set g % 2.  At the top of each group the wave waits for all
// its requests (the group's activations and weights, issued one group
// earlier) and passes the barrier (every wave's share has landed; every wave
// is done reading the other buffer), then requests group g + 1 into the
// other buffer and register set and computes group g.
template <int MS, int NS, class ACT>
__device__ inline void pg_gateup_loop(const uint8_t *blob, const uint32_t woff[NS], const ACT &act,
                                      uint8_t *lds, uint32_t ae, uint32_t ao, uint32_t sel_c,
                                      uint32_t sel_d, floatx4 acc[NS][4])
{
    PgWn<NS> w0, w1;
    act.request(lds, 0);
    pg_wload(blob, woff, 0, w0);
#pragma unroll 1
    for (int g = 0; g < PG_NG; g += 2) {
        pg_wait_all(w0);
        __builtin_amdgcn_s_barrier();
        act.request(lds + PG_ABYTES, g + 1);
        pg_wload(blob, woff, g + 1, w1);
        pg_group<0, MS, NS>(ae, ao, w0, sel_c, sel_d, acc);
        pg_wait_all(w1);
        __builtin_amdgcn_s_barrier();
        if (g + 2 < PG_NG) {
            act.request(lds, g + 2);
            pg_wload(blob, woff, g + 2, w0);
        }
        pg_group<1, MS, NS>(ae, ao, w1, sel_c, sel_d, acc);
    }
}

// Down: K = 640.  Groups 0 and 1 are as in gate/up (lane quarter q owns
// block 4 g + q); the last group holds blocks 8 and 9, quarter q owning half
// q % 2 of block 8 + q / 2 for 4 MFMA steps (its 20 loaded bytes hold the
// whole block; the half's two code dwords are picked by q % 2).  The item's
// whole activation tile (64 rows x 1,280 bytes of h) sits in LDS at once:
// groups 0 and 1 in the gate/up layout at 0 and 32 KB, the last group at
// 64 KB (16 chunks per row, row groups of 2 KB, chunk c at position
// c ^ (r & 1)).  Every request goes out at the start: one wait, one barrier.
constexpr int PD_G2 = 2 * PG_ABYTES;                    // offset of the last group
constexpr int PF_LDS_D = PD_G2 + PF_M * 256;            // 81,920
static_assert(2 * PG_BLK + 2 == NB_D, "two whole groups and two blocks");
static_assert(PD_G2 + 4096 * 3 + 2048 + 128 * 15 + 16 * 8 == PF_LDS_D, "last fragment read ends at the end");

// Position of h column c (0..FF-1) in the down activation order: blocks 0..7
// as in the gate/up order (chunk 8 q + j of 256-column group b / 4, q = b % 4);
// blocks 8 and 9 in a last group of 128 positions, chunk 4 q + j for half
// q % 2 of block 8 + q / 2.  Element s of the chunk of MFMA step j holds
// column 16 (j / 2) + 4 (j % 2) + s / 2 + 8 (s % 2) of its block (or half).
__device__ inline int pd_pos_of_col(int c)
{
    const int b = c >> 6, r = c & 15;
    const int sj = (r >> 2) & 1, s = 2 * (r & 3) + (r >> 3);
    if (b < 2 * PG_BLK) {
        const int j = 2 * ((c >> 4) & 3) + sj;
        return 256 * (b >> 2) + 64 * (b & 3) + 8 * j + s;
    }
    const int q = 2 * (b - 2 * PG_BLK) + ((c >> 5) & 1);
    const int j = 2 * ((c >> 4) & 1) + sj;
    return 2 * (PG_GBYTES / 2) + 32 * q + 8 * j + s;   // after the 2 x 256 positions of groups 0, 1
}

// The down K loop, from registers and the resident activation tile.
template <int MS>
__device__ inline void pd_down_loop(const PgW w[3], uint32_t sel_c, uint32_t sel_d, uint32_t sel_c2,
                                    uint32_t sel_d2, bool upper, uint32_t ae, uint32_t ao,
                                    uint32_t ae2, uint32_t ao2, floatx4 acc[4][4])
{
    pg_group<0, MS>(ae, ao, w[0], sel_c, sel_d, acc);
    pg_group<1, MS>(ae, ao, w[1], sel_c, sel_d, acc);
    uint32_t d2[4], cw[4][4];
    pg_extract(w[2], sel_c2, sel_d2, d2, cw);
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {   // code dwords 2 (q % 2), 2 (q % 2) + 1 of the block
        cw[ns][0] = upper ? cw[ns][2] : cw[ns][0];
        cw[ns][1] = upper ? cw[ns][3] : cw[ns][1];
    }
    half8 af[2][4];
    pg_aread<0, 4096, MS>(ae2, af[0]);
    pg_await<MS>(af[0]);
    pg_step<0, 4096, 4, MS, 0>(ae2, ao2, d2, cw, af, acc);
    pg_step<0, 4096, 4, MS, 1>(ae2, ao2, d2, cw, af, acc);
    pg_step<0, 4096, 4, MS, 2>(ae2, ao2, d2, cw, af, acc);
    pg_step<0, 4096, 4, MS, 3>(ae2, ao2, d2, cw, af, acc);
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

// The activations carry a per-token power-of-two scale 2^k and h a second
// one, 2^hs (both 0 for rows whose largest |xhat| lies in [1, 8); see the prep
// kernel): gate and up come out of the MFMAs times 2^k and are divided by it
// before SiLU, h is stored times 2^hs so that it stays inside fp16's range at
// any input magnitude, and down's sums are divided by 2^hs again.  Every
// scaling is an exact power of two.  xexp[t] holds k in its low 16 bits and
// hs in its high 16 bits, both signed.
__device__ inline int pf_k(int v) { return (int)(int16_t)(v & 0xffff); }
__device__ inline int pf_hs(int v) { return v >> 16; }

// Threads 0..PF_M-1 (wave 0) put the packed exponents of item row tid (0 past
// the item's end) into kx and whether any is nonzero into kx[PF_M]; the
// caller's next barrier publishes them.  N-tile 0 also records each row's hs
// for the down kernel (hexp, in grouped order).
__device__ inline void pf_row_exps(const PfItem &it, int nt, const int32_t *__restrict__ slots,
                                   const int32_t *__restrict__ xexp, int32_t *__restrict__ hexp,
                                   int T, int *kx)
{
    const int tid = threadIdx.x;
    if (tid < PF_M) {
        int v = 0;
        if (tid < it.rows) {
            const int sl = slots[it.gp0 + tid];
            if (sl >= 0 && sl < T * K)
                v = xexp[sl / K];
            if (nt == 0)
                hexp[it.gp0 + tid] = pf_hs(v);
        }
        kx[tid] = v;
        const bool any = __ballot(v != 0) != 0;
        if (tid == 0)
            kx[PF_M] = any;
    }
}

// Work item `item` (rows of one expert, in grouped order) from the planner's
// record; ok = 0 past the list's end or for a record that fails the checks.
__device__ inline PfItem pf_item(int item, const int32_t *mlist, const int32_t *nitems, int T)
{
    PfItem it{0, 0, 0, 0};
    const int4 r = reinterpret_cast<const int4 *>(mlist)[item];   // padded: always in bounds
    if (item >= nitems[0] || !pf_rec_ok(r.x, r.y, r.z, T))
        return it;
    it.ok = 1;
    it.e = r.x;
    it.gp0 = r.y;
    it.rows = r.z;
    return it;
}

// Gate/up runs eight waves per workgroup, each on 16 FF rows (one gate and one
// up subtile), so that two workgroups per CU put four waves on every SIMD:
// while some wait at a group's loads or barrier, others compute.  Wave w
// requests the activations of row group w.
constexpr int PG_WAVES = 8;
constexpr int PG_THREADS = 64 * PG_WAVES;
constexpr int PG_NS = 2;                                // subtiles per wave
static_assert(PG_WAVES * 16 == PF_NT_G && PG_WAVES * 8 == PF_M, "a wave per 16 FF rows and 8 item rows");

// Activation requests of gate/up group g for this wave: 4 requests of 1 KB,
// request i filling row group w, chunk octet i.
struct PgAct8 {
    const uint8_t *row;   // row 8 w + lane % 8 (valid memory for every lane)
    uint32_t coff;        // byte offset of this lane's chunk in the octet
    __device__ void request(uint8_t *abuf, int g) const
    {
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds(row + PG_GBYTES * g + 128 * i + coff,
                                             abuf + (4 * w + i) * 1024, 16, 0, 0);
    }
};

__global__ __launch_bounds__(PG_THREADS, 4) void pf_gateup(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ slots,
    const int32_t *__restrict__ mlist, const int32_t *__restrict__ nitems,
    const __half *__restrict__ xperm, const int32_t *__restrict__ xexp, __half *__restrict__ hperm,
    int32_t *__restrict__ hexp, int T)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[PF_LDS_G];
    __shared__ int kx[PF_M + 1];
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int item = 8 * (idx / PF_NTILES_G) + xcd;
    const int nt = idx % PF_NTILES_G;
    const PfItem it = pf_item(item, mlist, nitems, T);
    if (!it.ok)
        return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int jw = nt * PF_NT_G + 16 * wave;   // this wave's first FF row
    pf_row_exps(it, nt, slots, xexp, hexp, T, kx);
    const uint8_t *blob = blobs + (size_t)it.e * BLOB;
    // Activation row this lane requests (rows past the item's end read its
    // first row; their results are never stored): row 8 w + lane % 8, chunk
    // (lane / 8) ^ (w % 2) of each octet.
    PgAct8 act;
    {
        const int r = 8 * wave + (lane & 7);
        const int sl = slots[it.gp0 + (r < it.rows ? r : 0)];
        const int t = (sl >= 0 && sl < T * K) ? sl / K : 0;
        act.row = reinterpret_cast<const uint8_t *>(xperm + (size_t)t * H);
        act.coff = 16 * ((lane >> 3) ^ (wave & 1));
    }
    // Weight bytes: subtile 0 is gate rows jw + lane % 16, subtile 1 the same
    // up rows; quarter q loads from the dword at or below block q's start.
    const int q = lane >> 4, odd = q & 1;
    uint32_t woff[PG_NS];
#pragma unroll
    for (int ns = 0; ns < PG_NS; ++ns)
        woff[ns] = (uint32_t)((ns ? MAT : 0) + (size_t)(jw + (lane & 15)) * ROW_G + BB * q - 2 * odd);
    const uint32_t sel_c = odd ? 0x07060504u : 0x05040302u;   // code dword i: bytes 2..5 or 4..7 of L[i], L[i+1]
    const uint32_t sel_d = odd ? 0x03020302u : 0x01000100u;   // (d, d) from bytes 0, 1 or 2, 3 of L[0]
    // Fragment reads: row 16 mi + lane % 16 (row group 2 mi + b), chunk 8 q + j at
    // position 8 q + (j ^ b) of the row group.
    const int b = (lane >> 3) & 1;
    const uint32_t abase = lds_addr(lds) + (32 * b + 8 * q) * 128 + 16 * (lane & 7);
    const uint32_t ae = abase + 128 * b, ao = abase - 128 * b;
    floatx4 acc[PG_NS][4];
#pragma unroll
    for (int ns = 0; ns < PG_NS; ++ns)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            acc[ns][mi] = (floatx4){0.f, 0.f, 0.f, 0.f};
    // one straight-line loop per number of 16-row groups holding item rows
    switch ((it.rows + 15) >> 4) {
    case 1:
        pg_gateup_loop<1, PG_NS>(blob, woff, act, lds, ae, ao, sel_c, sel_d, acc);
        break;
    case 2:
        pg_gateup_loop<2, PG_NS>(blob, woff, act, lds, ae, ao, sel_c, sel_d, acc);
        break;
    case 3:
        pg_gateup_loop<3, PG_NS>(blob, woff, act, lds, ae, ao, sel_c, sel_d, acc);
        break;
    default:
        pg_gateup_loop<4, PG_NS>(blob, woff, act, lds, ae, ao, sel_c, sel_d, acc);
        break;
    }
    __syncthreads();   // kx
    // Epilogue: h = silu(g) * u for FF row jw + lane%16, stored times 2^hs:
    // g = acc 2^-k, and silu(g) acc_u = silu(g) u 2^k.  Items whose rows are
    // all unscaled skip the exponents.
    const bool scaled = kx[PF_M] != 0;
    const int j = jw + (lane & 15);
    const int col = pd_pos_of_col(j);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * mi + 4 * (lane >> 4) + r;
            if (m < it.rows) {
                float h;
                if (scaled) {
                    const int v = kx[m], k = pf_k(v);
                    const float g = ldexpf(acc[0][mi][r], -k);
                    h = ldexpf(pf_silu_mul(g, acc[1][mi][r]), pf_hs(v) - k);
                } else {
                    h = pf_silu_mul(acc[0][mi][r], acc[1][mi][r]);
                }
                hperm[(size_t)(it.gp0 + m) * FF + col] = __float2half_rn(h);
            }
        }
    }
}

__global__ __launch_bounds__(PF_THREADS, 2) void pf_down(
    const uint8_t *__restrict__ blobs, const int32_t *__restrict__ slots,
    const int32_t *__restrict__ mlist, const int32_t *__restrict__ nitems,
    const int32_t *__restrict__ hexp, const __half *__restrict__ hperm, float *__restrict__ out,
    int T)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[PF_LDS_D];
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int item = 8 * (idx / PF_NTILES_D) + xcd;
    const int nt = idx % PF_NTILES_D;
    const PfItem it = pf_item(item, mlist, nitems, T);
    if (!it.ok)
        return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rw = nt * PF_NT_D + 64 * wave;   // this wave's first output row
    // The slot and the h exponent of this lane's 16 output rows, loaded now so
    // the epilogue does not wait for them (rows past the item's end read its
    // first row and are never stored).
    int osl[4][4], ohs[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * mi + 4 * (lane >> 4) + r;
            const int gp = it.gp0 + (m < it.rows ? m : 0);
            osl[mi][r] = slots[gp];
            ohs[mi][r] = hexp[gp];
        }
    }
    // Activation rows (past the item's end: its first row, never stored).
    PgAct act;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 16 * wave + 8 * h + (lane & 7);
        act.row[h] = reinterpret_cast<const uint8_t *>(hperm + (size_t)(it.gp0 + (r < it.rows ? r : 0)) * FF);
        act.coff[h] = 16 * ((lane >> 3) ^ h);
    }
    act.request(lds, 0);
    act.request(lds + PG_ABYTES, 1);
    {   // last group: request i fills row group 2 w + i / 2, chunk octet i % 2
        const int w = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds(act.row[i >> 1] + 2 * PG_GBYTES + 128 * (i & 1) + act.coff[i >> 1],
                                             lds + PD_G2 + (4 * w + i) * 1024, 16, 0, 0);
    }
    // Weight bytes of output rows rw + 16 ns + lane % 16: quarter q loads
    // from the dword at or below its block's start (groups 0, 1: block
    // 4 g + q; last group: block 8 + q / 2).
    const int q = lane >> 4;
    const uint8_t *wbase = blobs + (size_t)it.e * BLOB + 2 * MAT;
    PgW wr[3];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
        const uint32_t row = (uint32_t)(rw + 16 * ns + (lane & 15)) * ROW_D;
#pragma unroll
        for (int g = 0; g < 3; ++g) {
            const uint32_t off = row + (g < 2 ? PG_BLK * BB * g + BB * q - 2 * (q & 1)
                                              : 2 * PG_BLK * BB + (BB - 2) * (q >> 1));
            wr[g].lo[ns] = *reinterpret_cast<const u32x4 *>(wbase + off);
            wr[g].hi[ns] = *reinterpret_cast<const uint32_t *>(wbase + off + 16);
        }
    }
    pg_wait_all(wr[0]);
    pg_wait_all(wr[1]);
    pg_wait_all(wr[2]);
    __builtin_amdgcn_s_barrier();   // every wave's activations have landed
    const int odd = q & 1, odd2 = q >> 1;
    const uint32_t sel_c = odd ? 0x07060504u : 0x05040302u, sel_d = odd ? 0x03020302u : 0x01000100u;
    const uint32_t sel_c2 = odd2 ? 0x07060504u : 0x05040302u, sel_d2 = odd2 ? 0x03020302u : 0x01000100u;
    const int b = (lane >> 3) & 1;
    const uint32_t abase = lds_addr(lds) + (32 * b + 8 * q) * 128 + 16 * (lane & 7);
    const uint32_t ae = abase + 128 * b, ao = abase - 128 * b;
    const uint32_t abase2 = lds_addr(lds) + PD_G2 + 2048 * b + 512 * q + 16 * (lane & 7);
    const uint32_t ae2 = abase2 + 128 * b, ao2 = abase2 - 128 * b;
    floatx4 acc[4][4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            acc[ns][mi] = (floatx4){0.f, 0.f, 0.f, 0.f};
    switch ((it.rows + 15) >> 4) {
    case 1:
        pd_down_loop<1>(wr, sel_c, sel_d, sel_c2, sel_d2, odd, ae, ao, ae2, ao2, acc);
        break;
    case 2:
        pd_down_loop<2>(wr, sel_c, sel_d, sel_c2, sel_d2, odd, ae, ao, ae2, ao2, acc);
        break;
    case 3:
        pd_down_loop<3>(wr, sel_c, sel_d, sel_c2, sel_d2, odd, ae, ao, ae2, ao2, acc);
        break;
    default:
        pd_down_loop<4>(wr, sel_c, sel_d, sel_c2, sel_d2, odd, ae, ao, ae2, ao2, acc);
        break;
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * mi + 4 * (lane >> 4) + r;
            if (m < it.rows) {
                const int s = osl[mi][r];
                const int sh = -ohs[mi][r];   // h was stored times 2^hs
                if (s >= 0 && s < T * K) {
#pragma unroll
                    for (int ns = 0; ns < 4; ++ns)
                        out[(size_t)s * H + rw + 16 * ns + (lane & 15)] = ldexpf(acc[ns][mi][r], sh);
                }
            }
        }
    }
}

hipError_t launch_prefill_experts(const uint8_t *blobs, const int32_t *offsets,
                                  const int32_t *slots, const int32_t *active,
                                  const int32_t *mlist, const int32_t *nitems, int max_items,
                                  const __half *xperm, const int32_t *xexp, __half *hperm,
                                  int32_t *hexp, float *out, int T, hipEvent_t ev0, hipEvent_t ev1,
                                  hipStream_t st)
{
    const int groups = (max_items + 7) / 8;
    const dim3 grid_g(8 * PF_NTILES_G * groups), block(PG_THREADS);
    if (ev0) {   // timed launch: the events carry the dispatch's own start and end
        void *args[] = {&blobs, &slots, &mlist, &nitems, &xperm, &xexp, &hperm, &hexp, &T};
        const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(&pf_gateup), grid_g,
                                                block, args, 0, st, ev0, ev1, 0);
        if (e != hipSuccess)
            return e;
    } else {
        hipLaunchKernelGGL(pf_gateup, grid_g, block, 0, st, blobs, slots, mlist, nitems, xperm,
                           xexp, hperm, hexp, T);
    }
    hipLaunchKernelGGL(pf_down, dim3(8 * PF_NTILES_D * groups), dim3(PF_THREADS), 0, st, blobs,
                       slots, mlist, nitems, hexp, hperm, out, T);
    return hipGetLastError();
}

} // namespace strata
