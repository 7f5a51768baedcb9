// experts_decode.hip -- SwiGLU experts for decode-sized T (verify windows).
//
// The expert FFN of every routed (token, expert) pair: g = W_g x, u = W_u x,
// h = silu(g) * u, o = W_d h, on Q2_0 weights ("Strata in the source...",
// section "The byte budget, in code": gate, up and down of 2,560 x 640 in
// 18-byte blocks).  Tokens are grouped per expert first, so each active
// expert's blob is read once per call however many tokens of the window chose
// it (the window dedup of section "The plan: three destinations per expert").
//
// One launch, dec_experts, runs three kinds of workgroup.  Each puts one
// weight row on each lane: the workgroup reads its rows with coalesced 16-byte
// loads into LDS, then every lane walks its own row block by block.  The 16
// code bytes give two nibble-masked dwords per 16 codes, and v_dot8
// multiplies them with the token's 16-bit activation digits (quant.hpp).  The
// activation operand is the same for the 16 lanes of a row, so it reaches them
// by a DPP row broadcast inside the v_dot8: per lane, two registers carry a
// whole 64-value block.
//
//  gate/up item  (active expert, 16 FF rows): the 16 gate and 16 up rows
//              (23 KB).  256 threads = 4 waves; lane (r = lane / 16, l) takes
//              row l of gate (r even) or up (r odd) and block columns
//              5 s .. 5 s + 4 with s = 2 w + r / 2.  Partial sums meet in a
//              fixed order; wave 0 forms h = silu(g) * u for the 16 rows and
//              quantises them as one 16-value segment.  A shared expert's
//              tokens go two at a time (codes split once).  Workgroups of
//              23 KB LDS run six to a CU.
//  down group  four items (active expert, 32 output rows), one per wave:
//              lane (r, l) takes row 16 (r % 2) + l and block columns
//              2 j + r / 2; the two halves of each row are added and the
//              row's value written per slot.  A down group waits for its
//              expert's gate/up items (a counter per active expert).  In a
//              layer call it also finishes the combine (the last slot of a
//              token's rows to be done sums the token's K slots).
//  lookahead   only for strata_moe_layer_lookahead: reads the next layer's
//              predicted experts, line by line, and writes nothing.
// Every sum has a fixed order, so results are bitwise reproducible and do not
// depend on the other tokens of the call.
#include "common.hpp"
#include "quant.hpp"
#include "route_token.hpp"
#include <hip/hip_ext.h>

namespace strata {

// ------------------------------------------------------------------ gate / up
constexpr int DG_WAVES = 4;
constexpr int DG_THREADS = 64 * DG_WAVES;
constexpr int DG_SEG = 16;                          // FF rows per item (one h segment)
constexpr int DG_SEGS = FF / DG_SEG;                // 40
constexpr int DG_ROWS = 2 * DG_SEG;                 // 16 gate + 16 up rows
constexpr int DG_CPR = ROW_G / 16;                  // 45 16-byte chunks per row
constexpr int DG_CHUNKS = DG_ROWS * DG_CPR;         // 1,440
constexpr int DG_RS = ROW_G / 4 + 1;                // LDS row stride in dwords (181, odd)
constexpr int DG_COLS = 5;                          // block columns per lane
static_assert(DG_WAVES * 2 * DG_COLS == NB_G, "4 waves x 2 column streams x 5 block columns");
static_assert(DG_CHUNKS > 5 * DG_THREADS && DG_CHUNKS <= 6 * DG_THREADS, "six loads per thread");

// Records of the grouping for the decode kernels: erec[0].x = number of active
// experts, erec[1 + a] = {expert, first grouped slot, token count, first slot}.
__device__ inline int active_count(const int4 *erec, int T)
{
    return min(max(erec[0].x, 0), min(T * K, E));
}

// Activation operands of one token for lane column stream s (block columns
// 5 s + j): the digit pairs (dword l, dword 16 + l) of each column, and in
// lane j < 5 of each 16-lane row the column's scale times the inverse RMS and
// its -sum q (handed to the row by DPP broadcast).
struct XOps {
    uint2 d[DG_COLS];
    float sc;
    int nq;
};

__device__ inline XOps load_xops(const XQ &xq, int t, int s, int l)
{
    XOps o;
    const size_t xb = (size_t)t * XBLK + DG_COLS * s;
    const uint2 *dp = reinterpret_cast<const uint2 *>(xq.dig + xb * BLK_DWORDS) + l;
#pragma unroll
    for (int j = 0; j < DG_COLS; ++j)
        o.d[j] = dp[16 * j];
    const int j = l < DG_COLS ? l : 0;
    o.sc = xq.scale[xb + j] * xq.inv_rms[t];
    o.nq = xq.nsum[xb + j];
    return o;
}

// One block of a row held in LDS: the 5 dwords from p hold it; sel and sh
// place the codes and the scale (they depend on the column parity); J is the
// block's index among the lane's columns.
template <int J>
__device__ inline float block_dot(const uint32_t *p, uint32_t sel, uint32_t sh, uint2 D,
                                  const XOps &xo)
{
    const uint32_t v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3], v4 = p[4];
    const Codes c = split_codes(__builtin_amdgcn_perm(v1, v0, sel), __builtin_amdgcn_perm(v2, v1, sel),
                                __builtin_amdgcn_perm(v3, v2, sel), __builtin_amdgcn_perm(v4, v3, sel));
    const float d = half_bits_to_float(v0 >> sh);
    const int a = block_codes_dot(c, D.x, D.y, row_bcast_i<J>(xo.nq));
    return (d * row_bcast_f<J>(xo.sc)) * (float)a;
}

// The same block against two tokens' operands: the codes are split once and
// each token's result is the expression block_dot computes for it alone.
template <int J>
__device__ inline float2 block_dot2(const uint32_t *p, uint32_t sel, uint32_t sh, uint2 DA,
                                    uint2 DB, const XOps &xa, const XOps &xb)
{
    const uint32_t v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3], v4 = p[4];
    const Codes c = split_codes(__builtin_amdgcn_perm(v1, v0, sel), __builtin_amdgcn_perm(v2, v1, sel),
                                __builtin_amdgcn_perm(v3, v2, sel), __builtin_amdgcn_perm(v4, v3, sel));
    const float d = half_bits_to_float(v0 >> sh);
    const int a = block_codes_dot(c, DA.x, DA.y, row_bcast_i<J>(xa.nq));
    const int b = block_codes_dot(c, DB.x, DB.y, row_bcast_i<J>(xb.nq));
    return make_float2((d * row_bcast_f<J>(xa.sc)) * (float)a, (d * row_bcast_f<J>(xb.sc)) * (float)b);
}

// Per-call counters of the fused kernel (zeroed by the router / prep kernel):
// sync[1 + SYNC_STRIDE * a] counts the finished gate/up items of active expert a.
// Status bits the kernel ORs into the caller's status word.
constexpr int ST_WAIT_GAVE_UP = STRATA_STATUS_WAIT_TIMEOUT;

// h values are stored and read at agent scope (coherent across the XCDs'
// L2 caches): the down part of the same launch reads them.
__device__ inline void store_h(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0: h = silu(g) * u of one token's 16 FF rows from the partial sums
// part [DG_WAVES][DG_ROWS], quantised and stored as segment seg of slot (at
// agent scope when the down part of the same launch reads it, FUSED; plain
// stores when a later launch does).
template <bool FUSED>
__device__ inline void emit_h(const float (*part)[DG_ROWS], int slot, int seg, const HQ &hq)
{
    const int lane = threadIdx.x & 63;
    const int j = lane & 31;
    const float v = ((part[0][j] + part[1][j]) + part[2][j]) + part[3][j];
    const float u = __shfl(v, (lane & 15) + DG_SEG, 64);
    const float h = lane < DG_SEG ? v / (1.f + expf(-v)) * u : 0.f;
    const QuantOut qo = quant_lanes<false>(h);
    if (lane == 12 || lane == 13) {
        uint32_t *blk = hq.dig + ((size_t)slot * HBLK + (seg >> 2)) * BLK_DWORDS;
#pragma unroll
        for (int i = 0; i < 4; ++i)
        {
            if (FUSED)
                store_h(blk + dig_pos(8 * (seg & 3) + 4 * (lane - 12) + i), qo.pk[i]);
            else
                blk[dig_pos(8 * (seg & 3) + 4 * (lane - 12) + i)] = qo.pk[i];
        }
    }
    if (lane == 0) {
        if (FUSED) {
            store_h(reinterpret_cast<uint32_t *>(hq.scale) + (size_t)slot * HSEG16 + seg,
                    __float_as_uint(qo.scale));
            store_h(reinterpret_cast<uint32_t *>(hq.nsum) + (size_t)slot * HSEG16 + seg,
                    (uint32_t)(-qo.sum));
        } else {
            hq.scale[(size_t)slot * HSEG16 + seg] = qo.scale;
            hq.nsum[(size_t)slot * HSEG16 + seg] = -qo.sum;
        }
    }
}

// The 23,040 bytes of one gate/up item in flight in a workgroup's registers:
// thread tid holds 16-byte chunks tid + 256 i, i = 0..5 (the sixth only where
// it exists).  Chunk q < 720 is of the 16 gate rows, the rest of the 16 up
// rows; it goes to LDS row q / 45 at dword 4 (q % 45).
struct GuChunks {
    uint4 p[6];
};

// Request segment seg (FF rows 16 seg .. + 15) of expert e's gate and up rows.
__device__ inline GuChunks gu_request(const uint8_t *__restrict__ blobs, int e, int seg)
{
    const int tid = threadIdx.x;
    const uint8_t *blob = blobs + (size_t)e * BLOB + (size_t)seg * DG_SEG * ROW_G;
    const uint4 *g = reinterpret_cast<const uint4 *>(blob);
    const uint4 *u = reinterpret_cast<const uint4 *>(blob + MAT);
    GuChunks c;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int q = tid + DG_THREADS * i;
        c.p[i] = q < DG_CHUNKS / 2 ? g[q] : u[q - DG_CHUNKS / 2];
    }
    const bool has5 = tid + 5 * DG_THREADS < DG_CHUNKS;
    c.p[5] = has5 ? u[tid + 5 * DG_THREADS - DG_CHUNKS / 2] : make_uint4(0, 0, 0, 0);
    return c;
}

// Write the chunks to LDS wl [DG_ROWS][DG_RS] dwords (the caller's next
// barrier publishes them).
__device__ inline void gu_stage(const GuChunks &c, uint32_t *wl)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const int q = tid + DG_THREADS * i;
        if (i < 5 || q < DG_CHUNKS) {
            uint32_t *d = wl + (q / DG_CPR) * DG_RS + 4 * (q % DG_CPR);
            d[0] = c.p[i].x;
            d[1] = c.p[i].y;
            d[2] = c.p[i].z;
            d[3] = c.p[i].w;
        }
    }
}

template <bool FUSED>
__device__ void gateup_compute(int4 rec, int seg, int a, const int32_t *__restrict__ slots,
                               const XQ &xq, const HQ &hq, int T, uint32_t *wl,
                               float (*part)[DG_ROWS], int32_t *gdone, XOps xo);

// One gate/up item, segment seg (FF rows 16 seg .. + 15) of the active
// expert with record rec = {expert, first grouped slot, token count, first
// slot}: LDS wl [DG_ROWS][DG_RS] dwords and part [2 DG_WAVES][DG_ROWS].
// FUSED: h at agent scope and the item counted in gdone[SYNC_STRIDE a] for the
// down groups of the same launch.
template <bool FUSED>
__device__ void gateup_item(int4 rec, int seg, int a, const uint8_t *__restrict__ blobs,
                            const int32_t *__restrict__ slots, const XQ &xq, const HQ &hq, int T,
                            uint32_t *wl, float (*part)[DG_ROWS], int32_t *gdone)
{
    const int nslot = T * K;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int s = 2 * wave + ((lane >> 4) >> 1);       // column stream: columns 5s .. 5s+4
    const int slot = rec.w;
    // token 0's operands are in flight with the weights
    const XOps xo = load_xops(xq, slot >= 0 && slot < nslot ? slot / K : 0, s, lane & 15);
    gu_stage(gu_request(blobs, rec.x, seg), wl);
    gateup_compute<FUSED>(rec, seg, a, slots, xq, hq, T, wl, part, gdone, xo);
}

// The item's arithmetic once its rows are written to LDS (the barrier below
// publishes them): xo holds token rec.w / K's operands for this lane.
template <bool FUSED>
__device__ void gateup_compute(int4 rec, int seg, int a, const int32_t *__restrict__ slots,
                               const XQ &xq, const HQ &hq, int T, uint32_t *wl,
                               float (*part)[DG_ROWS], int32_t *gdone, XOps xo)
{
    const int nslot = T * K;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = lane >> 4, l = lane & 15;
    const int s = 2 * wave + (r >> 1);                 // column stream: columns 5s .. 5s+4
    int slot = rec.w;
    // Block column 5 s + j starts at byte 90 s + 18 j of the row; its 5-dword
    // window starts 2 bytes earlier when the column is odd.
    const uint32_t *row = wl + ((r & 1) * DG_SEG + l) * DG_RS;
    const int odd_s = s & 1;
    const uint32_t sel_e = odd_s ? 0x07060504u : 0x05040302u;   // columns with j even
    const uint32_t sel_o = odd_s ? 0x05040302u : 0x07060504u;   // columns with j odd
    const uint32_t sh_e = odd_s ? 16u : 0u, sh_o = odd_s ? 0u : 16u;
    const uint32_t *w0 = row + (90 * s - 2 * odd_s) / 4;         // j = 0
    const uint32_t *w1 = row + (90 * s + 18 - 2 * (1 - odd_s)) / 4;
    const uint32_t *w2 = row + (90 * s + 36 - 2 * odd_s) / 4;
    const uint32_t *w3 = row + (90 * s + 54 - 2 * (1 - odd_s)) / 4;
    const uint32_t *w4 = row + (90 * s + 72 - 2 * odd_s) / 4;
    __syncthreads();
    // Tokens two at a time: the weights of a block are decoded once for both,
    // and each token's arithmetic is what it gets alone.  part[w] holds the
    // first token's partial sums, part[DG_WAVES + w] the second's.
    for (int ti = 0; ti < rec.z; ti += 2) {
        const bool two = ti + 1 < rec.z;   // uniform per workgroup
        if (ti > 0) {
            slot = slots[rec.y + ti];
            xo = load_xops(xq, slot >= 0 && slot < nslot ? slot / K : 0, s, l);
        }
        int slot2 = -1;
        XOps xo2 = xo;
        if (two) {
            slot2 = slots[rec.y + ti + 1];
            xo2 = load_xops(xq, slot2 >= 0 && slot2 < nslot ? slot2 / K : 0, s, l);
        }
        float acc, acc2 = 0.f;
        if (two) {
            float2 t = block_dot2<0>(w0, sel_e, sh_e, xo.d[0], xo2.d[0], xo, xo2);
            acc = t.x;
            acc2 = t.y;
            t = block_dot2<1>(w1, sel_o, sh_o, xo.d[1], xo2.d[1], xo, xo2);
            acc += t.x;
            acc2 += t.y;
            t = block_dot2<2>(w2, sel_e, sh_e, xo.d[2], xo2.d[2], xo, xo2);
            acc += t.x;
            acc2 += t.y;
            t = block_dot2<3>(w3, sel_o, sh_o, xo.d[3], xo2.d[3], xo, xo2);
            acc += t.x;
            acc2 += t.y;
            t = block_dot2<4>(w4, sel_e, sh_e, xo.d[4], xo2.d[4], xo, xo2);
            acc += t.x;
            acc2 += t.y;
            acc2 += __shfl_xor(acc2, 32, 64);
        } else {
            acc = block_dot<0>(w0, sel_e, sh_e, xo.d[0], xo);
            acc += block_dot<1>(w1, sel_o, sh_o, xo.d[1], xo);
            acc += block_dot<2>(w2, sel_e, sh_e, xo.d[2], xo);
            acc += block_dot<3>(w3, sel_o, sh_o, xo.d[3], xo);
            acc += block_dot<4>(w4, sel_e, sh_e, xo.d[4], xo);
        }
        acc += __shfl_xor(acc, 32, 64);   // the wave's two column streams
        if (ti > 0)
            __syncthreads();   // wave 0 is done with the previous tokens' partials
        if (lane < DG_ROWS) {
            part[wave][lane] = acc;
            if (two)
                part[DG_WAVES + wave][lane] = acc2;
        }
        __syncthreads();
        if (wave == 0) {
            if (slot >= 0 && slot < nslot)   // only a corrupt grouping fails this
                emit_h<FUSED>(part, slot, seg, hq);
            if (two && slot2 >= 0 && slot2 < nslot)
                emit_h<FUSED>(part + DG_WAVES, slot2, seg, hq);
        }
    }
    if (FUSED && wave == 0) {   // every h value of the item is in memory: count the item
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (lane == 0)
            __hip_atomic_fetch_add(gdone + SYNC_STRIDE * a, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ----------------------------------------------------------------------- down
constexpr int DD_WAVES = 4;                         // items per workgroup
constexpr int DD_ROWS = 32;                         // output rows per item
constexpr int DD_ITEMS_PER_E = H / DD_ROWS;         // 80
constexpr int DD_CHUNKS = DD_ROWS * ROW_D / 16;     // 360 16-byte chunks per item
constexpr int DD_RS = ROW_D / 4;                    // 45 dwords per row (odd: no bank conflicts)
static_assert(DD_CHUNKS > 5 * 64 && DD_CHUNKS <= 6 * 64, "six loads per lane");

// Operands of one slot's h for lane column set c0 = r / 2 (block columns
// 2 j + c0): per column the digit pair, and in lane l of each row the scale
// and -sum q of segment 4 (2 j + c0) + k for index 4 j + k = 16 m + l (m = 0, 1).
struct HOps {
    uint2 d[5];
    float sh0, sh1;
    int nq0, nq1;
};

template <class V> __device__ inline V load_h(const V *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// FUSED: agent-scope loads (h written in the same launch); else plain ones.
template <bool FUSED> __device__ inline unsigned long long ld_h(const unsigned long long *p)
{
    if (FUSED)
        return load_h(p);
    return *p;
}
template <bool FUSED> __device__ inline float ld_h(const float *p) { return FUSED ? load_h(p) : *p; }
template <bool FUSED> __device__ inline int32_t ld_h(const int32_t *p) { return FUSED ? load_h(p) : *p; }

template <bool FUSED = true>
__device__ inline HOps load_hops(const HQ &hq, int slot, int c0, int l)
{
    HOps o;
    const unsigned long long *dp =
        reinterpret_cast<const unsigned long long *>(hq.dig + (size_t)slot * HBLK * BLK_DWORDS) + l;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const unsigned long long v = ld_h<FUSED>(dp + 16 * (2 * j + c0));
        o.d[j] = make_uint2((uint32_t)v, (uint32_t)(v >> 32));
    }
    const int seg0 = 4 * (2 * (l >> 2) + c0) + (l & 3);   // index l: j = l / 4, k = l % 4
    const int seg1 = 4 * (2 * 4 + c0) + (l & 3);          // index 16 + l (l < 4): j = 4
    const size_t sb = (size_t)slot * HSEG16;
    o.sh0 = ld_h<FUSED>(hq.scale + sb + seg0);
    o.nq0 = ld_h<FUSED>(hq.nsum + sb + seg0);
    o.sh1 = l < 4 ? ld_h<FUSED>(hq.scale + sb + seg1) : 0.f;
    o.nq1 = l < 4 ? ld_h<FUSED>(hq.nsum + sb + seg1) : 0;
    return o;
}

// ACC += (scale of lane N of the row) * V
#define STRATA_FMA_BCAST(ACC, SH, V, N)                                                            \
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"                    \
        : "+v"(ACC)                                                                                \
        : "v"(SH), "v"(V), "i"(N))

// One down block from the 5 dwords at p: sel and sh place the codes and the
// scale (they depend on the block column parity, which is fixed per lane).
// Its four 16-value segments have their scales at broadcast indices N..N+3.
template <int N>
__device__ inline float down_block(const uint32_t *p, uint32_t sel, uint32_t sh, uint2 D, float shr,
                                   int nqr)
{
    const uint32_t v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3], v4 = p[4];
    const Codes c = split_codes(__builtin_amdgcn_perm(v1, v0, sel), __builtin_amdgcn_perm(v2, v1, sel),
                                __builtin_amdgcn_perm(v3, v2, sel), __builtin_amdgcn_perm(v4, v3, sel));
    const float d = half_bits_to_float(v0 >> sh);
    const Quad qd = quarters_codes_dot(c, D.x, D.y);
    float bacc = 0.f;
    const float f0 = (float)(qd.q[0] + row_bcast_i<N>(nqr));
    STRATA_FMA_BCAST(bacc, shr, f0, N);
    const float f1 = (float)(qd.q[1] + row_bcast_i<N + 1>(nqr));
    STRATA_FMA_BCAST(bacc, shr, f1, N + 1);
    const float f2 = (float)(qd.q[2] + row_bcast_i<N + 2>(nqr));
    STRATA_FMA_BCAST(bacc, shr, f2, N + 2);
    const float f3 = (float)(qd.q[3] + row_bcast_i<N + 3>(nqr));
    STRATA_FMA_BCAST(bacc, shr, f3, N + 3);
    return d * bacc;
}

// down_block against two slots' h: the codes are split once and each slot's
// result is the expression down_block computes for it alone.
template <int N>
__device__ inline float2 down_block2(const uint32_t *p, uint32_t sel, uint32_t sh, uint2 DA,
                                     uint2 DB, float shrA, int nqrA, float shrB, int nqrB)
{
    const uint32_t v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3], v4 = p[4];
    const Codes c = split_codes(__builtin_amdgcn_perm(v1, v0, sel), __builtin_amdgcn_perm(v2, v1, sel),
                                __builtin_amdgcn_perm(v3, v2, sel), __builtin_amdgcn_perm(v4, v3, sel));
    const float d = half_bits_to_float(v0 >> sh);
    const Quad qa = quarters_codes_dot(c, DA.x, DA.y);
    const Quad qb = quarters_codes_dot(c, DB.x, DB.y);
    float ba = 0.f, bb = 0.f;
    const float a0 = (float)(qa.q[0] + row_bcast_i<N>(nqrA));
    STRATA_FMA_BCAST(ba, shrA, a0, N);
    const float b0 = (float)(qb.q[0] + row_bcast_i<N>(nqrB));
    STRATA_FMA_BCAST(bb, shrB, b0, N);
    const float a1 = (float)(qa.q[1] + row_bcast_i<N + 1>(nqrA));
    STRATA_FMA_BCAST(ba, shrA, a1, N + 1);
    const float b1 = (float)(qb.q[1] + row_bcast_i<N + 1>(nqrB));
    STRATA_FMA_BCAST(bb, shrB, b1, N + 1);
    const float a2 = (float)(qa.q[2] + row_bcast_i<N + 2>(nqrA));
    STRATA_FMA_BCAST(ba, shrA, a2, N + 2);
    const float b2 = (float)(qb.q[2] + row_bcast_i<N + 2>(nqrB));
    STRATA_FMA_BCAST(bb, shrB, b2, N + 2);
    const float a3 = (float)(qa.q[3] + row_bcast_i<N + 3>(nqrA));
    STRATA_FMA_BCAST(ba, shrA, a3, N + 3);
    const float b3 = (float)(qb.q[3] + row_bcast_i<N + 3>(nqrB));
    STRATA_FMA_BCAST(bb, shrB, b3, N + 3);
    return make_float2(d * ba, d * bb);
}

// The five blocks 2 j + c0 of a row; their windows start at dwords 9 j (an
// odd column's window starts 2 bytes before its scale).
__device__ inline float down_row(const uint32_t *row, int c0, const HOps &ho)
{
    const uint32_t sel = c0 ? 0x07060504u : 0x05040302u;
    const uint32_t sh = c0 ? 16u : 0u;
    float acc = down_block<0>(row, sel, sh, ho.d[0], ho.sh0, ho.nq0);
    acc += down_block<4>(row + 9, sel, sh, ho.d[1], ho.sh0, ho.nq0);
    acc += down_block<8>(row + 18, sel, sh, ho.d[2], ho.sh0, ho.nq0);
    acc += down_block<12>(row + 27, sel, sh, ho.d[3], ho.sh0, ho.nq0);
    acc += down_block<0>(row + 36, sel, sh, ho.d[4], ho.sh1, ho.nq1);
    return acc;
}

// down_row for two slots.
__device__ inline float2 down_row2(const uint32_t *row, int c0, const HOps &a, const HOps &b)
{
    const uint32_t sel = c0 ? 0x07060504u : 0x05040302u;
    const uint32_t sh = c0 ? 16u : 0u;
    float2 acc = down_block2<0>(row, sel, sh, a.d[0], b.d[0], a.sh0, a.nq0, b.sh0, b.nq0);
    float2 t = down_block2<4>(row + 9, sel, sh, a.d[1], b.d[1], a.sh0, a.nq0, b.sh0, b.nq0);
    acc.x += t.x;
    acc.y += t.y;
    t = down_block2<8>(row + 18, sel, sh, a.d[2], b.d[2], a.sh0, a.nq0, b.sh0, b.nq0);
    acc.x += t.x;
    acc.y += t.y;
    t = down_block2<12>(row + 27, sel, sh, a.d[3], b.d[3], a.sh0, a.nq0, b.sh0, b.nq0);
    acc.x += t.x;
    acc.y += t.y;
    t = down_block2<0>(row + 36, sel, sh, a.d[4], b.d[4], a.sh1, a.nq1, b.sh1, b.nq1);
    acc.x += t.x;
    acc.y += t.y;
    return acc;
}

// The layer's combine, fused: when the counters cdone are given, the wave
// that finishes the last of token t's K slots for a 32-row chunk sums them in
// routing order, y_t = sum_k w[t][k] * out[t*K + k] (the fma order of
// combine_kernel), stores y and/or adds it to the residual x.  The per-slot
// rows are written and read with agent-scope (XCD-coherent) accesses, and a
// wave's rows are complete in memory before it counts its slot.
struct Combine {
    int32_t *cdone;     // [T][H/32] zeroed by the router, or NULL (no combine)
    const float *w;     // [T][K]
    float *y;           // [T][H] or NULL
    float *res;         // [T][H] or NULL: res += y
};

// A wave's output rows ch * 32 .. + 31 of one slot (lanes < 32 hold them):
// stored, and -- when the combine is fused -- counted, and the wave that
// completes a token's K slots for these rows writes their weighted sum.
__device__ inline void finish_slot(int slot, float acc, int ch, float *__restrict__ out, int T,
                                   const Combine &cb)
{
    const int lane = threadIdx.x & 63;
    if (slot < 0 || slot >= T * K)
        return;   // only a corrupt grouping gets here; uniform per wave
    float *orow = out + (size_t)slot * H + ch * DD_ROWS;
    if (!cb.cdone) {
        if (lane < DD_ROWS)
            orow[lane] = acc;
        return;
    }
    if (lane < DD_ROWS)
        __hip_atomic_store(orow + lane, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the rows are in memory
    const int t = slot / K;
    int done = 0;
    if (lane == 0)
        done = __hip_atomic_fetch_add(cb.cdone + (size_t)t * (H / DD_ROWS) + ch, 1,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    done = __shfl(done, 0, 64);
    if (done != K - 1)
        return;
    // the last of the token's slots for these rows: combine them
    if (lane < DD_ROWS) {
        const int r0 = ch * DD_ROWS + lane;
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float o = __hip_atomic_load(out + ((size_t)t * K + k) * H + r0, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
            sum = fmaf(cb.w[(size_t)t * K + k], o, sum);
        }
        if (cb.y)
            cb.y[(size_t)t * H + r0] = sum;
        if (cb.res)
            cb.res[(size_t)t * H + r0] += sum;
    }
}

// One down group: DD_WAVES items (32-row chunks) of one expert, one per wave,
// each in its own LDS slice wl [DD_ROWS * DD_RS] dwords.  The weights are
// requested first; the expert's h is read once its gate/up items are counted.
__device__ void down_group(int grp, const uint8_t *__restrict__ blobs,
                           const int4 *__restrict__ erec, const int32_t *__restrict__ slots,
                           const HQ &hq, float *__restrict__ out, int T, const Combine &cb,
                           uint32_t *wl, const int32_t *gdone, int32_t *status, int wait_limit,
                           int *ok_flag)
{
    const int nslot = T * K;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int item = grp * DD_WAVES + wave;
    const int r = lane >> 4, l = lane & 15;
    const int c0 = r >> 1;
    const int a = item / DD_ITEMS_PER_E;
    const int4 rec = erec[1 + a];
    const int ch = item % DD_ITEMS_PER_E;
    int slot = rec.w;
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(blobs + (size_t)rec.x * BLOB + 2 * MAT +
                                                           (size_t)ch * DD_ROWS * ROW_D);
        uint4 *dst = reinterpret_cast<uint4 *>(wl);
        const bool has5 = lane + 320 < DD_CHUNKS;
        const uint4 v0 = src[lane], v1 = src[lane + 64], v2 = src[lane + 128];
        const uint4 v3 = src[lane + 192], v4 = src[lane + 256];
        const uint4 v5 = has5 ? src[lane + 320] : make_uint4(0, 0, 0, 0);
        dst[lane] = v0;
        dst[lane + 64] = v1;
        dst[lane + 128] = v2;
        dst[lane + 192] = v3;
        dst[lane + 256] = v4;
        if (has5)
            dst[lane + 320] = v5;
    }
    // wait (bounded) until the expert's DG_SEGS gate/up items have stored h;
    // h itself is read with agent-scope loads, so the poll needs no cache
    // invalidation, only to stay ahead of those loads in program order.  One
    // lane of the workgroup polls, sparsely.  If the wait gives up, the
    // group's outputs are NaN and the status word records it.
    if (threadIdx.x == 0) {
        int n = 0;
        while (__hip_atomic_load(gdone + SYNC_STRIDE * a, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT) < DG_SEGS &&
               ++n < wait_limit)
            __builtin_amdgcn_s_sleep(32);
        const int ok = n < wait_limit;
        *ok_flag = ok;
        if (!ok)
            __hip_atomic_fetch_or(status, ST_WAIT_GAVE_UP, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const bool gave_up = *ok_flag == 0;
    HOps ho = load_hops(hq, slot >= 0 && slot < nslot ? slot : 0, c0, l);
    // the wave reads back what its own lanes wrote: LDS keeps a wave's order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t *row = wl + ((r & 1) * 16 + l) * DD_RS + 4 * c0;
    // Slots two at a time (the weights of a block decoded once for both).
    for (int ti = 0; ti < rec.z; ti += 2) {
        const bool two = ti + 1 < rec.z;   // uniform per wave
        if (ti > 0) {
            slot = slots[rec.y + ti];
            ho = load_hops(hq, slot >= 0 && slot < nslot ? slot : 0, c0, l);
        }
        int slot2 = -1;
        float acc, acc2 = 0.f;
        if (two) {
            slot2 = slots[rec.y + ti + 1];
            const HOps ho2 = load_hops(hq, slot2 >= 0 && slot2 < nslot ? slot2 : 0, c0, l);
            const float2 r2 = down_row2(row, c0, ho, ho2);
            acc = r2.x;
            acc2 = r2.y;
            acc2 += __shfl_xor(acc2, 32, 64);
        } else {
            acc = down_row(row, c0, ho);
        }
        acc += __shfl_xor(acc, 32, 64);
        if (gave_up) {
            acc = __builtin_nanf("");
            acc2 = __builtin_nanf("");
        }
        finish_slot(slot, acc, ch, out, T, cb);
        if (two)
            finish_slot(slot2, acc2, ch, out, T, cb);
    }
}

constexpr int EX_THREADS = 64 * DG_WAVES;
static_assert(DD_WAVES == DG_WAVES, "gate/up and down workgroups have one shape");
static_assert(DD_ITEMS_PER_E % DD_WAVES == 0, "a down group stays within one expert");
constexpr int EX_DN_PER_E = DD_ITEMS_PER_E / DD_WAVES;   // 20 down groups per expert
constexpr size_t EX_LDS_GU = (size_t)DG_ROWS * DG_RS * 4 + (size_t)2 * DG_WAVES * DG_ROWS * 4;
constexpr size_t EX_LDS_DN = (size_t)DD_WAVES * DD_ROWS * DD_RS * 4;
constexpr size_t EX_LDS_MAX = EX_LDS_GU > EX_LDS_DN ? EX_LDS_GU : EX_LDS_DN;
constexpr size_t EX_LDS = EX_LDS_MAX + 16;   // + the down group's wait flag

// Lookahead: workgroups past the down groups read the blobs of the experts
// predicted for the next layer, one request per 128-byte line, so that the
// next layer's experts kernel finds them in the memory-side cache.  Slot s of
// the prediction gets XT_PER_SLOT workgroups; a slot whose expert an earlier
// slot already names is skipped.  Nothing waits for them and they write
// nothing; they only pull lines in.
constexpr int XT_PER_SLOT = 16;
constexpr int XT_LINES = BLOB / 128;                                   // 10,800
constexpr int XT_LINES_PER_WG = (XT_LINES + XT_PER_SLOT - 1) / XT_PER_SLOT;   // 675
static_assert(BLOB % 128 == 0, "whole lines");

// Each lane's 4 bytes of a line go straight into the workgroup's LDS (lds:
// 1 KB it does not otherwise use, one 256-byte row per wave), so no register
// is written by a load still in flight.
__device__ void touch_next(int b, int nslot, const int32_t *__restrict__ pred,
                           const uint8_t *__restrict__ blobs_next, uint8_t *lds)
{
    const int s = b / XT_PER_SLOT, part = b % XT_PER_SLOT;
    if (s >= nslot)
        return;
    const int e = pred[s];
    if (e < 0 || e >= E)
        return;
    for (int i = 0; i < s; ++i)   // uniform: every lane reads the same ids
        if (pred[i] == e)
            return;
    const uint8_t *base = blobs_next + (size_t)e * BLOB + (size_t)part * XT_LINES_PER_WG * 128;
    const int n = min(XT_LINES_PER_WG, XT_LINES - part * XT_LINES_PER_WG);
    uint8_t *row = lds + 256 * __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int i = threadIdx.x; i < n; i += EX_THREADS)
        __builtin_amdgcn_global_load_lds(base + (size_t)i * 128, row, 4, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The experts of a decode call in one launch.  Workgroup b < 40 amax runs
// gate/up item b; workgroup 40 amax + g runs down group g (items beyond the
// call's na active experts exit at once).  A down group waits only for its
// expert's gate/up items.  Workgroups go to the XCDs round-robin and each XCD
// dispatches its workgroups in index order, so every gate/up workgroup of an
// XCD holds a slot before any down workgroup of that XCD can take one: gate/up
// workgroups never wait behind the down ones, and the waits end.  The wait is
// bounded all the same; a wait that gives up leaves NaN outputs and sets
// ST_WAIT_GAVE_UP in the caller's status word.
__global__ __launch_bounds__(EX_THREADS) void dec_experts(const uint8_t *__restrict__ blobs,
                                                          const int4 *__restrict__ erec,
                                                          const int32_t *__restrict__ slots, XQ xq,
                                                          HQ hq, float *__restrict__ out, int T,
                                                          Combine cb, int32_t *__restrict__ gdone,
                                                          int32_t *__restrict__ status,
                                                          int wait_limit,
                                                          const int32_t *__restrict__ pred,
                                                          const uint8_t *__restrict__ blobs_next)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[EX_LDS];
    const int na = active_count(erec, T);
    const int amax = T * K < E ? T * K : E;
    const int b = blockIdx.x;
    if (b < amax * DG_SEGS) {
        if (b >= na * DG_SEGS)
            return;
        uint32_t *wl = reinterpret_cast<uint32_t *>(lds);
        float(*part)[DG_ROWS] =
            reinterpret_cast<float(*)[DG_ROWS]>(lds + (size_t)DG_ROWS * DG_RS * 4);
        gateup_item<true>(erec[1 + b / DG_SEGS], b % DG_SEGS, b / DG_SEGS, blobs, slots, xq, hq, T,
                          wl, part, gdone);
    } else if (b < amax * (DG_SEGS + EX_DN_PER_E)) {
        const int g = b - amax * DG_SEGS;
        if (g >= na * EX_DN_PER_E)
            return;
        uint32_t *wl = reinterpret_cast<uint32_t *>(lds) +
                       (size_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * DD_ROWS * DD_RS;
        down_group(g, blobs, erec, slots, hq, out, T, cb, wl, gdone, status, wait_limit,
                   reinterpret_cast<int *>(lds + EX_LDS_MAX));
    } else {
        touch_next(b - amax * (DG_SEGS + EX_DN_PER_E), T * K, pred, blobs_next, lds);
    }
}

// ------------------------------- T <= ROUTED_T_MAX: two launches, no wait
// For up to ROUTED_T_MAX tokens the layer runs the experts as two launches in
// stream order instead (the kernel boundary publishes h, so nothing waits
// inside a kernel): dec_route_gateup (below) routes each token and runs its
// ten heads' gate/up items (plain stores of h, no counters), then dec_down,
// with one workgroup per 16 output rows of a token, 5 waves with two of its
// slots each, lane (r, l) taking row l of slot 2 w + r % 2's expert and block
// columns 2 j + r / 2 from five 20-byte windows loaded straight into
// registers.  The two halves of each row are added, the ten slot rows meet in
// LDS and are summed in routing order with fma from 0, the order of the fused
// combine, so a token's results are bitwise those of the fused kernel.  At
// T = 4 the fused kernel is faster for tokens that share few experts (its
// down groups read an expert's rows once for all the tokens that share it;
// here each token reads its own).
constexpr int DS_ROWS = 16;                         // output rows per workgroup
constexpr int DS_WAVES = K / 2;                     // 5: two slots per wave
constexpr int DS_THREADS = 64 * DS_WAVES;
constexpr int DS_CHUNKS_PER_T = H / DS_ROWS;        // 160
constexpr size_t DS_LDS_GU = (size_t)DG_ROWS * DG_RS * 4 + (size_t)2 * DG_WAVES * DG_ROWS * 4;
static_assert(DG_WAVES * 256 <= DS_LDS_GU && DG_WAVES * 256 <= EX_LDS,
              "the line reads' LDS rows fit in every kernel that makes them");

// A lane's down weights: five 20-byte windows of its row (window j holds block
// column 2 j + c0, starting 2 bytes in when c0 = 1).
struct DnW {
    uint4 lo[5];
    uint32_t hi[5];
};

__device__ inline void dn_request(const uint8_t *__restrict__ blobs, int e, int row, int c0, DnW &w)
{
    const uint8_t *p = blobs + (size_t)e * BLOB + 2 * MAT + (size_t)row * ROW_D + 16 * c0;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        w.lo[j] = *reinterpret_cast<const uint4 *>(p + 36 * j);
        w.hi[j] = *reinterpret_cast<const uint32_t *>(p + 36 * j + 16);
    }
}

// down_block on a window held in registers (the same arithmetic).
template <int N>
__device__ inline float down_block_r(const uint4 lo, uint32_t v4, uint32_t sel, uint32_t sh, uint2 D,
                                     float shr, int nqr)
{
    const uint32_t v0 = lo.x, v1 = lo.y, v2 = lo.z, v3 = lo.w;
    const Codes c = split_codes(__builtin_amdgcn_perm(v1, v0, sel), __builtin_amdgcn_perm(v2, v1, sel),
                                __builtin_amdgcn_perm(v3, v2, sel), __builtin_amdgcn_perm(v4, v3, sel));
    const float d = half_bits_to_float(v0 >> sh);
    const Quad qd = quarters_codes_dot(c, D.x, D.y);
    float bacc = 0.f;
    const float f0 = (float)(qd.q[0] + row_bcast_i<N>(nqr));
    STRATA_FMA_BCAST(bacc, shr, f0, N);
    const float f1 = (float)(qd.q[1] + row_bcast_i<N + 1>(nqr));
    STRATA_FMA_BCAST(bacc, shr, f1, N + 1);
    const float f2 = (float)(qd.q[2] + row_bcast_i<N + 2>(nqr));
    STRATA_FMA_BCAST(bacc, shr, f2, N + 2);
    const float f3 = (float)(qd.q[3] + row_bcast_i<N + 3>(nqr));
    STRATA_FMA_BCAST(bacc, shr, f3, N + 3);
    return d * bacc;
}

// down_row on register windows (the same blocks in the same order).
__device__ inline float down_row_r(const DnW &w, int c0, const HOps &ho)
{
    const uint32_t sel = c0 ? 0x07060504u : 0x05040302u;
    const uint32_t sh = c0 ? 16u : 0u;
    float acc = down_block_r<0>(w.lo[0], w.hi[0], sel, sh, ho.d[0], ho.sh0, ho.nq0);
    acc += down_block_r<4>(w.lo[1], w.hi[1], sel, sh, ho.d[1], ho.sh0, ho.nq0);
    acc += down_block_r<8>(w.lo[2], w.hi[2], sel, sh, ho.d[2], ho.sh0, ho.nq0);
    acc += down_block_r<12>(w.lo[3], w.hi[3], sel, sh, ho.d[3], ho.sh0, ho.nq0);
    acc += down_block_r<0>(w.lo[4], w.hi[4], sel, sh, ho.d[4], ho.sh1, ho.nq1);
    return acc;
}

// Workgroup b: token b / 160, output rows 16 (b % 160) .. + 15.  sexp[t K + k]
// is the expert of slot (t, k) (a slot whose expert is outside 0..E-1 gives
// zero rows).  y_t = sum_k w[t][k] o_k, stored and/or added to res.
__global__ __launch_bounds__(DS_THREADS) void dec_down(const uint8_t *__restrict__ blobs,
                                                       const int32_t *__restrict__ sexp, HQ hq,
                                                       const float *__restrict__ w, float *y,
                                                       float *res)
{
    __shared__ float orow[K][DS_ROWS];
    const int t = blockIdx.x / DS_CHUNKS_PER_T, ch = blockIdx.x % DS_CHUNKS_PER_T;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane >> 4, l = lane & 15;
    const int k = 2 * wave + (r & 1), c0 = r >> 1;
    const int slot = t * K + k;
    const int row = ch * DS_ROWS + l;
    const int e = sexp[slot];
    const bool ok = e >= 0 && e < E;
    DnW dw;
    dn_request(blobs, ok ? e : 0, row, c0, dw);
    const HOps ho = load_hops<false>(hq, slot, c0, l);
    float acc = down_row_r(dw, c0, ho);
    acc += __shfl_xor(acc, 32, 64);   // the row's two halves
    if (!ok)
        acc = 0.f;
    if (lane < 32)
        orow[k][l] = acc;
    __syncthreads();
    if (threadIdx.x < DS_ROWS) {
        float sum = 0.f;
#pragma unroll
        for (int kk = 0; kk < K; ++kk)
            sum = fmaf(w[(size_t)t * K + kk], orow[kk][threadIdx.x], sum);
        const size_t at = (size_t)t * H + ch * DS_ROWS + threadIdx.x;
        if (y)
            y[at] = sum;
        if (res)
            res[at] += sum;
    }
}

// ------------------------------- T <= ROUTED_T_MAX: the routing in every item
// A layer call for up to ROUTED_T_MAX tokens has no top-k launch: each token
// gets 400 gate/up workgroups,
// and wave 0 of every one of them routes that token itself from the router's
// logits -- the top-k kernel's code on the same inputs, so every workgroup of
// a token gets the same ten ids and weights, bitwise.  A token's ten experts
// are distinct, so there is nothing to group: workgroup b of token t's 400
// takes head m = b / 40 (the m-th expert in routing order) and segment b % 40,
// slot t K + m.  An expert two tokens share is read once per token (each
// token's items are its own); against the grouped launches that read it once,
// this was faster at T = 2 and 3 (20.7 vs 22.9 us, 22.1 vs 25.0 us per layer
// step) and slower from T = 4 (28.5 vs 27.4 us).  The first workgroup of each
// token writes its ids and weights, which the down launch (dec_down, above)
// and the caller read.
//
// With a hint -- ten expert ids expected for this token, e.g. the previous
// layer's lookahead prediction -- 400 more workgroups come first: workgroup
// (j, seg) requests segment seg of hinted expert j's rows before the routing
// has finished (the ~2 us of routing overlap the loads), and afterwards
// computes them for the head whose expert that is, or exits if no head is.
// The 400 plain workgroups then cover, in routing order, only the heads whose
// expert no hint names.  Every head's h is computed exactly once, with the
// same arithmetic either way, so the results never depend on the hint.
//
// With the lookahead (lraw2: the next layer's raw logits of the same input),
// wave 1 of each token's first workgroup routes them to the token's predicted
// ids for the next layer (pred), and K * XT_PER_SLOT trailing workgroups per
// token, each routing them again, read the predicted experts' blobs in
// blobs_next line by line (an expert two tokens predict is read for each).
constexpr int DR_WG = K * DG_SEGS;   // 400 workgroups per set

__global__ __launch_bounds__(DG_THREADS) void dec_route_gateup(
    const uint8_t *__restrict__ blobs, const float *__restrict__ lraw,
    const float *__restrict__ bias, XQ xq, HQ hq, int32_t *__restrict__ ids,
    float *__restrict__ wout, const int32_t *__restrict__ hint, const float *__restrict__ lraw2,
    const float *__restrict__ bias2, int32_t *__restrict__ pred,
    const uint8_t *__restrict__ blobs_next, int T)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[DS_LDS_GU];
    __shared__ int head[K];
    const int nh = hint ? DR_WG : 0;
    const int b = blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (b >= nh + T * DR_WG) {   // lookahead reads: K * XT_PER_SLOT workgroups per token
        const int i = b - nh - T * DR_WG, tt = i / (K * XT_PER_SLOT);
        if (wave == 0) {
            int my_id;
            float my_p, sel;
            route_token(lraw2 + (size_t)tt * E, xq.inv_rms[tt], bias2, my_id, my_p, sel);
            if (lane < K)
                head[lane] = my_id;
        }
        __syncthreads();
        touch_next(i % (K * XT_PER_SLOT), K, head, blobs_next, lds);
        return;
    }
    const bool hinted = b < nh;
    // token t of the plain sets (hints and the lookahead come with one token)
    const int t = hinted ? 0 : (b - nh) / DR_WG;
    const int bb = hinted ? b : (b - nh) % DR_WG;
    const int j = bb / DG_SEGS, seg = bb % DG_SEGS;
    const bool writer = bb == 0 && (hinted || !hint);   // writes token t's ids and weights
    // the hinted expert: a valid id and the first of its value in the hint
    int eh = -1;
    if (hinted) {
        const int v = hint[j];
        bool first = v >= 0 && v < E;
        for (int i = 0; i < j; ++i)
            first = first && hint[i] != v;
        eh = first ? v : -1;
    }
    // the logits first, so that waiting for them does not wait for the rows
    TokLogits tl, tl2;
    if (wave == 0)
        tl = load_logits(lraw + (size_t)t * E, bias);
    const bool predict = writer && pred != nullptr;
    if (wave == 1 && predict)
        tl2 = load_logits(lraw2 + (size_t)t * E, bias2);
    const float sc = xq.inv_rms[t];
    const int s = 2 * wave + ((lane >> 4) >> 1);
    XOps xo;
    GuChunks ch;
    if (eh >= 0) {
        xo = load_xops(xq, 0, s, lane & 15);
        ch = gu_request(blobs, eh, seg);
    }
    if (wave == 0) {
        // the writer needs all ten heads, and so does every workgroup of a
        // hinted call; a plain workgroup needs heads 0 .. j only, so it can
        // request its rows sooner
        int my_id;
        float my_p, sel;
        route_logits(tl, sc, bias != nullptr, my_id, my_p, sel, (writer || hint) ? K - 1 : j);
        if (writer && lane < K) {
            ids[t * K + lane] = my_id;
            wout[t * K + lane] = my_p / renorm_den(sel);
        }
        if (lane < K)
            head[lane] = my_id;
    } else if (wave == 1 && predict) {
        int my_id;
        float my_p, sel;
        route_logits(tl2, sc, bias2 != nullptr, my_id, my_p, sel);
        if (lane < K)
            pred[t * K + lane] = my_id;
    }
    uint32_t *wl = reinterpret_cast<uint32_t *>(lds);
    float(*part)[DG_ROWS] = reinterpret_cast<float(*)[DG_ROWS]>(lds + (size_t)DG_ROWS * DG_RS * 4);
    if (eh >= 0)
        gu_stage(ch, wl);
    __syncthreads();   // head, and the hinted rows
    if (hinted) {
        int k = -1;
        for (int i = 0; i < K; ++i)
            k = head[i] == eh ? i : k;
        if (eh < 0 || k < 0)
            return;
        gateup_compute<false>(make_int4(eh, 0, 1, k), seg, 0, nullptr, xq, hq, 1, wl, part,
                              nullptr, xo);
        return;
    }
    // the j-th head, in routing order, whose expert no hint names
    int k = -1, n = 0;
    for (int i = 0; i < K; ++i) {
        bool named = false;
        if (hint)
            for (int h = 0; h < K; ++h)
                named = named || hint[h] == head[i];
        if (!named) {
            k = n == j ? i : k;
            ++n;
        }
    }
    if (k < 0)
        return;
    const int e = head[k];
    if (e < 0 || e >= E)   // not reached: the ten heads are expert ids
        return;
    gateup_item<false>(make_int4(e, 0, 1, t * K + k), seg, 0, blobs, nullptr, xq, hq, T, wl, part,
                       nullptr);
}

hipError_t launch_decode_routed(const uint8_t *blobs, const float *lraw, int T, const float *bias,
                                XQ xq, HQ hq, int32_t *ids, float *w, float *y, float *res,
                                const int32_t *hint, const float *lraw2, const float *bias2,
                                int32_t *pred, const uint8_t *blobs_next, hipEvent_t ev0,
                                hipEvent_t ev1, hipStream_t st)
{
    if (T > 1)   // hints come with one token only
        hint = nullptr;
    if (!lraw2)
        pred = nullptr;
    if (!pred)
        blobs_next = nullptr;
    const int nwg = (hint ? DR_WG : 0) + T * DR_WG + (blobs_next ? T * K * XT_PER_SLOT : 0);
    void *args[] = {&blobs, &lraw, &bias, &xq, &hq, &ids, &w, &hint, &lraw2, &bias2, &pred,
                    &blobs_next, &T};
    hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(&dec_route_gateup),
                                      dim3(nwg), dim3(DG_THREADS), args, 0, st, ev0, nullptr, 0);
    if (e != hipSuccess)
        return e;
    const int32_t *sexp = ids;
    const float *wc = w;
    void *dargs[] = {&blobs, &sexp, &hq, &wc, &y, &res};
    return hipExtLaunchKernel(reinterpret_cast<const void *>(&dec_down),
                              dim3(T * DS_CHUNKS_PER_T), dim3(DS_THREADS), dargs, 0, st, nullptr,
                              ev1, 0);
}

hipError_t launch_decode_experts(const uint8_t *blobs, const int4 *erec, const int32_t *slots,
                                 XQ xq, HQ hq, float *out, int T, int32_t *sync, int32_t *cdone,
                                 const float *w, float *y, float *res, const int32_t *pred,
                                 const uint8_t *blobs_next, int32_t *status, int wait_limit,
                                 hipEvent_t ev0, hipEvent_t ev1, hipStream_t st)
{
    Combine cb{cdone, w, y, res};
    const int amax = T * K < E ? T * K : E;
    int32_t *gdone = sync + 1;
    if (!blobs_next)
        pred = nullptr;
    const dim3 grid(amax * (DG_SEGS + EX_DN_PER_E) + (pred ? T * K * XT_PER_SLOT : 0));
    const dim3 block(EX_THREADS);
    if (ev0) {   // timed launch: the events carry the dispatch's own start and end
        void *args[] = {&blobs, &erec,  &slots,  &xq,         &hq,   &out,       &T,
                        &cb,    &gdone, &status, &wait_limit, &pred, &blobs_next};
        return hipExtLaunchKernel(reinterpret_cast<const void *>(&dec_experts), grid, block, args,
                                  0, st, ev0, ev1, 0);
    }
    hipLaunchKernelGGL(dec_experts, grid, block, 0, st, blobs, erec, slots, xq, hq, out, T, cb,
                       gdone, status, wait_limit, pred, blobs_next);
    return hipGetLastError();
}

} // namespace strata
