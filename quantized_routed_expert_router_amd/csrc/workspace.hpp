// workspace.hpp -- the layout of the caller's workspace: byte offsets of the
// regions the kernels of one call use (host code only).
#pragma once
#include "common.hpp"

namespace strata {

// Workspace regions (byte offsets, 256-aligned) for a call with T tokens;
// Td = T on the decode path (T <= DECODE_T_MAX) else 0, Tp the converse.
struct Ws {
    size_t status;     // i32 [1] (256 bytes reserved) status word, always at offset 0
    size_t xsplit;     // bf16 [Tp][3][H]    router input (prefill): x = x1 + x2 + x3 exactly
    size_t xperm;      // f16 [Tp][H]        MFMA-ordered activations (prefill), times 2^xexp
    size_t xexp;       // i32 [Tp]           per-token power-of-two exponents of xperm (low 16 bits) and h (high)
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
    size_t mlist;      // i32 [max items + 8][4]  prefill work items {e, gp0, rows, 0}
    size_t nitems;     // i32 [4]
    size_t hq_dig;     // u32 [Td*K][10][32] 16-bit h per 16 values (64-value blocks)
    size_t hq_scale;   // f32 [Td*K][40]
    size_t hq_sum;     // i32 [Td*K][40]
    size_t hperm;      // f16 [Tp*K][FF]     (grouped order)
    size_t hexp;       // i32 [Tp*K]         the exponent h of each grouped row carries
    size_t out;        // f32 [T*K][H]
    size_t cdone;      // i32 [Td][H/32]      decode layer: finished slots per (token, 32 rows)
    size_t esync;      // i32 [1+32E]        decode experts: finished gate/up items per active expert (128-B apart)
    size_t gcount;     // i32 [ceil(Tp*K/1024)][E] prefill grouping: per-block expert counts / starts
    size_t lraw2;      // f32 [Td][E]        lookahead: the next layer's raw logits
    size_t pred;       // i32 [Td*K]         lookahead: the next layer's predicted ids
    size_t x8;         // i8 [Tp][H]         int8 variant: activations per 64-block
    size_t xs8;        // f32 [Tp][40]       their scales
    size_t xn8;        // i32 [Tp][40]       -(sum q) per block
    size_t h8;         // i8 [Tp*K][FF]      int8 variant: h per 64-block (grouped order)
    size_t hs8;        // f32 [Tp*K][10]
    size_t hn8;        // i32 [Tp*K][10]
    size_t total;
    int max_items;
};

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Bytes at the start of every workspace that hold the status word.
constexpr size_t WS_STATUS_BYTES = 256;

constexpr Ws ws_layout(int T)
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
    L.status = take(4);
    L.xsplit = take(Tp * 3 * H * 2);
    L.xperm = take(Tp * H * 2);
    L.xexp = take(Tp * 4);
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
    L.mlist = take((size_t)4 * (L.max_items + PF_LIST_PAD) * 4);
    L.nitems = take(16);
    L.hq_dig = take(Td * K * (FF / QK) * 32 * 4);
    L.hq_scale = take(Td * K * ns * 4);
    L.hq_sum = take(Td * K * ns * 4);
    L.hperm = take(Tp * K * FF * 2);
    L.hexp = take(Tp * K * 4);
    L.out = take((size_t)T * K * H * 4);
    L.cdone = take(Td * (H / 32) * 4);
    L.esync = take(Td ? (size_t)(1 + 32 * E) * 4 : 0);
    L.gcount = take((Tp * K + GB_SLOTS - 1) / GB_SLOTS * E * 4);
    L.lraw2 = take(Td * E * 4);
    L.pred = take(Td * K * 4);
    L.x8 = take(Tp * H);
    L.xs8 = take(Tp * nb * 4);
    L.xn8 = take(Tp * nb * 4);
    L.h8 = take(Tp * K * FF);
    L.hs8 = take(Tp * K * (FF / QK) * 4);
    L.hn8 = take(Tp * K * (FF / QK) * 4);
    L.total = o;
    return L;
}

// The largest workspace any T in 1..tmax needs.
constexpr size_t ws_max_bytes(int tmax)
{
    size_t m = 0;
    for (int T = 1; T <= tmax; ++T)
        m = ws_layout(T).total > m ? ws_layout(T).total : m;
    return m;
}

} // namespace strata
