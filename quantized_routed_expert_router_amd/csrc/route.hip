// route.hip -- activation prep and the router: logits = xhat . R^T (+ bias),
// softmax over all 512 experts, stable descending top-10, gather and
// renormalisation with a lower clamp ("MoE 遇上消费级显卡..." (zwxr.cn), the
// passage following one token through a layer: a BF16 GEMV to 512 logits, then
// a fused 512-expert softmax / stable argsort / gather / clamped renorm).
//
// Kernels:
//  prep_kernel    one workgroup per token: optional RMSNorm (eps 1e-6, unit
//                 gain), xhat as three bf16 terms for the router and fp16
//                 xhat in the K order the prefill MFMA kernels consume.  (Decode-sized T
//                 uses route_decode.hip.)
//  gemm_kernel    bf16 MFMA over the exact three-term bf16 split of xhat
//                 (fp32-accurate logits); identical router rows give
//                 identical logits.
//  topk_kernel    one wave per token (route_token, shared with the decode
//                 top-k): softmax in fp32, each lane's 8 candidates sorted,
//                 ten rounds of a wave-wide max over the lanes' heads (the
//                 order p desc, id asc), clamped renorm.
#include "common.hpp"
#include "route_token.hpp"

namespace strata {

// Position pos (0..H-1) of a row in the gate/up activation order holds input
// column 64 (4 g + q) + 16 (j / 2) + 4 (j % 2) + s / 2 + 8 (s % 2) with
// pos = 256 g + 64 q + 8 j + s: 16-byte chunk 8 q + j of 256-column group g
// is the fragment of MFMA step j for the lanes that own block 4 g + q (see
// experts_prefill).
__device__ inline int pg_col_of_pos(int pos)
{
    const int g = pos >> 8, q = (pos >> 6) & 3, j = (pos >> 3) & 7, s = pos & 7;
    return 64 * (4 * g + q) + 16 * (j >> 1) + 4 * (j & 1) + (s >> 1) + 8 * (s & 1);
}

constexpr int PREP_THREADS = 256;

// bf16 bits of v, round to nearest even (finite inputs)
__device__ inline uint16_t bf16_rn_bits(float v)
{
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// The fp16 activations of the prefill GEMMs carry a per-token power-of-two
// scale 2^k, and the h the gate/up GEMM writes a second one, 2^hs.  A row
// whose max |xhat_t| lies in [1, 8) (every RMSNorm'd row without a large
// outlier, and unnormalised rows of unit-scale values) is stored unscaled:
// k = hs = 0.  Any other row gets k with max |xhat_t| 2^k in [2^12, 2^13)
// (|k| <= 100) and hs = 2 min(k - 10, 0) + 2 max(k - 12, 0), h growing as
// x^2 (an all-zero row: k = hs = 0).  That keeps every input magnitude inside
// fp16's normal range; xexp[t] = k in the low 16 bits, hs in the high 16
// (both signed), lets the GEMM epilogues undo both exactly.
constexpr int XEXP_TARGET = 13;
constexpr int XEXP_MAX = 100;

// Thread tid handles the column pairs (2 tid + 512 i, + 1), i = 0..4, so that
// every load is 8 bytes and every store 4 (two bf16 or two fp16 values).
constexpr int PREP_PAIRS = H / (2 * PREP_THREADS);   // 5
static_assert(PREP_PAIRS * 2 * PREP_THREADS == H, "whole pairs");

__device__ inline uint32_t pack16(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

__global__ __launch_bounds__(PREP_THREADS) void prep_kernel(
    const float *__restrict__ x, int rmsnorm, uint16_t *__restrict__ xsplit,
    __half *__restrict__ xperm, int32_t *__restrict__ xexp)
{
    __shared__ __attribute__((aligned(8))) float xs[H];
    __shared__ float wsum[PREP_THREADS / 64];
    __shared__ float wmax[PREP_THREADS / 64];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const float *xt = x + (size_t)t * H;
    float2 v[PREP_PAIRS];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PREP_PAIRS; ++i) {
        v[i] = *reinterpret_cast<const float2 *>(xt + 2 * tid + 2 * PREP_THREADS * i);
        ss = fmaf(v[i].x, v[i].x, ss);
        ss = fmaf(v[i].y, v[i].y, ss);
    }
    float inv = 1.f;
    if (rmsnorm) {
        ss = wave_sum63(ss);
        if ((tid & 63) == 0)
            wsum[tid >> 6] = ss;
        __syncthreads();
        const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
        inv = 1.f / sqrtf(tot / (float)H + 1e-6f);
    }
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < PREP_PAIRS; ++i) {
        const int c = 2 * tid + 2 * PREP_THREADS * i;
        const float h0 = v[i].x * inv, h1 = v[i].y * inv;
        mx = fmaxf(mx, fmaxf(fabsf(h0), fabsf(h1)));
        *reinterpret_cast<float2 *>(xs + c) = make_float2(h0, h1);
        // the router's exact three-term bf16 split of xhat
        if (xsplit) {
            const uint16_t a1 = bf16_rn_bits(h0), b1 = bf16_rn_bits(h1);
            const float ra = h0 - bf16_bits_to_float(a1), rb = h1 - bf16_bits_to_float(b1);   // exact
            const uint16_t a2 = bf16_rn_bits(ra), b2 = bf16_rn_bits(rb);
            const float sa = ra - bf16_bits_to_float(a2), sb = rb - bf16_bits_to_float(b2);   // exact
            uint32_t *xo = reinterpret_cast<uint32_t *>(xsplit + (size_t)t * 3 * H + c);
            xo[0] = pack16(a1, b1);
            xo[H / 2] = pack16(a2, b2);
            xo[H] = pack16(bf16_rn_bits(sa), bf16_rn_bits(sb));
        }
    }
    mx = wave_max63(mx);
    if ((tid & 63) == 0)
        wmax[tid >> 6] = mx;
    __syncthreads();
    if (xperm) {
        mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        int ex = 0;
        (void)frexpf(mx, &ex);   // mx in [2^(ex-1), 2^ex)
        int k = mx > 0.f ? min(max(XEXP_TARGET - ex, -XEXP_MAX), XEXP_MAX) : 0;
        int hs = 2 * min(k - 10, 0) + 2 * max(k - 12, 0);
        if (mx == 0.f || (k >= 10 && k <= 12))
            k = hs = 0;
        if (tid == 0)
            xexp[t] = (int32_t)(((uint32_t)hs << 16) | ((uint32_t)k & 0xffffu));
        // positions pos and pos + 1 (pos even) hold columns 8 apart
#pragma unroll
        for (int i = 0; i < PREP_PAIRS; ++i) {
            const int pos = 2 * tid + 2 * PREP_THREADS * i;
            const __half lo = __float2half_rn(ldexpf(xs[pg_col_of_pos(pos)], k));
            const __half hi = __float2half_rn(ldexpf(xs[pg_col_of_pos(pos + 1)], k));
            *reinterpret_cast<uint32_t *>(xperm + (size_t)t * H + pos) =
                pack16(__half_as_ushort(lo), __half_as_ushort(hi));
        }
    }
}

// ---------------------------------------------------------------- router GEMM
// logits = xhat . R^T on the bf16 matrix cores.  R is bf16 already; the prep
// kernel splits each fp32 xhat value exactly into three bf16 terms
// x1 + x2 + x3 (x1 = bf16(x), x2 = bf16(x - x1), x3 = bf16(x - x1 - x2):
// together all 24 bits of the fp32 significand), and bf16 x bf16 products are
// exact in the fp32 accumulation, so the logits keep fp32 accuracy.  Every
// logit is the same sequence of MFMAs (K ascending in steps of 32, the three
// terms in turn), so identical router rows give identical logits.
//
// Workgroup tile: 32 tokens x 128 experts; wave w owns experts 32 w .. + 31,
// all 32 tokens (2 x 2 subtiles of 16 x 16).  K goes in stages of 64: both
// operands of a stage (the three x terms of 32 rows and 128 router rows, 64
// bf16 each) reach LDS by direct global-to-LDS loads into one of four
// buffers, three stages ahead, one barrier per stage.  Rows are 128 bytes in
// LDS with 16-byte chunk c of row r at position c ^ (r % 8), so the fragment
// reads of 16 consecutive rows fall in distinct banks.  The LDS reads are
// inline assembly because the compiler would otherwise wait for every
// outstanding LDS-bound load before each of them.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
constexpr int GR_M = 32, GR_N = 128, GR_SK = 64, GR_STAGES = H / GR_SK;
constexpr int GR_NBUF = 4;
constexpr int GR_ABYTES = 3 * GR_M * GR_SK * 2;                 // 12,288
constexpr int GR_BBYTES = GR_N * GR_SK * 2;                     // 16,384
constexpr int GR_BUF = GR_ABYTES + GR_BBYTES;                   // 28,672
constexpr int GR_REQ = GR_BUF / 16 / 256;                       // 7 requests per lane per stage
static_assert(GR_REQ * 16 * 256 == GR_BUF && GR_ABYTES == 3 * 256 * 16, "request split");
static_assert(E % GR_N == 0 && H % GR_SK == 0 && GR_STAGES >= GR_NBUF - 1, "router GEMM tiling");

typedef __attribute__((address_space(3))) uint8_t gr_lds_u8;
__device__ inline uint32_t gr_lds_addr(uint8_t *p)
{
    return (uint32_t)(uintptr_t)(gr_lds_u8 *)p;
}

template <int N> __device__ inline void gr_vm_wait()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// The operand fragments of one stage for one wave: a[s][term][mi], b[s][ni]
// (K-step s of the stage, token subtile mi, expert subtile ni).
struct GrFrag {
    uint4 a[2][3][2];
    uint4 b[2][2];
};

// Reads of one stage's fragments; va[s] / vb[s] are this lane's A / B read
// addresses for K-step s (the subtile and term offsets are immediates).
__device__ inline void gr_reads(uint32_t va0, uint32_t va1, uint32_t vb0, uint32_t vb1, GrFrag &f)
{
    asm volatile("ds_read_b128 %0, %16 offset:0\n\t"
                 "ds_read_b128 %1, %16 offset:2048\n\t"
                 "ds_read_b128 %2, %16 offset:4096\n\t"
                 "ds_read_b128 %3, %16 offset:6144\n\t"
                 "ds_read_b128 %4, %16 offset:8192\n\t"
                 "ds_read_b128 %5, %16 offset:10240\n\t"
                 "ds_read_b128 %6, %18 offset:0\n\t"
                 "ds_read_b128 %7, %18 offset:2048\n\t"
                 "ds_read_b128 %8, %17 offset:0\n\t"
                 "ds_read_b128 %9, %17 offset:2048\n\t"
                 "ds_read_b128 %10, %17 offset:4096\n\t"
                 "ds_read_b128 %11, %17 offset:6144\n\t"
                 "ds_read_b128 %12, %17 offset:8192\n\t"
                 "ds_read_b128 %13, %17 offset:10240\n\t"
                 "ds_read_b128 %14, %19 offset:0\n\t"
                 "ds_read_b128 %15, %19 offset:2048\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(f.a[0][0][0]), "=&v"(f.a[0][0][1]), "=&v"(f.a[0][1][0]), "=&v"(f.a[0][1][1]),
                   "=&v"(f.a[0][2][0]), "=&v"(f.a[0][2][1]), "=&v"(f.b[0][0]), "=&v"(f.b[0][1]),
                   "=&v"(f.a[1][0][0]), "=&v"(f.a[1][0][1]), "=&v"(f.a[1][1][0]), "=&v"(f.a[1][1][1]),
                   "=&v"(f.a[1][2][0]), "=&v"(f.a[1][2][1]), "=&v"(f.b[1][0]), "=&v"(f.b[1][1])
                 : "v"(va0), "v"(va1), "v"(vb0), "v"(vb1)
                 : "memory");
}

__device__ inline void gr_math(const GrFrag &f, floatx4 acc[2][2])
{
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, f.a[s][j][mi]),
                        __builtin_bit_cast(bf16x8, f.b[s][ni]), acc[mi][ni], 0, 0, 0);
}

__global__ __launch_bounds__(256) void gemm_kernel(
    const uint16_t *__restrict__ xsplit, int T, const uint16_t *__restrict__ R,
    const float *__restrict__ bias, float *__restrict__ logits)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[GR_NBUF * GR_BUF];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int l = lane & 15, q = lane >> 4;
    const int m0 = blockIdx.x * GR_M, n0 = blockIdx.y * GR_N;
    // This lane's source of LDS chunk Q = 256 i + 64 wave + lane of a stage
    // buffer, i = 0..6: chunks 0..767 are the x terms (term, row, position),
    // the rest the router rows (row, position); chunk c = position ^ (row % 8).
    const uint8_t *src[GR_REQ];
#pragma unroll
    for (int i = 0; i < GR_REQ; ++i) {
        const int Q = 256 * i + 64 * wave + lane;
        if (i < 3) {
            const int row = (Q >> 3) & 31, c = (Q & 7) ^ (row & 7);
            const int m = min(m0 + row, T - 1);   // rows past T load a copy, never stored
            src[i] = reinterpret_cast<const uint8_t *>(xsplit + ((size_t)m * 3 + i) * H + 8 * c);
        } else {
            const int row = (Q - 768) >> 3, c = (Q & 7) ^ (row & 7);
            src[i] = reinterpret_cast<const uint8_t *>(R + (size_t)(n0 + row) * H + 8 * c);
        }
    }
    // stage k of K into the buffer of stage slot
    auto request = [&](int k, int slot) {
        uint8_t *buf = lds + (slot % GR_NBUF) * GR_BUF;
#pragma unroll
        for (int i = 0; i < GR_REQ; ++i)
            __builtin_amdgcn_global_load_lds(src[i] + GR_SK * 2 * k,
                                             buf + (256 * i + 64 * wave) * 16, 16, 0, 0);
    };
    // this lane's fragment read addresses in buffer 0, per K-step s of a stage
    const uint32_t off0 = 16 * ((0 + q) ^ (l & 7)), off1 = 16 * ((4 + q) ^ (l & 7));
    const uint32_t ra = gr_lds_addr(lds) + l * 128;
    const uint32_t rb = gr_lds_addr(lds) + GR_ABYTES + (32 * wave + l) * 128;
    floatx4 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = (floatx4){0.f, 0.f, 0.f, 0.f};
    request(0, 0);
    request(1, 1);
    request(2, 2);
#pragma unroll 1
    for (int st = 0; st < GR_STAGES; ++st) {
        gr_vm_wait<2 * GR_REQ>();   // this stage landed; the two younger stages may not have
        __builtin_amdgcn_s_barrier();
        // the buffer of stage st - 1 is free: stage st + 3 goes there (past
        // the end the last stage again, into that same free buffer, never
        // read: every iteration issues the same number of requests)
        request(min(st + GR_NBUF - 1, GR_STAGES - 1), st + GR_NBUF - 1);
        const uint32_t bo = (st % GR_NBUF) * GR_BUF;
        GrFrag f;
        gr_reads(ra + bo + off0, ra + bo + off1, rb + bo + off0, rb + bo + off1, f);
        gr_math(f, acc);
    }
    gr_vm_wait<0>();
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int n = n0 + 32 * wave + 16 * ni + l;
        const float bn = bias ? bias[n] : 0.f;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int mr = m0 + 16 * mi + 4 * q + r;
                if (mr < T)
                    logits[(size_t)mr * E + n] = acc[mi][ni][r] + bn;
            }
    }
}

// ---------------------------------------------------------------- softmax / top-k
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T,
                                                   int32_t *__restrict__ ids,
                                                   float *__restrict__ wout)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T)
        return;
    int my_id;
    float my_p, sel_sum;
    route_token(logits + (size_t)t * E, 1.f, nullptr, my_id, my_p, sel_sum);
    const float den = renorm_den(sel_sum);
    if (lane < K) {
        ids[(size_t)t * K + lane] = my_id;
        wout[(size_t)t * K + lane] = my_p / den;
    }
}

hipError_t launch_prep(const float *x, int T, int rmsnorm, uint16_t *xsplit, __half *xperm,
                       int32_t *xexp, hipStream_t st)
{
    hipLaunchKernelGGL(prep_kernel, dim3(T), dim3(PREP_THREADS), 0, st, x, rmsnorm, xsplit, xperm,
                       xexp);
    return hipGetLastError();
}

hipError_t launch_logits(const uint16_t *xsplit, int T, const uint16_t *R, const float *bias,
                         float *logits, hipStream_t st)
{
    hipLaunchKernelGGL(gemm_kernel, dim3((T + GR_M - 1) / GR_M, E / GR_N), dim3(256), 0, st,
                       xsplit, T, R, bias, logits);
    return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int T, int32_t *ids, float *w, hipStream_t st)
{
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, ids, w);
    return hipGetLastError();
}

} // namespace strata
