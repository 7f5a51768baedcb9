// fill.hip -- device side of the seeded input generator (not the layer's
// arithmetic).  Writes expert blobs byte-identical to inputs/__init__.py's
// gen_blob(): SplitMix64 (Steele, Lea & Flood 2014; Vigna's splitmix64.c
// constants) keyed by (seed, blob id), three 64-bit words per 18-byte block:
// two words of codes, one word whose top 16 bits index the fp16 scale table.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __host__ inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Output number i (0-based) of the SplitMix64 stream started at `state`.
__device__ __host__ inline uint64_t sm64(uint64_t state, uint64_t i)
{
    return mix64(state + (i + 1) * kGamma);
}

// One thread writes 8 consecutive 18-byte blocks = 144 bytes = 9 x 16 B.
__global__ void fill_kernel(uint8_t *__restrict__ dst, uint64_t base, uint64_t first_blob,
                            uint64_t groups_per_blob, uint64_t total_groups,
                            uint64_t blob_bytes, const uint16_t *__restrict__ table)
{
    uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= total_groups)
        return;
    uint64_t blob = g / groups_per_blob;
    uint64_t grp = g - blob * groups_per_blob;
    uint64_t key = sm64(base, first_blob + blob);
    uint32_t out[36];
#pragma unroll
    for (int i = 0; i < 36; ++i)
        out[i] = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint64_t n = grp * 8 + j;
        uint64_t w0 = sm64(key, 3 * n);
        uint64_t w1 = sm64(key, 3 * n + 1);
        uint64_t w2 = sm64(key, 3 * n + 2);
        uint32_t sc = table[w2 >> 48];
        uint8_t b[18];
        b[0] = (uint8_t)sc;
        b[1] = (uint8_t)(sc >> 8);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            b[2 + q] = (uint8_t)(w0 >> (8 * q));
            b[10 + q] = (uint8_t)(w1 >> (8 * q));
        }
#pragma unroll
        for (int q = 0; q < 18; ++q) {
            int byte = 18 * j + q;
            out[byte >> 2] |= (uint32_t)b[q] << (8 * (byte & 3));
        }
    }
    uint4 *d = reinterpret_cast<uint4 *>(dst + blob * blob_bytes + grp * 144);
#pragma unroll
    for (int i = 0; i < 9; ++i)
        d[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

} // namespace

extern "C" {

// Fill n_blobs consecutive blobs at dst with the blobs of ids first_blob ..
// first_blob + n_blobs - 1 for `seed`.  H and FF are multiples of 64; dst is
// 16-byte aligned; table is a device array of 65536 fp16 bit patterns.
// Returns 0, -1 on bad arguments, -4 on a launch error.
int strata_inputs_fill_blobs(void *dst, uint64_t seed, int64_t first_blob, int64_t n_blobs,
                             int H, int FF, const uint16_t *table, void *stream)
{
    if (!dst || !table || n_blobs <= 0 || first_blob < 0 || H <= 0 || FF <= 0 || H % 64 ||
        FF % 64 || ((uintptr_t)dst & 15))
        return -1;
    uint64_t blocks = 3ull * (uint64_t)H * (uint64_t)FF / 64;
    uint64_t blob_bytes = blocks * 18;
    uint64_t gpb = blocks / 8;
    uint64_t total = gpb * (uint64_t)n_blobs;
    uint64_t base = sm64(seed, 0);
    const int tpb = 256;
    uint64_t grid = (total + tpb - 1) / tpb;
    if (grid > 0x7fffffffull)
        return -1;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)grid), dim3(tpb), 0, (hipStream_t)stream,
                       (uint8_t *)dst, base, (uint64_t)first_blob, gpb, total, blob_bytes, table);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

} // extern "C"
