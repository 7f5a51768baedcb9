// store_check.hip -- checksums of the expert blobs in HBM, and a verification
// that refuses a store whose blobs differ from the checksums expected of them.
//
// The engine the pages describe reads every cache slot back, byte for byte,
// after filling it, and refuses to run on a mismatch ("MoE 遇上消费级显卡..."
// (zwxr.cn), the passage on how the design differs from static offload, its
// third point).  Here the whole store lives in HBM and is filled once; its
// analogue is a checksum per blob, computed on the device and compared with
// the checksums of the bytes the store was filled from.
//
// checksum(blob) = sum over the blob's little-endian 64-bit words w_j
// (j = 0 .. BLOB / 8 - 1) of mix(w_j + (j + 1) * 0x9E3779B97F4A7C15), mod 2^64,
// where mix is the output function of SplitMix64 (Steele, Lea and Flood,
// "Fast splittable pseudorandom number generators", 2014).  The terms are
// added as integers, so the order of the additions does not matter and each
// lane of the device kernel takes its own words; a changed byte changes one
// term, and two words that trade places change two (the index is mixed in).
#include "common.hpp"
#include "strata_moe.h"

namespace strata {
namespace {

constexpr uint64_t CK_GOLD = 0x9E3779B97F4A7C15ull;
constexpr int CK_WORDS = BLOB / 8;      // 172,800 words per blob
constexpr int CK_PAIRS = CK_WORDS / 2;  // 86,400 16-byte loads per blob
constexpr int CK_THREADS = 256;
static_assert(BLOB % 16 == 0, "whole 16-byte pairs");

__host__ __device__ inline uint64_t ck_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t ck_term(uint64_t w, uint64_t j)
{
    return ck_mix(w + (j + 1) * CK_GOLD);
}

// One workgroup per blob.
__global__ __launch_bounds__(CK_THREADS) void checksum_kernel(const uint8_t *__restrict__ blobs,
                                                              uint64_t *__restrict__ sums)
{
    __shared__ uint64_t part[CK_THREADS / 64];
    const int tid = threadIdx.x;
    const ulonglong2 *p = reinterpret_cast<const ulonglong2 *>(blobs + (size_t)blockIdx.x * BLOB);
    uint64_t s = 0;
    for (int i = tid; i < CK_PAIRS; i += CK_THREADS) {
        const ulonglong2 v = p[i];
        s += ck_term(v.x, 2 * (uint64_t)i) + ck_term(v.y, 2 * (uint64_t)i + 1);
    }
    for (int d = 32; d > 0; d >>= 1)
        s += __shfl_xor(s, d, 64);
    if ((tid & 63) == 0)
        part[tid >> 6] = s;
    __syncthreads();
    if (tid == 0)
        sums[blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

} // namespace
} // namespace strata

extern "C" {

STRATA_API int strata_moe_blob_checksums(const uint8_t *blobs, int64_t nblobs, uint64_t *sums,
                                         void *stream)
{
    using namespace strata;
    if (!blobs || !sums)
        return STRATA_E_ARG;
    if (nblobs <= 0 || nblobs > STRATA_MOE_CHECK_BLOBS_MAX)
        return STRATA_E_SHAPE;
    if (!aligned(blobs, 256) || !aligned(sums, 8))
        return STRATA_E_ALIGN;
    hipLaunchKernelGGL(checksum_kernel, dim3((unsigned)nblobs), dim3(CK_THREADS), 0,
                       (hipStream_t)stream, blobs, sums);
    return hipGetLastError() == hipSuccess ? STRATA_OK : STRATA_E_HIP;
}

STRATA_API uint64_t strata_moe_blob_checksum_host(const uint8_t *blob)
{
    using namespace strata;
    if (!blob)
        return 0;
    uint64_t s = 0;
    for (int j = 0; j < CK_WORDS; ++j) {
        uint64_t w = 0;
        for (int b = 7; b >= 0; --b)   // little-endian word j
            w = (w << 8) | blob[8 * (size_t)j + b];
        s += ck_term(w, (uint64_t)j);
    }
    return s;
}

STRATA_API int strata_moe_verify_blobs(const uint8_t *blobs, int64_t nblobs,
                                       const uint64_t *expected, uint64_t *sums,
                                       int64_t *first_bad, void *stream)
{
    using namespace strata;
    if (!expected || !first_bad)
        return STRATA_E_ARG;
    *first_bad = -1;
    int rc = strata_moe_blob_checksums(blobs, nblobs, sums, stream);
    if (rc != STRATA_OK)
        return rc;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
        return STRATA_E_HIP;
    uint64_t got[512];   // compared a chunk at a time: nothing allocated
    for (int64_t b0 = 0; b0 < nblobs; b0 += 512) {
        const int64_t n = nblobs - b0 < 512 ? nblobs - b0 : 512;
        if (hipMemcpy(got, sums + b0, (size_t)n * sizeof(uint64_t), hipMemcpyDeviceToHost) !=
            hipSuccess)
            return STRATA_E_HIP;
        for (int64_t i = 0; i < n; ++i) {
            if (got[i] != expected[b0 + i]) {
                *first_bad = b0 + i;
                return STRATA_E_CORRUPT;
            }
        }
    }
    return STRATA_OK;
}

} // extern "C"
