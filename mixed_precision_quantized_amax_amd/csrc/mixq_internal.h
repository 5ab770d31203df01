// Internal helpers of the mixq library (host validation, device check,
// small device utilities).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mixq.h"

namespace mixq {

constexpr int kWave = 64;

// ---- host side -------------------------------------------------------------
int check_device_cached();  // MIXQ_OK / MIXQ_ERR_NO_DEVICE / MIXQ_ERR_UNSUPPORTED_DEVICE
int device_cu_count();      // compute units of the current device (after the check)

// Split-K plan of the thin-product GEMM (128x128 K-pair tiles): K is split
// in two when the product has fewer tiles than the device has compute units
// (INT8 weights, whole 128-byte K pairs in each half).  The kernel handles
// any split count S (the last of S blocks to arrive reduces).
constexpr int kSplitTile = 128;
constexpr int64_t kSplitSyncBytes = 4096;                          // tile counters
constexpr int64_t kSplitSlotBytes = (int64_t)kSplitTile * kSplitTile * 4;  // int32 partial tile
inline int64_t split_tiles(int64_t M, int64_t N) {
    return ((M + kSplitTile - 1) / kSplitTile) * ((N + kSplitTile - 1) / kSplitTile);
}
inline int split_plan(int64_t M, int64_t N, int64_t K, int bits, int cus) {
    if (bits != 8 || K % 256 != 0 || M <= 0 || N <= 0) return 1;
    if (((M + 255) / 256) * ((N + 255) / 256) >= 192) return 1;  // the 256x256 path
    const int64_t tiles = split_tiles(M, N);
    if (tiles >= cus || tiles > kSplitSyncBytes / 4) return 1;
    return 2;  // (four-way splits measured slower: the last block reads three partials)
}
inline int64_t split_workspace_bytes(int64_t M, int64_t N, int S) {
    return kSplitSyncBytes + split_tiles(M, N) * S * kSplitSlotBytes;
}
// Tail split of a product on 256 x 256 tiles (K a multiple of 128) that
// needs one round of the device plus a short second one: the columns
// [0, n_split) keep 256 x 256 tiles, the rest run as 128 x 128 tiles with K
// split *S ways (S in 1, 2, 4) so that the tail fills about two blocks per
// compute unit.  Returns n_split, or 0 for no tail split.
inline int tail_plan(int64_t M, int64_t N, int64_t K, int cus, int* S) {
    *S = 1;
    if (M <= 0 || N <= 0 || K % 128 != 0 || cus <= 0) return 0;
    const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256;
    if (tm * tn < 192) return 0;  // not the 256x256 path
    const int64_t fit = cus / tm;  // whole tile columns in one round
    if (fit <= 0 || tn <= fit || 2 * (tn - fit) * tm > cus) return 0;
    const int64_t n_split = fit * 256;
    const int64_t tail = split_tiles(M, N - n_split);
    if (tail <= kSplitSyncBytes / 4)
        while (*S < 4 && tail * *S * 2 <= 2 * (int64_t)cus && K % (128 * 2 * *S) == 0) *S *= 2;
    return (int)n_split;
}
inline int64_t tail_workspace_bytes(int64_t M, int64_t N, int64_t n_split, int S) {
    return kSplitSyncBytes + split_tiles(M, N - n_split) * S * kSplitSlotBytes;
}

inline bool valid_k(int64_t K) { return K > 0 && K % MIXQ_K_MULTIPLE == 0 && K <= MIXQ_K_MAX; }

// Value of a non-negative fp16 bit pattern (host side, exact).
inline float half_bits_value(uint32_t h) {
    const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
    if (e == 0u) return ldexpf((float)m, -24);
    return ldexpf((float)(m + 1024u), (int)e - 25);
}

inline int64_t outlier_ld(int32_t k_cap) {
    return ((int64_t)k_cap + MIXQ_OUTLIER_ALIGN - 1) / MIXQ_OUTLIER_ALIGN * MIXQ_OUTLIER_ALIGN;
}

inline int64_t bitmap_words(int64_t K) { return (K + 31) / 32; }

// Bit pattern of the largest finite fp16 value <= t (t >= 0, finite).  For an
// fp16 value x >= 0:  x > t  <=>  bits(x) > half_floor_bits(t).
inline uint32_t half_floor_bits(float t) {
    if (!(t > 0.0f)) return 0u;
    if (t >= 65504.0f) return 0x7BFFu;
    // binary search over the bit patterns, which are ordered like the values
    uint32_t lo = 0u, hi = 0x7BFFu;
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1u) / 2u;
        if (half_bits_value(mid) <= t)
            lo = mid;
        else
            hi = mid - 1u;
    }
    return lo;
}

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MIXQ_OK : MIXQ_ERR_HIP;
}

// ---- device side -------------------------------------------------------------
// Source row of packed row n: n itself, or for a gated weight ([W_gate;
// W_up], N = 2I) the 32-row blocks of gate and up rows interleaved, so that
// the GEMM epilogue finds gate j and up j in neighbouring fragments.
__device__ __forceinline__ int64_t src_row(int64_t n, int64_t N, int gated) {
    if (!gated) return n;
    const int64_t blk = n >> 6, within = n & 63;
    return within < 32 ? blk * 32 + within : N / 2 + blk * 32 + (within - 32);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (float)v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o, kWave);
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int u = __shfl_up(v, o, kWave);
        if (lane >= o) v += u;
    }
    return v;
}

// Device-scope (L2) load that bypasses the non-coherent per-CU cache.
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_agent(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mixq
