// Activation side of the mixed-precision linear layer: fused amax, gate,
// outlier detection, per-token INT8 quantization and outlier extraction.
//
// MixQ article, section "MixQ的解决方案":
//   - outliers recur in fixed channels across decode steps (Fig. 9), so the
//     channel set is cached in device memory and re-used;
//   - the amax needed for the quantization scale also says whether any
//     outlier exists (amax greater than the threshold), so detection only
//     matters when that amax, taken over the uncached channels, crosses the
//     threshold (Fig. 10, the equivalent transform);
//   - outliers go, in channel order, into a separate FP16 matrix (Fig. 11).
//   Prior systems lost time to atomics (Fig. 8): here the steady-state path
//   issues none.
//
// Two kernels per call, both on the caller's stream, one wave per token:
//   gate_quant  one pass over X: masked amax, quantization with the cached
//               set, X_out gather (a channel's column is its rank in the set,
//               kept as a prefix-popcount table in the state).  Uncached
//               values above the threshold -- the gate -- are marked in LDS
//               and, only then, OR-ed into a pending bitmap with one marker.
//   requant     reads the marker.  No marker: writes flag = 0 and exits.
//               Marker: every block forms the union set and its rank table in
//               LDS, re-quantizes its tokens with it, and the last block to
//               finish commits the set (bitmap, ranks, ascending ids, count,
//               flag) and clears the scratch.
#include "mixq_internal.h"

#pragma clang fp contract(off)

namespace mixq {
namespace {

struct ActArgs {
    const uint16_t* X;
    int64_t M;
    int32_t K;
    int64_t ldx;
    float tau;
    uint32_t tau_bits;  // bits of the largest fp16 value <= tau
    int32_t* idx;
    int32_t* count;
    int32_t* flag;
    uint32_t* bitmap;
    uint32_t* pending;  // work[0, words)
    int32_t* rank;      // work[words, 2 words): exclusive popcount prefix of bitmap
    uint32_t* marker;   // work[2 words]
    uint32_t* arrive;   // work[2 words + 1]
    uint32_t* set_id;   // work[2 words + 2]: serial of the committed set (0 = empty)
    uint32_t* pend_id;  // work[2 words + 3]: serial the pending set will commit under
    int32_t k_cap;
    int32_t words;
    int32_t nchunks;  // K / 8
    int8_t* Xq;
    float* s_x;
    uint16_t* X_out;
    int32_t ld_out;
    // RMSNorm prologue (gamma null: X is quantized as given)
    const uint16_t* gamma;
    float eps;
    float* rstd;
    // residual add before the norm (D null: none): X is R, H = R + D is written
    const uint16_t* D;
    int64_t ldd;
    uint16_t* H;
    int64_t ldh;
};

// LDS table: for the 8 cached-channel bits of a chunk (8 halves = 4 dwords),
// the dword masks that keep the uncached halves (0xFFFF) and clear the cached
// ones.  Built once per block.
constexpr int kLutEntries = 256;

__device__ __forceinline__ void build_keep_lut(uint4* lut) {
    for (int c = threadIdx.x; c < kLutEntries; c += blockDim.x) {
        uint32_t d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            d[j] = (((c >> (2 * j)) & 1) ? 0u : 0x0000FFFFu) |
                   (((c >> (2 * j + 1)) & 1) ? 0u : 0xFFFF0000u);
        lut[c] = make_uint4(d[0], d[1], d[2], d[3]);
    }
}

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Buffer descriptor over `bytes` bytes from base (raw, no stride): loads past
// the end read zeros, stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes,
                                             0x00020000);
}

// Two 16-bit unsigned maxima in one packed integer operation.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a),
                                                                  __builtin_bit_cast(us2, b)));
}

__device__ __forceinline__ uint16_t half_at(const uint4& v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (uint16_t)(w >> ((e & 1) * 16));
}

// Code of one value: round half to even of x*r.  The product is one fp32
// rounding (fma with a zero addend, the fp16 operand widened exactly);
// adding 1.5 * 2^23 rounds it to the nearest integer (ties to even) and
// leaves that integer in the low bits of the sum.  No clamp is needed: every
// quantized value satisfies |x| <= g with r = fl(127 / g), so
// |fl(x * r)| <= 127 (1 + 2^-24)^2 < 127.5 and the code is within [-127, 127]
// (finite inputs; g = 0 gives r = 1 and all-zero values).
__device__ __forceinline__ uint32_t code_bits(uint16_t h, float r) {
    const float t = __builtin_fmaf(half_bits_to_float(h), r, 0.0f);
    return __float_as_uint(t + 12582912.0f);
}

// Low bytes of four code words -> one dword (byte k from word k).
__device__ __forceinline__ uint32_t pack4(uint32_t u0, uint32_t u1, uint32_t u2, uint32_t u3) {
    const uint32_t p01 = __builtin_amdgcn_perm(u1, u0, 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm(u3, u2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}

// ---- RMSNorm prologue ------------------------------------------------------------
// The token's sum of squares is kept exact as an unevaluated pair hi + lo of
// doubles.  Every fp16 value is a multiple of 2^-24, so every square, partial
// sum and rounding error below is a multiple of 2^-48, and a square is exact
// in binary32 (22 significant bits, no underflow).  two_sum is Knuth's
// error-free transform: hi + lo does not change.  lo, the running sum of the
// rounding errors, is itself exact while |lo| < 2^5 (53 bits of 2^-48 steps):
// with |h| < 2^16, K <= 2^15 and at most K/256 squares per lane, a lane's
// partial stays below 2^39, so each of its errors is at most 2^-15 and their
// sum below 2^-8; the 255 combines of lane and wave partials add at most
// 2^-7 each.  So |lo| < 2, the pair is the exact sum, and fl(hi + lo) is that
// sum rounded once to binary64 -- whatever the order of accumulation.
// All terms are non-negative, so ordering the two addends by max/min meets
// the condition of Dekker's Fast2Sum (|a| >= |b|), which then gives the
// exact rounding error in three operations.
__device__ __forceinline__ void two_sum(double& hi, double& lo, double b) {
    const double x = __builtin_fmax(hi, b), y = __builtin_fmin(hi, b);
    const double s = x + y;
    lo += y - (s - x);
    hi = s;
}

__device__ __forceinline__ void pair_add(double& hi, double& lo, double hi2, double lo2) {
    two_sum(hi, lo, hi2);
    lo += lo2;
}

__device__ __forceinline__ void sumsq_chunk(const uint4& v, double& hi, double& lo) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // the square of an fp16 value is exact in binary32 (one fma from fp16)
        const float f = half_bits_to_float((uint16_t)(w[e >> 1] >> ((e & 1) * 16)));
        two_sum(hi, lo, (double)__builtin_fmaf(f, f, 0.0f));
    }
}

// Butterfly over the wave; every lane ends with the same exact pair.
__device__ __forceinline__ void wave_pair_sum(double& hi, double& lo) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const double h2 = __shfl_xor(hi, o, kWave);
        const double l2 = __shfl_xor(lo, o, kWave);
        pair_add(hi, lo, h2, l2);
    }
}

// rstd = 1 / sqrt(fp32(S / K) + eps): the exact sum rounded to binary64, one
// binary64 division, then binary32 add, square root and division (all
// correctly rounded).  A zero denominator (all-zero token, eps = 0) gives 0.
__device__ __forceinline__ float rstd_of(double hi, double lo, int K, float eps) {
    const double S = hi + lo;
    const float ms = (float)(S / (double)K);
    const float t = ms + eps;
    return t == 0.0f ? 0.0f : 1.0f / __builtin_sqrtf(t);
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// x = fp16(fp16(h * r) * gamma) for the two halves of a dword: the binary32
// product rounded to fp16, then the fp16 product (exact in binary32) rounded.
// The empty asm pins the binary32 products: without it the compiler may fold
// product and narrowing into one mixed-precision fma (v_fma_mixlo_f16), which
// rounds once instead of twice and so differs at rare ties.
__device__ __forceinline__ uint32_t norm2(uint32_t hw, uint32_t gw, float r) {
    float p0 = half_bits_to_float((uint16_t)hw) * r;
    float p1 = half_bits_to_float((uint16_t)(hw >> 16)) * r;
    asm volatile("" : "+v"(p0), "+v"(p1));
    const half2v n = {(_Float16)p0, (_Float16)p1};
    return __builtin_bit_cast(uint32_t, n * __builtin_bit_cast(half2v, gw));
}

__device__ __forceinline__ uint4 norm_chunk(const uint4& v, const uint4& g, float r) {
    return make_uint4(norm2(v.x, g.x, r), norm2(v.y, g.y, r), norm2(v.z, g.z, r),
                      norm2(v.w, g.w, r));
}

__device__ __forceinline__ uint16_t norm1(uint16_t h, uint16_t g, float r) {
    return (uint16_t)norm2(h, g, r);
}

// fp16 sums of two dwords of halves (v_pk_add_f16: the exact sum rounded to
// fp16, ties to even)
__device__ __forceinline__ uint32_t hadd2(uint32_t x, uint32_t y) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, x) + __builtin_bit_cast(half2v, y));
}

__device__ __forceinline__ uint4 hadd_chunk(const uint4& x, const uint4& y) {
    return make_uint4(hadd2(x.x, y.x), hadd2(x.y, y.y), hadd2(x.z, y.z), hadd2(x.w, y.w));
}

// One token processed by one wave.  Chunk = 8 consecutive channels (16 B);
// lane l owns chunks l, l+64, ... of each segment of 64*CPT chunks, so every
// load instruction of the wave reads 1 KB of the row contiguously.
//   set_words / rank: the set the token is quantized with (global or LDS)
//   lut: keep-mask table (LDS)
//   newbits: LDS detection bitmap, or null when detection is off
// The amax is taken on the fp16 bit patterns: for non-negative halves the
// integer order is the value order, so the packed unsigned max is exact.
// Returns (in every lane) whether this token had an uncached value above tau.
//   GATHER_IDX: X_out is filled from the ascending channel list a.idx (the
//   committed set) with one coalesced pass per row; otherwise from the
//   bitmap and rank table (the set being formed, whose list does not exist
//   yet).
//   NORM: the row is RMS-normalised as it is loaded, with the token's stored
//   rstd (requant only; the steady-state pass computed it).
template <int CPT, bool GATHER_IDX, bool NORM = false>
__device__ bool wave_row(const ActArgs& a, int64_t row, const uint32_t* set_words,
                         const int32_t* rank, int set_size, const uint4* lut, uint32_t* newbits) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint16_t* xr = a.X + row * a.ldx;
    const int seg_chunks = kWave * CPT;
    const int nseg = (a.nchunks + seg_chunks - 1) / seg_chunks;

    static_assert(!(NORM && GATHER_IDX), "the normalised gather reads the set from the bitmap");
    uint4 xv[CPT];
    uint32_t wv[CPT];
    int32_t rk[CPT];  // rank of the first channel of the chunk's bitmap word
    uint32_t amx = 0;  // packed max of |x| bits (two halves)
    const float rn = NORM ? a.rstd[row] : 0.0f;
    auto load_seg = [&](int s) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = s * seg_chunks + i * kWave + lane;
            if (c < a.nchunks) {
                xv[i] = *reinterpret_cast<const uint4*>(xr + (int64_t)c * 8);
                if constexpr (NORM)
                    xv[i] = norm_chunk(xv[i], *reinterpret_cast<const uint4*>(a.gamma + (int64_t)c * 8),
                                       rn);
                wv[i] = set_words[c >> 2];
                rk[i] = GATHER_IDX ? 0 : rank[c >> 2];
            } else {
                xv[i] = make_uint4(0, 0, 0, 0);
                wv[i] = 0u;
                rk[i] = 0;
            }
        }
    };
    auto keep_of = [&](int i, int c) -> uint4 {
        return lut[(wv[i] >> ((c & 3) * 8)) & 0xFFu];
    };
    for (int s = 0; s < nseg; ++s) {
        load_seg(s);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = s * seg_chunks + i * kWave + lane;
            const uint4 kp = keep_of(i, c);
            amx = pk_max_u16(amx, xv[i].x & kp.x & 0x7FFF7FFFu);
            amx = pk_max_u16(amx, xv[i].y & kp.y & 0x7FFF7FFFu);
            amx = pk_max_u16(amx, xv[i].z & kp.z & 0x7FFF7FFFu);
            amx = pk_max_u16(amx, xv[i].w & kp.w & 0x7FFF7FFFu);
        }
    }
    uint32_t gb = max(amx & 0xFFFFu, amx >> 16);
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) gb = max(gb, (uint32_t)__shfl_xor((int)gb, o, kWave));

    bool det = false;
    if (newbits && gb > a.tau_bits) {
        // The gate fired for this token (rare): mark every uncached channel
        // above the threshold.  Reads the row again segment by segment.
        for (int s = 0; s < nseg; ++s) {
            if (nseg > 1) load_seg(s);
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = s * seg_chunks + i * kWave + lane;
                if (c >= a.nchunks) continue;
                const uint32_t cb = (wv[i] >> ((c & 3) * 8)) & 0xFFu;
                uint32_t over = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (!((cb >> e) & 1u) && (uint32_t)(half_at(xv[i], e) & 0x7FFFu) > a.tau_bits)
                        over |= 1u << e;
                if (over) atomicOr(&newbits[c >> 2], over << ((c & 3) * 8));
            }
        }
        det = true;
    }

    // Scale and reciprocal: single IEEE divisions; zero amax -> 1.
    const float g = half_bits_to_float((uint16_t)gb);
    float sc, r;
    if (gb == 0u) {
        sc = 1.0f;
        r = 1.0f;
    } else {
        sc = g / 127.0f;
        r = 127.0f / g;
    }
    if (lane == 0) a.s_x[row] = sc;

    int8_t* qr = a.Xq + row * (int64_t)a.K;
    uint16_t* orow = a.ld_out ? a.X_out + row * (int64_t)a.ld_out : nullptr;
    for (int s = 0; s < nseg; ++s) {
        if (nseg > 1) load_seg(s);  // the row did not fit in registers: read it again
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = s * seg_chunks + i * kWave + lane;
            if (c >= a.nchunks) continue;
            const uint32_t cb = (wv[i] >> ((c & 3) * 8)) & 0xFFu;
            const uint4 kp = keep_of(i, c);
            // cached channels become +0 and so get code 0
            const uint32_t m[4] = {xv[i].x & kp.x, xv[i].y & kp.y, xv[i].z & kp.z, xv[i].w & kp.w};
            uint32_t u[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = code_bits((uint16_t)(m[e >> 1] >> ((e & 1) * 16)), r);
            *reinterpret_cast<uint2*>(qr + (int64_t)c * 8) =
                make_uint2(pack4(u[0], u[1], u[2], u[3]), pack4(u[4], u[5], u[6], u[7]));
            if (!GATHER_IDX && cb) {
                // outlier channels: column in X_out = rank in the set
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if ((cb >> e) & 1u) {
                        const int bit = (c & 3) * 8 + e;
                        orow[rk[i] + __popc(wv[i] & ((1u << bit) - 1u))] = half_at(xv[i], e);
                    }
            }
        }
    }
    if (orow) {
        if constexpr (GATHER_IDX) {
            // the row is still in the caches: one gather load and one
            // contiguous store per 64 set members
            for (int j = lane; j < set_size; j += kWave) orow[j] = xr[a.idx[j]];
        }
        const int kpad = (set_size + MIXQ_OUTLIER_ALIGN - 1) / MIXQ_OUTLIER_ALIGN * MIXQ_OUTLIER_ALIGN;
        for (int j = set_size + lane; j < kpad; j += kWave) orow[j] = 0;
    }
    return __any(det);
}

// Serial numbers of committed sets, unique within the process on each device
// (0 is never issued: it names the empty set of a zero-filled state).  A
// packed weight records the serial its outlier columns were gathered for, so
// a set that changed -- grown, reset, or another state's set of the same
// size -- is always told apart from the one the columns hold.
__device__ uint32_t g_set_serial = 0u;

__device__ __forceinline__ uint32_t next_set_serial() {
    uint32_t s = atomicAdd(&g_set_serial, 1u) + 1u;
    if (s == 0u) s = atomicAdd(&g_set_serial, 1u) + 1u;  // after 2^32 commits: skip 0
    return s;
}

constexpr int kGateThreads = 256;

// The steady-state pass: W waves per token, each owning a contiguous part of
// the row (CPT chunks per lane and segment), so that a token's chain of
// load -> amax -> quantize -> store is W times shorter than with one wave per
// token and the memory traffic of the waves overlaps.  The token's amax is
// combined through LDS (one barrier per token group).  The cached set's
// bitmap is staged in LDS; the outlier gather reads the committed channel
// list and issues its loads together with the row's, so their latency hides
// behind the amax.
//
// NORM: the pass starts with the RMSNorm of the token (the operation before
// the layer, fused as the MixQ article allows for the amax): its exact sum
// of squares is combined through LDS like the amax, the part in registers is
// normalised in place, rstd is stored for the re-quantize pass.  The whole
// part must fit in registers (one segment: K <= 32768).
// RES: before that, the residual add H = R + D (X is R), H written out; one
// token buffer (R and D both in flight) instead of two.
// EXACT: K is exactly one segment (W * 64 * CPT chunks of 8 channels), so no
// chunk of a row is out of range and no per-chunk test is compiled in (the
// tests and their masked paths were the larger part of the pass's vector
// instructions).
// ONE: the grid has a block for every token group, so each block takes one
// group and needs one register set, not two (fewer registers, more waves per
// SIMD).
template <int CPT, int W, bool NORM, bool RES = false, bool EXACT = false, bool ONE = false>
__global__ __launch_bounds__(kGateThreads) void gate_quant_kernel(ActArgs a) {
    static_assert(!(ONE && RES), "the residual variant keeps one register set anyway");
    static_assert(!RES || NORM, "the residual add comes with the norm");
    constexpr int kRB = kGateThreads / kWave / W;  // tokens per block and round
    extern __shared__ uint32_t dyn[];  // newbits[words], sbits[words], NORM: gamma[K]
    uint32_t* const newbits = dyn;
    uint32_t* const sbits = dyn + a.words;
    const uint16_t* const sgam = reinterpret_cast<const uint16_t*>(dyn + 2 * a.words);
    __shared__ uint4 lut[kLutEntries];
    __shared__ uint32_t red[2][kRB][W];
    __shared__ double rsum[NORM ? 2 : 1][kRB][W][2];
    __shared__ int any_det;
    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform (a scalar register): the token row and its buffer
    // descriptor are then scalar too, and each row load issues once (a
    // descriptor in vector registers needs a loop over its distinct values)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int slot = wave / W, part = wave % W;
    const int seg_chunks = W * kWave * CPT;
    const int nseg = EXACT ? 1 : (a.nchunks + seg_chunks - 1) / seg_chunks;
    auto chunk = [&](int s, int i) { return s * seg_chunks + (part * CPT + i) * kWave + lane; };
    auto in_range = [&](int c) __attribute__((always_inline)) { return EXACT || c < a.nchunks; };
    typedef uint4 XV[CPT];
    typedef uint32_t WV[CPT];
    // X chunks of one segment of a token's part (global loads only)
    // (buffer loads: a row past M or a chunk past K reads zeros through the
    // descriptor's range, and the per-lane offsets are 32-bit)
    auto load_x = [&](int64_t row, int s, XV& xv) {
        const bool valid = row < a.M;
        const __amdgpu_buffer_rsrc_t rx =
            row_rsrc(a.X + (valid ? row : 0) * a.ldx, valid ? (int64_t)a.K * 2 : 0);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = chunk(s, i);
            const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rx, c * 16, 0, 0);
            xv[i] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };
    // The first token's row loads go out before anything else: before the
    // set size is read (the wait for a scalar load holds back every later
    // instruction), and before the cached set is staged in LDS, so that the
    // memory latencies overlap (the set's bits are read from LDS only when
    // the amax needs them).
    XV xa, xb;
    WV wa, wb;
    uint16_t ga = 0, gb2 = 0;
    int64_t r0 = (int64_t)blockIdx.x * kRB;
    if (!RES && r0 < a.M) load_x(r0 + slot, 0, xa);
    const int set_size = *a.count;
    const int kpad = (set_size + MIXQ_OUTLIER_ALIGN - 1) / MIXQ_OUTLIER_ALIGN * MIXQ_OUTLIER_ALIGN;
    // first gather round: set member gj of each token (its channel id is
    // read once per block)
    const int gj = part * kWave + lane;
    const bool gset = a.ld_out && gj < set_size;
    // Its channel id: a range-checked load over the committed list (lanes
    // past the set read 0), with no branch around it, so that nothing waits
    // for it before the row loads go out (a load inside a divergent branch
    // is waited for where the branch ends).
    const int gch = (int)__builtin_amdgcn_raw_buffer_load_b32(
        row_rsrc(a.idx, a.ld_out ? (int64_t)set_size * 4 : 0), gj * 4, 0, 0);
    // the cached-set bits of the same chunks (from the bitmap staged in LDS)
    auto load_bits = [&](int s, WV& wv) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = chunk(s, i);
            wv[i] = in_range(c) ? sbits[c >> 2] : 0u;
        }
    };
    auto load_seg = [&](int64_t row, int s, XV& xv, WV& wv) {
        load_x(row, s, xv);
        load_bits(s, wv);
    };
    // a token's first gather value (a range-checked 2-byte load from its
    // row: 0 for a lane that holds no set member or a row past M, values
    // that are never stored)
    auto load_gather = [&](int64_t row, uint16_t& gv) {
        const bool valid = row < a.M;
        const __amdgpu_buffer_rsrc_t rx =
            row_rsrc(a.X + (valid ? row : 0) * a.ldx, valid ? (int64_t)a.K * 2 : 0);
        gv = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rx, gset ? gch * 2 : a.K * 2, 0, 0);
    };
    // the first segment of a token's part and its first gather value
    auto load_row = [&](int64_t row, XV& xv, uint16_t& gv) {
        load_x(row, 0, xv);
        load_gather(row, gv);
    };
    build_keep_lut(lut);
    for (int w = threadIdx.x; w < a.words; w += kGateThreads) {
        newbits[w] = 0u;
        sbits[w] = a.bitmap[w];
    }
    // after the set's staging: the channel-id load must have landed first,
    // and (completions in order) so have the row loads before it, whose
    // lines then hold this value
    if (!RES && r0 < a.M) load_gather(r0 + slot, ga);
    if constexpr (NORM) {
        uint4* const g4 = reinterpret_cast<uint4*>(dyn + 2 * a.words);
        for (int c = threadIdx.x; c < a.nchunks; c += kGateThreads)
            g4[c] = *reinterpret_cast<const uint4*>(a.gamma + (int64_t)c * 8);
    }
    if (threadIdx.x == 0) any_det = 0;
    __syncthreads();

    // RES: the matching D chunks and gather value
    auto load_d = [&](int64_t row, XV& dv, uint16_t& gd) {
        const bool valid = row < a.M;
        const uint16_t* dr = a.D + (valid ? row : 0) * a.ldd;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = chunk(0, i);
            dv[i] = (valid && in_range(c)) ? *reinterpret_cast<const uint4*>(dr + (int64_t)c * 8)
                                           : make_uint4(0, 0, 0, 0);
        }
        if (gset && valid) gd = dr[gch];
    };
    bool det = false;
    auto process = [&](int64_t row, XV& xv, WV& wv, uint16_t gval, int parity, const XV* dv,
                       uint16_t gd) {
        const bool valid = row < a.M;
        const uint16_t* xr = a.X + (valid ? row : 0) * a.ldx;
        uint16_t* orow = (a.ld_out && valid) ? a.X_out + row * (int64_t)a.ld_out : nullptr;
        auto keep_of = [&](int i, int c) -> uint4 { return lut[(wv[i] >> ((c & 3) * 8)) & 0xFFu]; };
        load_bits(0, wv);

        if constexpr (RES) {
            uint16_t* hr = a.H + (valid ? row : 0) * a.ldh;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = chunk(0, i);
                xv[i] = hadd_chunk(xv[i], (*dv)[i]);
                if (valid && in_range(c)) *reinterpret_cast<uint4*>(hr + (int64_t)c * 8) = xv[i];
            }
            gval = (uint16_t)hadd2(gval, gd);
        }

        float rn = 0.0f;
        if constexpr (NORM) {
            double hi = 0.0, lo = 0.0;
#pragma unroll
            for (int i = 0; i < CPT; ++i) sumsq_chunk(xv[i], hi, lo);
            wave_pair_sum(hi, lo);
            if (lane == 0) {
                rsum[parity][slot][part][0] = hi;
                rsum[parity][slot][part][1] = lo;
            }
            __syncthreads();
            hi = rsum[parity][slot][0][0];
            lo = rsum[parity][slot][0][1];
#pragma unroll
            for (int w = 1; w < W; ++w) pair_add(hi, lo, rsum[parity][slot][w][0], rsum[parity][slot][w][1]);
            rn = rstd_of(hi, lo, a.K, a.eps);
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = chunk(0, i);
                if (in_range(c))
                    xv[i] = norm_chunk(xv[i], *reinterpret_cast<const uint4*>(sgam + c * 8), rn);
            }
            gval = norm1(gval, sgam[gch], rn);  // gamma staged in LDS
            if (valid && part == 0 && lane == 0) a.rstd[row] = rn;
        }

        uint32_t amx = 0;
        for (int s = 0; s < nseg; ++s) {
            if (s > 0) load_seg(row, s, xv, wv);
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const uint4 kp = keep_of(i, chunk(s, i));
                amx = pk_max_u16(amx, xv[i].x & kp.x & 0x7FFF7FFFu);
                amx = pk_max_u16(amx, xv[i].y & kp.y & 0x7FFF7FFFu);
                amx = pk_max_u16(amx, xv[i].z & kp.z & 0x7FFF7FFFu);
                amx = pk_max_u16(amx, xv[i].w & kp.w & 0x7FFF7FFFu);
            }
        }
        uint32_t gb = max(amx & 0xFFFFu, amx >> 16);
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1)
            gb = max(gb, (uint32_t)__shfl_xor((int)gb, o, kWave));
        if (lane == 0) red[parity][slot][part] = gb;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < W; ++w) gb = max(gb, red[parity][slot][w]);

        if (gb > a.tau_bits) {
            // The gate fired for this token (rare): mark every uncached
            // channel of this wave's part above the threshold.
            for (int s = 0; s < nseg; ++s) {
                if (nseg > 1) load_seg(row, s, xv, wv);
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    const int c = chunk(s, i);
                    if (!valid || !in_range(c)) continue;
                    const uint32_t cb = (wv[i] >> ((c & 3) * 8)) & 0xFFu;
                    uint32_t over = 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (!((cb >> e) & 1u) && (uint32_t)(half_at(xv[i], e) & 0x7FFFu) > a.tau_bits)
                            over |= 1u << e;
                    if (over) atomicOr(&newbits[c >> 2], over << ((c & 3) * 8));
                }
            }
            det = true;
        }

        // scale and reciprocal: single IEEE divisions; zero amax -> 1
        const float g = half_bits_to_float((uint16_t)gb);
        float sc, r;
        if (gb == 0u) {
            sc = 1.0f;
            r = 1.0f;
        } else {
            sc = g / 127.0f;
            r = 127.0f / g;
        }
        if (valid && part == 0 && lane == 0) a.s_x[row] = sc;

        // codes: buffer stores, dropped past K or for a row past M
        const __amdgpu_buffer_rsrc_t rq =
            row_rsrc(a.Xq + (valid ? row : 0) * (int64_t)a.K, valid ? (int64_t)a.K : 0);
        for (int s = 0; s < nseg; ++s) {
            if (nseg > 1) load_seg(row, s, xv, wv);  // the part did not fit in registers
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = chunk(s, i);
                if (!EXACT && !in_range(c)) continue;
                const uint4 kp = keep_of(i, c);
                // cached channels become +0 and so get code 0
                const uint32_t m[4] = {xv[i].x & kp.x, xv[i].y & kp.y, xv[i].z & kp.z,
                                       xv[i].w & kp.w};
                uint32_t u[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    u[e] = code_bits((uint16_t)(m[e >> 1] >> ((e & 1) * 16)), r);
                const v2u q = {pack4(u[0], u[1], u[2], u[3]), pack4(u[4], u[5], u[6], u[7])};
                __builtin_amdgcn_raw_buffer_store_b64(q, rq, c * 8, 0, 0);
            }
        }
        if (orow) {
            if (gset) orow[gj] = gval;
            for (int j = gj + W * kWave; j < set_size; j += W * kWave) {
                const int ch = a.idx[j];
                uint16_t v = xr[ch];
                if constexpr (RES) v = (uint16_t)hadd2(v, a.D[row * a.ldd + ch]);
                orow[j] = NORM ? norm1(v, a.gamma[ch], rn) : v;
            }
            for (int j = set_size + gj; j < kpad; j += W * kWave) orow[j] = 0;
        }
    };
    // Tokens of this block, two register sets: the next token's loads are in
    // flight while the current one is processed.  The loop is block-uniform
    // (process has a barrier).
    const int64_t stride = (int64_t)gridDim.x * kRB;
    if constexpr (RES) {
        int par = 0;
        for (; r0 < a.M; r0 += stride) {
            XV da;
            uint16_t gd = 0;
            load_row(r0 + slot, xa, ga);
            load_d(r0 + slot, da, gd);
            process(r0 + slot, xa, wa, ga, par, &da, gd);
            par ^= 1;
        }
    } else if constexpr (ONE) {
        if (r0 < a.M) process(r0 + slot, xa, wa, ga, 0, nullptr, 0);
    } else {
    for (; r0 < a.M; r0 += 2 * stride) {
        if (r0 + stride < a.M) load_row(r0 + stride + slot, xb, gb2);
        process(r0 + slot, xa, wa, ga, 0, nullptr, 0);
        if (r0 + stride >= a.M) break;
        if (r0 + 2 * stride < a.M) load_row(r0 + 2 * stride + slot, xa, ga);
        process(r0 + stride + slot, xb, wb, gb2, 1, nullptr, 0);
    }
    }
    if (det && lane == 0) any_det = 1;
    __syncthreads();
    if (any_det) {  // block-uniform: only blocks whose tokens crossed the gate
        for (int w = threadIdx.x; w < a.words; w += kGateThreads)
            if (newbits[w]) atomicOr(&a.pending[w], newbits[w]);
        // the first block to raise the marker draws the serial that the grown
        // set will be committed under (a fused regather needs it before the
        // commit)
        if (threadIdx.x == 0 && atomicOr(a.marker, 1u) == 0u) *a.pend_id = next_set_serial();
    }
}

// Exclusive prefix of popcount(src[w]) into prefix[w] (LDS); returns the total.
// Block of any size; tot must hold one int per wave.
__device__ int scan_popcounts(const uint32_t* src, int words, int* prefix, int* tot) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nw = blockDim.x / kWave;
    const int per = (words + blockDim.x - 1) / blockDim.x;
    const int b = tid * per, e = min(words, b + per);
    int local = 0;
    for (int w = b; w < e; ++w) local += __popc(src[w]);
    const int incl = wave_inclusive_scan(local);
    if (lane == kWave - 1) tot[wave] = incl;
    __syncthreads();
    int off = 0, total = 0;
    for (int w = 0; w < nw; ++w) {
        off += (w < wave) ? tot[w] : 0;
        total += tot[w];
    }
    int run = off + incl - local;
    for (int w = b; w < e; ++w) {
        prefix[w] = run;
        run += __popc(src[w]);
    }
    __syncthreads();
    return total;
}

constexpr int kReqThreads = 256;

// One packed weight whose outlier columns the re-quantize launch also
// gathers (mixq_quantize_act_regather): the last `blocks` blocks of the grid
// take that role.  blocks == 0: no weight.  Block b of the role owns packed
// rows b, b + blocks, ... and gather slot k_out[b], as in mixq_pack_weight's
// gather (the same row-to-slot map, so either may serve a later call).
struct GatherArgs {
    const uint16_t* W;     // fp16 [n_out or N, K]
    int64_t N;             // packed rows
    uint16_t* w_out;       // [N, ld_out]
    int32_t* k_out;        // [MIXQ_GATHER_SLOTS]
    int32_t gated;
    const int32_t* rmap;   // row subset, or null
    int64_t n_out;
    int32_t blocks;
};

// packed row n's outlier columns for the channels of set_words (ranks from
// prefix), zeros from `total` up to the padded width
__device__ void gather_row_from_words(const ActArgs& a, const GatherArgs& g, int64_t n,
                                      const uint32_t* set_words, const int32_t* prefix,
                                      int total) {
    const int64_t srow = g.rmap ? (int64_t)g.rmap[n] : src_row(n, g.N, g.gated);
    const bool live = !g.rmap || (srow >= 0 && srow < g.n_out);
    uint16_t* out = g.w_out + n * (int64_t)a.ld_out;
    for (int w = threadIdx.x; w < a.words; w += blockDim.x) {
        uint32_t bits = set_words[w];
        int j = prefix[w];
        while (bits) {
            const int ch = w * 32 + __builtin_ctz(bits);
            out[j++] = live ? g.W[srow * (int64_t)a.K + ch] : (uint16_t)0;
            bits &= bits - 1u;
        }
    }
    const int kpad = (total + MIXQ_OUTLIER_ALIGN - 1) / MIXQ_OUTLIER_ALIGN * MIXQ_OUTLIER_ALIGN;
    for (int j = total + threadIdx.x; j < kpad; j += blockDim.x) out[j] = 0;
}

// the gather role on a call whose set did not change: re-gather only if this
// slot's rows hold another set's columns (first use, or another state)
__device__ void gather_committed(const ActArgs& a, const GatherArgs& g, int b) {
    const int32_t serial = (int32_t)*a.set_id;
    if (g.k_out[b] == serial) return;
    const int count = *a.count;
    const int kpad = (count + MIXQ_OUTLIER_ALIGN - 1) / MIXQ_OUTLIER_ALIGN * MIXQ_OUTLIER_ALIGN;
    for (int64_t n = b; n < g.N; n += g.blocks) {
        const int64_t srow = g.rmap ? (int64_t)g.rmap[n] : src_row(n, g.N, g.gated);
        const bool live = !g.rmap || (srow >= 0 && srow < g.n_out);
        uint16_t* out = g.w_out + n * (int64_t)a.ld_out;
        for (int j = threadIdx.x; j < kpad; j += blockDim.x)
            out[j] = (live && j < count) ? g.W[srow * (int64_t)a.K + a.idx[j]] : (uint16_t)0;
    }
    __syncthreads();
    if (threadIdx.x == 0) g.k_out[b] = serial;
}

template <int CPT, bool NORM>
__global__ __launch_bounds__(kReqThreads) void requant_kernel(ActArgs a, GatherArgs g) {
    const int nreq = gridDim.x - g.blocks;  // blocks of the re-quantize role
    const bool gather_role = (int)blockIdx.x >= nreq;
    if (*a.marker == 0u) {
        // the gate did not fire: the set stands (and flag = 0)
        if (blockIdx.x == 0 && threadIdx.x == 0) *a.flag = 0;
        if (gather_role) gather_committed(a, g, blockIdx.x - nreq);
        return;
    }
    extern __shared__ uint32_t dyn[];
    uint32_t* neww = dyn;                                // [words]
    int32_t* prefix = reinterpret_cast<int32_t*>(dyn + a.words);  // [words]
    __shared__ int tot[kReqThreads / kWave];
    __shared__ int last;
    __shared__ uint4 lut[kLutEntries];
    build_keep_lut(lut);

    // every block forms the grown set itself (the cached set or-ed with the
    // pending detections; every gate block finished before this launch)
    for (int w = threadIdx.x; w < a.words; w += kReqThreads) neww[w] = a.bitmap[w] | a.pending[w];
    __syncthreads();
    const int total = scan_popcounts(neww, a.words, prefix, tot);
    const bool overflow = total > a.k_cap;
    if (!gather_role) {
        if (!overflow) {
            const int wave = threadIdx.x / kWave;
            const int64_t stride = (int64_t)nreq * (kReqThreads / kWave);
            for (int64_t row = (int64_t)blockIdx.x * (kReqThreads / kWave) + wave; row < a.M;
                 row += stride)
                wave_row<CPT, false, NORM>(a, row, neww, prefix, total, lut, nullptr);
        }
    } else {
        const int b = blockIdx.x - nreq;
        if (overflow) {
            // the set is left as it was (capacity): the committed columns
            gather_committed(a, g, b);
        } else {
            for (int64_t n = b; n < g.N; n += g.blocks)
                gather_row_from_words(a, g, n, neww, prefix, total);
            __syncthreads();
            if (threadIdx.x == 0) g.k_out[b] = (int32_t)*a.pend_id;
        }
    }
    // arrival (fired calls only), over both roles: the last block commits,
    // once no block reads the state any more
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        last = atomicAdd(a.arrive, 1u) == gridDim.x - 1;
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    for (int w = threadIdx.x; w < a.words; w += kReqThreads) {
        if (!overflow) {
            uint32_t bits = neww[w];
            int j = prefix[w];
            a.bitmap[w] = bits;
            a.rank[w] = j;
            while (bits) {
                a.idx[j++] = w * 32 + __builtin_ctz(bits);
                bits &= bits - 1u;
            }
        }
        a.pending[w] = 0u;
    }
    if (threadIdx.x == 0) {
        if (!overflow) {
            *a.count = total;
            *a.set_id = *a.pend_id;
        }
        *a.flag = overflow ? MIXQ_FLAG_OVERFLOW : MIXQ_FLAG_FIRED;
        *a.marker = 0u;
        *a.arrive = 0u;
    }
}

constexpr int kGateWaves = 4;  // waves per token in the steady-state pass
static_assert(MIXQ_NORM_K_MAX == kGateWaves * kWave * 16 * 8,
              "the fused RMSNorm keeps a whole token in registers");

template <int CPT_G, int CPT_R, bool NORM, bool RES>
int launch_act(const ActArgs& a, const GatherArgs& g, hipStream_t st) {
    constexpr int kRowsPerBlock = kGateThreads / kWave / kGateWaves;
    int64_t g1 = (a.M + kRowsPerBlock - 1) / kRowsPerBlock;
    // Up to 2048 blocks (all variants fit four blocks per CU: at most 127
    // VGPRs).  At M = 2048 that is one token per block and two rounds of the
    // device: the second round's loads overlap the first round's arithmetic.
    // Measured with alternating builds on one box, per call at M = 2048,
    // K = 8192: the plain pass 18.8-19.1 us against 20.0-20.7 us with 1024
    // blocks of two tokens each; the RMSNorm pass 25.0-25.7 us against
    // 27.0-27.5 us (30.2-30.4 us with 512).  With the residual add the
    // second round's extra streams of D and H cost more than the overlap
    // gains (31.7-32.0 us against 28.9-29.4 us), so it keeps 1024.
    const int64_t cap = RES ? 1024 : 2048;
    const int grid = (int)(g1 < cap ? g1 : cap);
    const size_t lds = (size_t)a.words * 8 + (NORM ? (size_t)a.K * 2 : 0);
    const bool exact = a.nchunks == CPT_G * kWave * kGateWaves;
    const bool one = !RES && g1 <= cap;  // a block per token group
    const dim3 gd(grid), bd(kGateThreads);
    if (exact && one)
        hipLaunchKernelGGL((gate_quant_kernel<CPT_G, kGateWaves, NORM, RES, true, !RES>), gd, bd,
                           lds, st, a);
    else if (exact)
        hipLaunchKernelGGL((gate_quant_kernel<CPT_G, kGateWaves, NORM, RES, true>), gd, bd, lds,
                           st, a);
    else if (one)
        hipLaunchKernelGGL((gate_quant_kernel<CPT_G, kGateWaves, NORM, RES, false, !RES>), gd, bd,
                           lds, st, a);
    else
        hipLaunchKernelGGL((gate_quant_kernel<CPT_G, kGateWaves, NORM, RES, false>), gd, bd, lds,
                           st, a);
    int rc = launch_status();
    if (rc != MIXQ_OK) return rc;
    const int64_t rows_per_block = kReqThreads / kWave;
    int64_t g2 = (a.M + rows_per_block - 1) / rows_per_block;
    if (g2 > 128) g2 = 128;
    // with the residual add, the re-quantize pass reads the finished H
    ActArgs ar = a;
    if (RES) {
        ar.X = a.H;
        ar.ldx = a.ldh;
    }
    hipLaunchKernelGGL((requant_kernel<CPT_R, NORM>), dim3((int)g2 + g.blocks), dim3(kReqThreads),
                       (size_t)a.words * 8, st, ar, g);
    return launch_status();
}

template <int CPT_G, bool NORM, bool RES>
int launch_act_r(const ActArgs& a, const GatherArgs& g, int64_t K, hipStream_t st) {
    // requant: one wave per token, the whole row in registers up to K = 8192
    const int64_t per_lane = (K / 8 + kWave - 1) / kWave;
    if (per_lane <= 1) return launch_act<CPT_G, 1, NORM, RES>(a, g, st);
    if (per_lane <= 2) return launch_act<CPT_G, 2, NORM, RES>(a, g, st);
    if (per_lane <= 4) return launch_act<CPT_G, 4, NORM, RES>(a, g, st);
    if (per_lane <= 8) return launch_act<CPT_G, 8, NORM, RES>(a, g, st);
    return launch_act<CPT_G, 16, NORM, RES>(a, g, st);
}

}  // namespace
}  // namespace mixq

namespace mixq {
namespace {

// Bytes a row-major fp16 matrix spans.
inline uintptr_t span_end(const uint16_t* p, int64_t M, int64_t K, int64_t ld) {
    return reinterpret_cast<uintptr_t>(p) + (uintptr_t)(((M - 1) * ld + K) * 2);
}

inline bool overlaps(const uint16_t* p, const uint16_t* q, int64_t M, int64_t K, int64_t ldp,
                     int64_t ldq) {
    return reinterpret_cast<uintptr_t>(p) < span_end(q, M, K, ldq) &&
           reinterpret_cast<uintptr_t>(q) < span_end(p, M, K, ldp);
}

int act_call(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
             float eps, float* rstd, float threshold, const mixq_act_state* state, int8_t* Xq,
             float* s_x, uint16_t* X_out, void* stream, const uint16_t* D = nullptr,
             int64_t ldd = 0, uint16_t* H = nullptr, int64_t ldh = 0,
             const uint16_t* W = nullptr, const mixq_weight* w = nullptr) {
    if (!X || !state || !Xq || !s_x) return MIXQ_ERR_INVALID_ARG;
    if (!state->idx && state->k_cap > 0) return MIXQ_ERR_INVALID_ARG;
    if (!state->count || !state->flag || !state->bitmap || !state->work)
        return MIXQ_ERR_INVALID_ARG;
    if (M <= 0 || K <= 0 || ldx < K) return MIXQ_ERR_INVALID_ARG;
    if (!(threshold >= 0.0f) || !isfinite(threshold)) return MIXQ_ERR_INVALID_ARG;
    if (state->k_cap < 0 || state->k_cap > K) return MIXQ_ERR_INVALID_ARG;
    if (state->k_cap > 0 && !X_out) return MIXQ_ERR_INVALID_ARG;
    const bool norm = gamma != nullptr;
    const bool res = D != nullptr;
    if (norm && (!rstd || !(eps >= 0.0f) || !isfinite(eps))) return MIXQ_ERR_INVALID_ARG;
    if (res && (!norm || !H || ldd < K || ldh < K)) return MIXQ_ERR_INVALID_ARG;
    // H is written while X (R) and D are still read, by other waves
    if (res && M > 0 && K > 0 && ldx >= K &&
        (overlaps(H, X, M, K, ldh, ldx) || overlaps(H, D, M, K, ldh, ldd)))
        return MIXQ_ERR_INVALID_ARG;
    if (!valid_k(K)) return MIXQ_ERR_UNSUPPORTED_SHAPE;
    if (ldx % 8 != 0 || ((uintptr_t)X & 15u) != 0 || ((uintptr_t)Xq & 15u) != 0)
        return MIXQ_ERR_UNSUPPORTED_SHAPE;
    if (norm && (K > MIXQ_NORM_K_MAX || ((uintptr_t)gamma & 15u) != 0))
        return MIXQ_ERR_UNSUPPORTED_SHAPE;
    if (res && (ldd % 8 != 0 || ldh % 8 != 0 || ((uintptr_t)D & 15u) != 0 ||
                ((uintptr_t)H & 15u) != 0))
        return MIXQ_ERR_UNSUPPORTED_SHAPE;
    if (M > (int64_t)1 << 31) return MIXQ_ERR_UNSUPPORTED_SHAPE;
    // a weight whose outlier columns the same launches re-gather: the checks
    // of mixq_pack_weight's OUTLIER_COLS mode
    GatherArgs g{};
    if (w) {
        if (!W || w->K != K || w->k_cap != state->k_cap || !w->k_out || !state->work ||
            (state->k_cap > 0 && (!w->w_out || !state->idx)) || w->N <= 0 ||
            (w->bits != 8 && w->bits != 4) || (w->gated != 0 && w->gated != 1) ||
            (w->rmap && (w->gated || w->n_out < 1)))
            return MIXQ_ERR_INVALID_ARG;
        if (w->N > (int64_t)1 << 31 || ((uintptr_t)W & 15u) != 0) return MIXQ_ERR_UNSUPPORTED_SHAPE;
        g.W = W;
        g.N = w->N;
        g.w_out = w->w_out;
        g.k_out = w->k_out;
        g.gated = w->gated;
        g.rmap = w->rmap;
        g.n_out = w->n_out;
        g.blocks = (int32_t)(w->N < MIXQ_GATHER_SLOTS ? w->N : MIXQ_GATHER_SLOTS);
        if (state->k_cap == 0) g.blocks = 0;  // no outlier columns to hold
    }
    int rc = check_device_cached();
    if (rc != MIXQ_OK) return rc;

    ActArgs a;
    const int32_t words = (int32_t)bitmap_words(K);
    a.X = X;
    a.M = M;
    a.K = (int32_t)K;
    a.ldx = ldx;
    a.tau = threshold;
    a.tau_bits = half_floor_bits(threshold);
    a.idx = state->idx;
    a.count = state->count;
    a.flag = state->flag;
    a.bitmap = state->bitmap;
    a.pending = state->work;
    a.rank = reinterpret_cast<int32_t*>(state->work + words);
    a.marker = state->work + 2 * words;
    a.arrive = state->work + 2 * words + 1;
    a.set_id = state->work + 2 * words + 2;
    a.pend_id = state->work + 2 * words + 3;
    a.k_cap = state->k_cap;
    a.words = words;
    a.nchunks = (int32_t)(K / 8);
    a.Xq = Xq;
    a.s_x = s_x;
    a.X_out = state->k_cap > 0 ? X_out : nullptr;
    a.ld_out = (int32_t)outlier_ld(state->k_cap);
    a.gamma = gamma;
    a.eps = eps;
    a.rstd = rstd;
    a.D = D;
    a.ldd = ldd;
    a.H = H;
    a.ldh = ldh;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // steady-state pass: chunks per lane and segment, the whole row in
    // registers of its kGateWaves waves up to K = 32768
    const int64_t per_lane = (K / 8 + kWave * kGateWaves - 1) / (kWave * kGateWaves);
    if (res) {
        if (per_lane <= 1) return launch_act_r<1, true, true>(a, g, K, st);
        if (per_lane <= 2) return launch_act_r<2, true, true>(a, g, K, st);
        if (per_lane <= 4) return launch_act_r<4, true, true>(a, g, K, st);
        if (per_lane <= 8) return launch_act_r<8, true, true>(a, g, K, st);
        return launch_act_r<16, true, true>(a, g, K, st);
    }
    if (norm) {
        if (per_lane <= 1) return launch_act_r<1, true, false>(a, g, K, st);
        if (per_lane <= 2) return launch_act_r<2, true, false>(a, g, K, st);
        if (per_lane <= 4) return launch_act_r<4, true, false>(a, g, K, st);
        if (per_lane <= 8) return launch_act_r<8, true, false>(a, g, K, st);
        return launch_act_r<16, true, false>(a, g, K, st);
    }
    if (per_lane <= 1) return launch_act_r<1, false, false>(a, g, K, st);
    if (per_lane <= 2) return launch_act_r<2, false, false>(a, g, K, st);
    if (per_lane <= 4) return launch_act_r<4, false, false>(a, g, K, st);
    if (per_lane <= 8) return launch_act_r<8, false, false>(a, g, K, st);
    return launch_act_r<16, false, false>(a, g, K, st);
}

}  // namespace
}  // namespace mixq

extern "C" int mixq_quantize_act(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                 float threshold, const mixq_act_state* state, int8_t* Xq,
                                 float* s_x, uint16_t* X_out, void* stream) {
    return mixq::act_call(X, M, K, ldx, nullptr, 0.0f, nullptr, threshold, state, Xq, s_x, X_out,
                          stream);
}

extern "C" int mixq_quantize_act_regather(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                          float threshold, const mixq_act_state* state,
                                          int8_t* Xq, float* s_x, uint16_t* X_out,
                                          const uint16_t* W, const mixq_weight* w, void* stream) {
    if (!W || !w) return MIXQ_ERR_INVALID_ARG;
    return mixq::act_call(X, M, K, ldx, nullptr, 0.0f, nullptr, threshold, state, Xq, s_x, X_out,
                          stream, nullptr, 0, nullptr, 0, W, w);
}

extern "C" int mixq_rmsnorm_quantize_act(const uint16_t* H, int64_t M, int64_t K, int64_t ldh,
                                         const uint16_t* gamma, float eps, float threshold,
                                         const mixq_act_state* state, int8_t* Xq, float* s_x,
                                         uint16_t* X_out, float* rstd, void* stream) {
    if (!gamma) return MIXQ_ERR_INVALID_ARG;
    return mixq::act_call(H, M, K, ldh, gamma, eps, rstd, threshold, state, Xq, s_x, X_out,
                          stream);
}

extern "C" int mixq_add_rmsnorm_quantize_act(const uint16_t* R, int64_t ldr, const uint16_t* D,
                                             int64_t ldd, uint16_t* H, int64_t ldh, int64_t M,
                                             int64_t K, const uint16_t* gamma, float eps,
                                             float threshold, const mixq_act_state* state,
                                             int8_t* Xq, float* s_x, uint16_t* X_out, float* rstd,
                                             void* stream) {
    if (!gamma || !D || !H) return MIXQ_ERR_INVALID_ARG;
    return mixq::act_call(R, M, K, ldr, gamma, eps, rstd, threshold, state, Xq, s_x, X_out,
                          stream, D, ldd, H, ldh);
}
