// Weight side of the mixed-precision linear layer: per-output-channel
// symmetric INT8 / INT4 quantization and the FP16 outlier columns.
//
// FP6 explainer, section 3: each output channel's scale is its max |w| over
// the code range, a zero scale becomes 1, values round to nearest; weights
// are quantized once, when the layer is loaded.
// MixQ article, section "MixQ的解决方案", Fig. 11: the outlier channels are
// concatenated in order into a separate FP16 matrix -- here the weight's
// columns at those channels, w_out[n, j] = W[n, idx[j]].
// QServe notes, "寄存器压力和并行性" / "小结": INT4 weights are decoded to INT8
// inside the GEMM; the nibble layout below lets one 32-bit word expand into
// eight INT8 codes with a few bitwise operations.
#include "mixq_internal.h"

#pragma clang fp contract(off)

namespace mixq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;


// PROG: progressive INT4 (QServe page, progressive group quantization):
// first level to INT8 with the range 119, then per group of 128 channels (16
// chunks = 16 consecutive lanes) a 4-bit value, an integer scale and a zero;
// integer steps with IEEE binary32 divisions whose ties are exact.
// Byte offset of 4-bit chunk c (8 consecutive k, 4 bytes) of packed row n:
// K-tile-major inside 32-row blocks, [N/32][K/64][32 rows][32 bytes].
__device__ __forceinline__ int64_t int4_offset(int64_t n, int c, int K) {
    return ((n / 32) * (K / 64) + c / 8) * 1024 + (n % 32) * 32 + (c % 8) * 4;
}

template <int CPT, int BITS, bool PROG = false>
__global__ __launch_bounds__(kThreads) void quantize_weight_kernel(const uint16_t* __restrict__ W,
                                                                    int64_t N, int32_t K,
                                                                    void* __restrict__ wq,
                                                                    float* __restrict__ s_w,
                                                                    int gated,
                                                                    uint16_t* __restrict__ gsz,
                                                                    const int32_t* __restrict__ rmap,
                                                                    int64_t n_out) {
    static_assert(!PROG || BITS == 4, "progressive groups hold 4-bit values");
    __shared__ float red[kWaves];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nchunks = K / 8;
    constexpr float kQ = BITS == 8 ? 127.0f : PROG ? 119.0f : 7.0f;
    const int ngroups = K / MIXQ_PROGRESSIVE_GROUP;
    for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
        // the packed row's W row (a row subset: rmap[n]), the same for the
        // whole block; an entry outside W packs zeros
        int64_t srow = src_row(n, N, gated);
        if (rmap) {
            srow = rmap[n];
            if (srow < 0 || srow >= n_out) {
                uint8_t* const w8 = static_cast<uint8_t*>(wq);
                for (int c = tid; c < nchunks; c += kThreads) {
                    if (BITS == 8)
                        *reinterpret_cast<uint2*>(w8 + n * (int64_t)K + (int64_t)c * 8) =
                            make_uint2(0u, 0u);
                    else
                        *reinterpret_cast<uint32_t*>(w8 + int4_offset(n, c, K)) = 0u;
                }
                if constexpr (PROG)
                    for (int g = tid; g < ngroups; g += kThreads)
                        gsz[g * N + n] = (uint16_t)1;  // s2 1, z 0
                if (tid == 0) s_w[n] = 1.0f;
                continue;
            }
        }
        const uint16_t* wr = W + srow * (int64_t)K;
        uint4 v[CPT];
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * kThreads;
            v[i] = c < nchunks ? *reinterpret_cast<const uint4*>(wr + (int64_t)c * 8)
                               : make_uint4(0, 0, 0, 0);
            const uint32_t u[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                am = fmaxf(am, fabsf(half_bits_to_float((uint16_t)(u[e >> 1] >> ((e & 1) * 16)))));
        }
        am = wave_max(am);
        if (lane == 0) red[wave] = am;
        __syncthreads();
        float g = red[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) g = fmaxf(g, red[w]);
        __syncthreads();

        float s, rho;
        if (g == 0.0f) {
            s = 1.0f;
            rho = 1.0f;
        } else {
            s = g / kQ;
            rho = kQ / g;
        }
        if (tid == 0) s_w[n] = s;

#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * kThreads;
            if (c >= nchunks) continue;
            const uint32_t u[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            int q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float y = __builtin_rintf(
                    half_bits_to_float((uint16_t)(u[e >> 1] >> ((e & 1) * 16))) * rho);
                y = fminf(fmaxf(y, -kQ), kQ);
                q[e] = (int)y;
            }
            if constexpr (PROG) {
                // a group of 128 channels is 16 chunks, held by 16 consecutive lanes
                int mn = 0, mx = 0;  // zero kept in the range: z is a 4-bit value
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    mn = min(mn, q[e]);
                    mx = max(mx, q[e]);
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    mn = min(mn, __shfl_xor(mn, o, 16));
                    mx = max(mx, __shfl_xor(mx, o, 16));
                }
                const int s2 = max(1, (mx - mn + 14) / 15);  // ceil((mx - mn) / 15)
                const float fs2 = (float)s2;
                // |value| <= 238 and s2 <= 16: a quotient that is a tie is exact
                // in binary32, so rounding the binary32 quotient rounds the
                // exact one (half to even)
                const int z = (int)__builtin_rintf((float)(-mn) / fs2);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    q[e] = min(max((int)__builtin_rintf((float)q[e] / fs2) + z, 0), 15);
                if ((tid & 15) == 0)
                    gsz[(c / 16) * N + n] = (uint16_t)(s2 | (z << 8));
            }
            if (BITS == 8) {
                uint32_t p0 = 0, p1 = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p0 |= ((uint32_t)q[e] & 0xFFu) << (8 * e);
                    p1 |= ((uint32_t)q[e + 4] & 0xFFu) << (8 * e);
                }
                int8_t* dst = static_cast<int8_t*>(wq) + n * (int64_t)K + (int64_t)c * 8;
                *reinterpret_cast<uint2*>(dst) = make_uint2(p0, p1);
            } else {
                // one word per 8 consecutive k: byte j = q[j] | q[j+4] << 4
                uint32_t word = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    word |= (((uint32_t)q[j] & 0xFu) | (((uint32_t)q[j + 4] & 0xFu) << 4)) << (8 * j);
                *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(wq) + int4_offset(n, c, K)) =
                    word;
            }
        }
    }
}

// w_out[n, j] = W[n, idx[j]] for j < count, zeros up to the padded width.
// Block b owns rows b, b + G, b + 2G, ... (G = gridDim.x, fixed for a given N)
// and slot k_out[b], the serial of the set its rows were last gathered for
// (the state's work area holds the serial of its committed set, unique per
// commit): it runs when forced or when that differs from the state's serial.
// No block reads another block's slot, so the check needs no atomics.
__global__ __launch_bounds__(kThreads) void gather_cols_kernel(const uint16_t* __restrict__ W,
                                                               int64_t N, int32_t K,
                                                               const int32_t* __restrict__ idx,
                                                               const int32_t* __restrict__ count_p,
                                                               const uint32_t* __restrict__ set_id_p,
                                                               uint16_t* __restrict__ w_out,
                                                               int32_t ld_out, int32_t* k_out,
                                                               int force, int gated,
                                                               const int32_t* __restrict__ rmap,
                                                               int64_t n_out) {
    const int count = *count_p;
    const int32_t set_id = (int32_t)*set_id_p;
    if (!force && k_out[blockIdx.x] == set_id) return;
    const int kpad = (count + MIXQ_OUTLIER_ALIGN - 1) / MIXQ_OUTLIER_ALIGN * MIXQ_OUTLIER_ALIGN;
    const int64_t G = gridDim.x;
    const int64_t my_rows = (N - blockIdx.x + G - 1) / G;
    const int64_t total = my_rows * kpad;
    for (int64_t t = threadIdx.x; t < total; t += kThreads) {
        const int64_t n = blockIdx.x + (t / kpad) * G;
        const int j = (int)(t % kpad);
        // a row subset takes W row rmap[n]; an entry outside W gets zeros
        const int64_t srow = rmap ? (int64_t)rmap[n] : src_row(n, N, gated);
        const bool live = !rmap || (srow >= 0 && srow < n_out);
        w_out[n * ld_out + j] = (live && j < count) ? W[srow * (int64_t)K + idx[j]] : (uint16_t)0;
    }
    __syncthreads();
    if (threadIdx.x == 0) k_out[blockIdx.x] = set_id;
}

template <int CPT>
int launch_quant(const uint16_t* W, int64_t N, int32_t K, int bits, const mixq_weight* w,
                 hipStream_t st) {
    const int grid = (int)(N < 4096 ? N : 4096);
    if (bits == 8)
        hipLaunchKernelGGL((quantize_weight_kernel<CPT, 8>), dim3(grid), dim3(kThreads), 0, st, W,
                           N, K, w->wq, w->s_w, w->gated, nullptr, w->rmap,
                           (int64_t)w->n_out);
    else if (w->group)
        hipLaunchKernelGGL((quantize_weight_kernel<CPT, 4, true>), dim3(grid), dim3(kThreads), 0,
                           st, W, N, K, w->wq, w->s_w, w->gated, w->gsz, w->rmap,
                           (int64_t)w->n_out);
    else
        hipLaunchKernelGGL((quantize_weight_kernel<CPT, 4>), dim3(grid), dim3(kThreads), 0, st, W,
                           N, K, w->wq, w->s_w, w->gated, nullptr, w->rmap,
                           (int64_t)w->n_out);
    return launch_status();
}

}  // namespace
}  // namespace mixq

extern "C" int mixq_pack_weight(const uint16_t* W, int64_t N, int64_t K, int32_t bits,
                                const mixq_act_state* state, int32_t mode, const mixq_weight* w,
                                void* stream) {
    using namespace mixq;
    if (!W || !state || !w) return MIXQ_ERR_INVALID_ARG;
    if (N <= 0 || K <= 0) return MIXQ_ERR_INVALID_ARG;
    if (bits != 8 && bits != 4) return MIXQ_ERR_INVALID_ARG;
    if (mode != MIXQ_PACK_FULL && mode != MIXQ_PACK_OUTLIER_COLS) return MIXQ_ERR_INVALID_ARG;
    if (w->N != N || w->K != K || w->bits != bits || w->k_cap != state->k_cap)
        return MIXQ_ERR_INVALID_ARG;
    if (!w->wq || !w->s_w || !w->k_out) return MIXQ_ERR_INVALID_ARG;
    if (state->k_cap < 0 || state->k_cap > K) return MIXQ_ERR_INVALID_ARG;
    if (state->k_cap > 0 && (!w->w_out || !state->idx)) return MIXQ_ERR_INVALID_ARG;
    if (!state->count || !state->work) return MIXQ_ERR_INVALID_ARG;
    if (w->gated != 0 && w->gated != 1) return MIXQ_ERR_INVALID_ARG;
    if (w->group != 0 && (w->group != MIXQ_PROGRESSIVE_GROUP || bits != 4 || !w->gsz))
        return MIXQ_ERR_INVALID_ARG;
    // row subsets: INT8 or progressive INT4 rows
    if (w->rmap && (w->gated || w->n_out < 1 || (bits == 4 && w->group == 0)))
        return MIXQ_ERR_INVALID_ARG;
    if (!valid_k(K)) return MIXQ_ERR_UNSUPPORTED_SHAPE;
    if (w->gated && N % 64 != 0) return MIXQ_ERR_UNSUPPORTED_SHAPE;
    if (w->group && K % MIXQ_PROGRESSIVE_GROUP != 0) return MIXQ_ERR_UNSUPPORTED_SHAPE;
    if (((uintptr_t)W & 15u) != 0 || ((uintptr_t)w->wq & 15u) != 0)
        return MIXQ_ERR_UNSUPPORTED_SHAPE;
    if (N > (int64_t)1 << 31) return MIXQ_ERR_UNSUPPORTED_SHAPE;
    int rc = check_device_cached();
    if (rc != MIXQ_OK) return rc;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (mode == MIXQ_PACK_FULL) {
        const int64_t cpt = (K / 8 + kThreads - 1) / kThreads;
        if (cpt <= 1) rc = launch_quant<1>(W, N, (int32_t)K, bits, w, st);
        else if (cpt <= 2) rc = launch_quant<2>(W, N, (int32_t)K, bits, w, st);
        else if (cpt <= 4) rc = launch_quant<4>(W, N, (int32_t)K, bits, w, st);
        else if (cpt <= 8) rc = launch_quant<8>(W, N, (int32_t)K, bits, w, st);
        else if (cpt <= 16) rc = launch_quant<16>(W, N, (int32_t)K, bits, w, st);
        else rc = launch_quant<32>(W, N, (int32_t)K, bits, w, st);
        if (rc != MIXQ_OK) return rc;
    }
    const int ld_out = (int)outlier_ld(state->k_cap);
    const int grid = (int)(N < MIXQ_GATHER_SLOTS ? N : MIXQ_GATHER_SLOTS);
    hipLaunchKernelGGL(gather_cols_kernel, dim3(grid), dim3(kThreads), 0, st, W, N, (int32_t)K,
                       state->idx, state->count, state->work + 2 * bitmap_words(K) + 2,
                       w->w_out, ld_out, w->k_out,
                       mode == MIXQ_PACK_FULL ? 1 : 0, w->gated, w->rmap,
                       (int64_t)w->n_out);
    return launch_status();
}
