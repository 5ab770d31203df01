// Matrix-core rate probe: the INT8 MFMA stream of the GEMM's main loop with
// no memory traffic, run on a workload's own operand bytes.
//
// The MixQ article (section "MixQ的解决方案", Fig. 14) reports its kernels as
// throughput against the hardware's peak.  On gfx950 the published INT8 peak
// assumes the 2.4 GHz engine clock, but the board lowers the clock under
// sustained matrix work, by how much depending on the operand bits that
// toggle.  This kernel measures what the matrix cores deliver at the clock
// the board then sustains, for the same operand bytes, so that the GEMM's
// rate can be set against a ceiling that its memory traffic does not enter.
//
// Shape of the work, per wave, as in the GEMM's 256 x 256 tile: a 128 x 128
// sub-tile as 4 x 4 fragments of 32 x 32 (v_mfma_i32_32x32x32_i8), 256 int32
// accumulators per lane, 32 MFMAs per 64 bytes of K.  Each wave loads eight
// 16-byte A operands and eight B operands per lane once (its own 8 KiB of
// each source, wrapping), then runs `iters` rounds of the 32 MFMAs, every
// MFMA on a different operand pair in the GEMM's order.  One wave per SIMD,
// four per block, as in the GEMM.
#include "mixq_internal.h"

namespace mixq {
namespace {

typedef int p4i __attribute__((ext_vector_type(4)));
typedef int p16i __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_probe_kernel(const int8_t* a, const int8_t* b, int64_t a_bytes, int64_t b_bytes,
                       int32_t iters, int32_t* out, int64_t* clk) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * (kProbeThreads / kWave) + threadIdx.x / kWave;
    // operand q of this lane: bytes [((gw * 8 + q) * 1024 + 16 * lane) mod size, +16)
    p4i af[2][4], bf[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t q = gw * 8 + ks * 4 + i;
            af[ks][i] = *reinterpret_cast<const p4i*>(a + (q * 1024 + 16 * lane) % a_bytes);
            bf[ks][i] = *reinterpret_cast<const p4i*>(b + (q * 1024 + 16 * lane) % b_bytes);
        }
    p16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = p16i{};
    const int64_t t0 = (int64_t)__builtin_amdgcn_s_memtime();
    const int64_t r0 = (int64_t)__builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[ks][i], bf[ks][j],
                                                                      acc[i][j], 0, 0, 0);
    }
    const int64_t t1 = (int64_t)__builtin_amdgcn_s_memtime();
    const int64_t r1 = (int64_t)__builtin_amdgcn_s_memrealtime();
    // one checksum per lane: the sum of its 256 accumulators (wrapping)
    uint32_t s = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += (uint32_t)acc[i][j][e];
    out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = (int32_t)s;
    if (clk && threadIdx.x == 0) {
        int64_t* c = clk + 4 * (int64_t)blockIdx.x;
        c[0] = t0;
        c[1] = t1;
        c[2] = r0;
        c[3] = r1;
    }
}

}  // namespace
}  // namespace mixq

extern "C" int mixq_mfma_probe(const int8_t* a, int64_t a_bytes, const int8_t* b,
                               int64_t b_bytes, int32_t iters, int32_t blocks, int32_t* out,
                               int64_t* clk, void* stream) {
    if (!a || !b || !out || iters < 1 || blocks < 1) return MIXQ_ERR_INVALID_ARG;
    if (a_bytes < 16 || b_bytes < 16 || a_bytes % 16 || b_bytes % 16) return MIXQ_ERR_INVALID_ARG;
    if (((uintptr_t)a & 15u) || ((uintptr_t)b & 15u)) return MIXQ_ERR_INVALID_ARG;
    int rc = mixq::check_device_cached();
    if (rc != MIXQ_OK) return rc;
    hipLaunchKernelGGL(mixq::mfma_probe_kernel, dim3(blocks), dim3(mixq::kProbeThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), a, b, a_bytes, b_bytes, iters, out,
                       clk);
    return mixq::launch_status();
}
