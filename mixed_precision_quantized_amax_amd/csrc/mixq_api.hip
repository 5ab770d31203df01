// Host-side entry points of the mixq library that launch nothing: status
// strings, size helpers and the device check (FP6 explainer, section 3:
// an explicit error on hardware the kernels were not built for).
#include <string.h>

#include <mutex>

#include "mixq_internal.h"

namespace mixq {

int check_device_cached() {
    // One answer per device ordinal, computed on first use.
    static std::mutex mu;
    static int cache[64];
    static bool init = false;
    int dev = 0;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return MIXQ_ERR_NO_DEVICE;
    }
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return MIXQ_ERR_NO_DEVICE;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!init) {
        for (int i = 0; i < 64; ++i) cache[i] = -1;
        init = true;
    }
    if (cache[dev] < 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
            (void)hipGetLastError();
            return MIXQ_ERR_NO_DEVICE;
        }
        cache[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? MIXQ_OK
                                                               : MIXQ_ERR_UNSUPPORTED_DEVICE;
    }
    return cache[dev];
}

int device_cu_count() {
    static std::mutex mu;
    static int cache[64];
    static bool init = false;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 0;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!init) {
        for (int i = 0; i < 64; ++i) cache[i] = -1;
        init = true;
    }
    if (cache[dev] < 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            n = 0;
        }
        cache[dev] = n;
    }
    return cache[dev];
}

}  // namespace mixq

extern "C" {

size_t mixq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t bits) {
    using namespace mixq;
    // the plan of the current device (256 compute units on a whole MI355X;
    // fewer on a partition), or 256 when no gfx950 device is current
    const int cus = check_device_cached() == MIXQ_OK && device_cu_count() > 0 ? device_cu_count()
                                                                               : 256;
    const int S = split_plan(M, N, K, bits, cus);
    if (S > 1) return (size_t)split_workspace_bytes(M, N, S);
    int St = 1;
    const int n_split = tail_plan(M, N, K, cus, &St);
    if (n_split > 0 && St > 1) return (size_t)tail_workspace_bytes(M, N, n_split, St);
    return 0;
}


int64_t mixq_outlier_ld(int32_t k_cap) { return k_cap <= 0 ? 0 : mixq::outlier_ld(k_cap); }

int64_t mixq_bitmap_words(int64_t K) { return K <= 0 ? 0 : mixq::bitmap_words(K); }

int64_t mixq_state_work_words(int64_t K) { return K <= 0 ? 0 : 2 * mixq::bitmap_words(K) + 4; }

size_t mixq_packed_weight_bytes(int64_t N, int64_t K, int32_t bits) {
    if (N <= 0 || K <= 0 || K % 2) return 0;
    if (bits == 8) return (size_t)N * (size_t)K;
    if (bits == 4) return (size_t)((N + 31) / 32 * 32) * (size_t)(K / 2);  // whole 32-row blocks
    return 0;
}

const char* mixq_status_string(int status) {
    switch (status) {
        case MIXQ_OK: return "ok";
        case MIXQ_ERR_INVALID_ARG: return "invalid argument";
        case MIXQ_ERR_UNSUPPORTED_SHAPE:
            return "unsupported shape (K must be a positive multiple of 64 up to 65536; "
                   "buffers 16-byte aligned; byte offsets within a tile below 2^31)";
        case MIXQ_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
        case MIXQ_ERR_NO_DEVICE: return "no HIP device";
        case MIXQ_ERR_HIP: return "HIP launch error";
        case MIXQ_ERR_WORKSPACE: return "workspace too small for the split this product takes";
        default: return "unknown status";
    }
}

int mixq_check_device(void) { return mixq::check_device_cached(); }

int mixq_version(void) { return 100; }

}  // extern "C"
