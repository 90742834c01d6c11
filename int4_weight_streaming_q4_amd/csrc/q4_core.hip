// Status handling, argument checks and device queries of libq4stream.
#include <cstdarg>
#include <mutex>
#include <vector>

#include "q4_internal.h"

namespace q4 {

static thread_local std::string g_last_error;

q4_status fail(q4_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

q4_status ok() { return Q4_OK; }

q4_status check_matrix(const void *packed, const void *scales, int64_t N,
                       int64_t K, const char *what) {
    if (!packed || !scales)
        return fail(Q4_ERR_INVALID_ARG, "%s: null weight or scale pointer", what);
    if (N < 1 || N > INT32_MAX)
        return fail(Q4_ERR_INVALID_ARG, "%s: N=%lld outside [1, 2^31-1]", what,
                    (long long)N);
    if (K < 32 || K % 32 != 0)
        return fail(Q4_ERR_INVALID_ARG, "%s: K=%lld must be a positive multiple of 32",
                    what, (long long)K);
    if (K > Q4_MAX_K)
        return fail(Q4_ERR_UNSUPPORTED, "%s: K=%lld above the supported maximum %d",
                    what, (long long)K, Q4_MAX_K);
    if (!aligned(packed, 16))
        return fail(Q4_ERR_INVALID_ARG, "%s: packed weights not 16-byte aligned", what);
    if (!aligned(scales, 2))
        return fail(Q4_ERR_INVALID_ARG, "%s: scales not 2-byte aligned", what);
    return Q4_OK;
}

int device_cus() {
    // fixed table per device index (no heap allocation on the launch path)
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int cache[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 256;
    if (dev < 0 || dev >= kMaxDevices) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess ||
            cus <= 0)
            cus = 256;
        return cus;
    }
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess ||
            cus <= 0)
            cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

} // namespace q4

extern "C" const char *q4_last_error(void) { return q4::g_last_error.c_str(); }

extern "C" int32_t q4_abi_version(void) { return Q4_ABI_VERSION; }
