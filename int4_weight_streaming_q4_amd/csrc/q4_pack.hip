// Packing of 4-bit codes: two codes per byte, even column in the low nibble.
// Pure byte work, bit-exact.  Each thread handles 16 output bytes with a
// scalar tail, so any N x K (K even) works without alignment requirements.
#include "q4_internal.h"

namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
pack_kernel(const uint8_t *__restrict__ codes, uint8_t *__restrict__ packed,
            int64_t nbytes) {
    int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 16;
    if (i0 >= nbytes)
        return;
    int64_t n = nbytes - i0 < 16 ? nbytes - i0 : 16;
    for (int64_t j = 0; j < n; ++j) {
        uint8_t lo = codes[2 * (i0 + j)] & 0x0F;
        uint8_t hi = codes[2 * (i0 + j) + 1] & 0x0F;
        packed[i0 + j] = (uint8_t)(lo | (hi << 4));
    }
}

__global__ void __launch_bounds__(kThreads)
unpack_kernel(const uint8_t *__restrict__ packed, uint8_t *__restrict__ codes,
              int64_t nbytes) {
    int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 16;
    if (i0 >= nbytes)
        return;
    int64_t n = nbytes - i0 < 16 ? nbytes - i0 : 16;
    for (int64_t j = 0; j < n; ++j) {
        uint8_t b = packed[i0 + j];
        codes[2 * (i0 + j)] = b & 0x0F;
        codes[2 * (i0 + j) + 1] = b >> 4;
    }
}

q4_status check_pack_args(const void *a, const void *b, int64_t N, int64_t K,
                          const char *what) {
    if (!a || !b)
        return q4::fail(Q4_ERR_INVALID_ARG, "%s: null pointer", what);
    if (N < 1 || K < 2 || K % 2 != 0)
        return q4::fail(Q4_ERR_INVALID_ARG, "%s: need N >= 1 and even K >= 2 (N=%lld K=%lld)",
                        what, (long long)N, (long long)K);
    if (N > ((int64_t)1 << 40) || K > ((int64_t)1 << 40) / N)
        return q4::fail(Q4_ERR_INVALID_ARG, "%s: N*K too large", what);
    return Q4_OK;
}

} // namespace

extern "C" q4_status q4_pack(const uint8_t *codes, uint8_t *packed, int64_t N,
                             int64_t K, hipStream_t stream) {
    Q4_CHECK(check_pack_args(codes, packed, N, K, "q4_pack"));
    int64_t nbytes = N * K / 2;
    int64_t blocks = (nbytes + 16 * kThreads - 1) / (16 * kThreads);
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       codes, packed, nbytes);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

extern "C" q4_status q4_unpack(const uint8_t *packed, uint8_t *codes, int64_t N,
                               int64_t K, hipStream_t stream) {
    Q4_CHECK(check_pack_args(packed, codes, N, K, "q4_unpack"));
    int64_t nbytes = N * K / 2;
    int64_t blocks = (nbytes + 16 * kThreads - 1) / (16 * kThreads);
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       packed, codes, nbytes);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}
