// Glue of the batched decode step that verifies a speculative draft: B
// token columns go through every layer together, each product as one
// small-batch INT4 product (every unpacked weight used B times) and the
// glue between them per column.
//
// PipeInfer (repository page, "Run" and "Tuning PipeInfer"): speculative
// micro-batches of a few draft tokens (kept under 8) are verified by the
// target model; PIPO: Pipelined Offloading for Efficient Inference on
// Consumer Devices, "Method", "Automatic configuration": its 4-bit kernel
// serves batches below 16.  The glue is the same one-token glue as the
// single-token step (RMSNorm to binary16, the V of each query head's group,
// SiLU gate); a causal batch gives every column exactly the result of
// decoding its token alone.
#include <cmath>

#include "q4_verify.h"

namespace q4 {
namespace {

constexpr int kVThreads = 256;

__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// One workgroup per column.
__global__ void __launch_bounds__(kVThreads)
rmsnorm_batch_kernel(const float *__restrict__ H, uint16_t *__restrict__ X, int32_t d,
                     float eps) {
    __shared__ float part[kVThreads / 64];
    const float *h = H + (size_t)blockIdx.x * d;
    uint16_t *x = X + (size_t)blockIdx.x * d;
    float ss = 0.0f;
    for (int i = threadIdx.x; i < d; i += kVThreads)
        ss = fmaf(h[i], h[i], ss);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        ss += __shfl_xor(ss, o);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = part[0];
#pragma unroll
    for (int w = 1; w < kVThreads / 64; ++w)
        tot += part[w];
    const float r = 1.0f / sqrtf(tot / (float)d + eps);
    for (int i = threadIdx.x; i < d; i += kVThreads)
        x[i] = f2h(h[i] * r);
}

__global__ void __launch_bounds__(kVThreads)
gather_batch_kernel(const float *__restrict__ qkv, uint16_t *__restrict__ o, int32_t H,
                    int32_t Hkv, int32_t hd) {
    const int b = blockIdx.y;
    const int j = blockIdx.x * kVThreads + threadIdx.x;
    if (j >= H * hd)
        return;
    const int nqkv = (H + 2 * Hkv) * hd;
    const int g = (j / hd) / (H / Hkv);
    o[(size_t)b * H * hd + j] = f2h(qkv[(size_t)b * nqkv + (H + Hkv) * hd + g * hd + j % hd]);
}

__global__ void __launch_bounds__(kVThreads)
silu_batch_kernel(const float *__restrict__ gu, uint16_t *__restrict__ m, int32_t dff) {
    const int b = blockIdx.y;
    const int j = blockIdx.x * kVThreads + threadIdx.x;
    if (j >= dff)
        return;
    const float g = gu[(size_t)b * 2 * dff + j];
    const float u = gu[(size_t)b * 2 * dff + dff + j];
    const float silu = g / (1.0f + expf(-g));
    m[(size_t)b * dff + j] = f2h(silu * u);
}

} // namespace

q4_status launch_rmsnorm_batch(const float *H, uint16_t *X, int32_t B, int32_t d, float eps,
                               hipStream_t s) {
    hipLaunchKernelGGL(rmsnorm_batch_kernel, dim3((unsigned)B), dim3(kVThreads), 0, s, H, X, d,
                       eps);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

q4_status launch_gather_batch(const float *qkv, uint16_t *o, int32_t B, int32_t H,
                              int32_t Hkv, int32_t hd, hipStream_t s) {
    const unsigned gx = (unsigned)((H * hd + kVThreads - 1) / kVThreads);
    hipLaunchKernelGGL(gather_batch_kernel, dim3(gx, (unsigned)B), dim3(kVThreads), 0, s, qkv,
                       o, H, Hkv, hd);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

q4_status launch_silu_batch(const float *gu, uint16_t *m, int32_t B, int32_t dff,
                            hipStream_t s) {
    const unsigned gx = (unsigned)((dff + kVThreads - 1) / kVThreads);
    hipLaunchKernelGGL(silu_batch_kernel, dim3(gx, (unsigned)B), dim3(kVThreads), 0, s, gu, m,
                       dff);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace q4
