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
// single-token step (RMSNorm to binary16, the V of each query head's group;
// the SiLU gate runs in the gate+up product's epilogue); a causal batch
// gives every column exactly the result of decoding its token alone.
#include <cmath>

#include "q4_verify.h"
#include "q4_lanes.h"

namespace q4 {
namespace {

constexpr int kVThreads = 256;

__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// One workgroup per column; the column stays in registers between the sum
// of squares and the scaling (d <= 8192; a larger d rereads the rest).
constexpr int kNThreads = 512;
constexpr int kNKeep = 4; // float4 per thread held in registers

__global__ void __launch_bounds__(kNThreads)
rmsnorm_batch_kernel(const float *__restrict__ H, uint16_t *__restrict__ X, int32_t d,
                     float eps) {
    __shared__ float part[kNThreads / 64];
    const float4 *h = reinterpret_cast<const float4 *>(H + (size_t)blockIdx.x * d);
    uint2 *x = reinterpret_cast<uint2 *>(X + (size_t)blockIdx.x * d);
    const int n4 = d / 4;
    float4 keep[kNKeep];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kNKeep; ++i) {
        const int j = threadIdx.x + i * kNThreads;
        keep[i] = j < n4 ? h[j] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        ss = fmaf(keep[i].x, keep[i].x, ss);
        ss = fmaf(keep[i].y, keep[i].y, ss);
        ss = fmaf(keep[i].z, keep[i].z, ss);
        ss = fmaf(keep[i].w, keep[i].w, ss);
    }
    for (int j = threadIdx.x + kNKeep * kNThreads; j < n4; j += kNThreads) {
        const float4 v = h[j];
        ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
    }
    ss = lanes::wave_sum(ss);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = part[0];
#pragma unroll
    for (int w = 1; w < kNThreads / 64; ++w)
        tot += part[w];
    const float r = 1.0f / sqrtf(tot / (float)d + eps);
    auto emit = [&](int j, const float4 &v) {
        x[j] = make_uint2((uint32_t)f2h(v.x * r) | ((uint32_t)f2h(v.y * r) << 16),
                          (uint32_t)f2h(v.z * r) | ((uint32_t)f2h(v.w * r) << 16));
    };
#pragma unroll
    for (int i = 0; i < kNKeep; ++i) {
        const int j = threadIdx.x + i * kNThreads;
        if (j < n4)
            emit(j, keep[i]);
    }
    for (int j = threadIdx.x + kNKeep * kNThreads; j < n4; j += kNThreads)
        emit(j, h[j]);
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

} // namespace

q4_status launch_rmsnorm_batch(const float *H, uint16_t *X, int32_t B, int32_t d, float eps,
                               hipStream_t s) {
    hipLaunchKernelGGL(rmsnorm_batch_kernel, dim3((unsigned)B), dim3(kNThreads), 0, s, H, X, d,
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

} // namespace q4
