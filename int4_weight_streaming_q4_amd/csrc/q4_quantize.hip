// Quantization of real weights (binary32 or binary16) into the 4-bit format:
// symmetric round-to-nearest per group of 32 consecutive k.
//
// PIPO: Pipelined Offloading for Efficient Inference on Consumer Devices,
// "Method", bullet "Computation optimization" runs its kernel on 4-bit
// weights but gives no rule for producing them.  The rule here, per group:
//   s = binary16(max |w| / 8)              the stored scale (nearest even)
//   c = clamp(rint(w / s) + 8, 0, 15)      w / s the exact quotient,
//                                          rint ties to even
// and a group whose stored scale is 0 gets code 8 everywhere.  One
// correctly rounded binary32 division (the compiler's default division;
// not a reciprocal product) decides that rounding exactly: w has at most 24
// significant bits and s at most 11, so each boundary (n + 1/2) s is a
// binary32 value; a weight next to it differs by at least one unit in the
// last place of w, which moves the quotient by more than half a unit in the
// last place of the quotient, so the rounded quotient never lands on
// n + 1/2 or crosses it, and a weight on the boundary divides to n + 1/2
// exactly.
//
// Four lanes per group: a lane loads 8 consecutive weights (32 bytes of
// binary32 or 16 of binary16), the group maximum is taken across the quad
// with DPP, the lane writes the 4 bytes holding its 8 codes (code 2j in the
// low nibble of byte j) and lane 0 of the quad the scale.  A wave covers 16
// consecutive groups with coalesced loads and stores; the kernel is bound
// by HBM: 4.5 bytes moved per binary32 weight (2.5 for binary16).
#include "q4_internal.h"

namespace {

constexpr int kQThreads = 256;

__device__ __forceinline__ float quad_max(float x) {
    // quad_perm [1,0,3,2] then [2,3,0,1]
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                               0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                               0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true)));
    return x;
}

template <bool F16>
__global__ void __launch_bounds__(kQThreads)
quantize_kernel(const void *__restrict__ w, uint8_t *__restrict__ packed,
                uint16_t *__restrict__ scales, int64_t ngroups) {
    const int64_t tid = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
    const int64_t grp = tid >> 2; // row-major group index n * (K / 32) + g
    const int part = (int)(tid & 3);
    // the four lanes of a quad share grp: they leave together
    if (grp >= ngroups)
        return;
    // rows are contiguous, so group grp starts at element 32 * grp
    const int64_t e0 = grp * 32 + part * 8;
    float v[8];
    if constexpr (F16) {
        const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(w) + e0);
        const uint32_t word[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(word[i] & 0xFFFFu));
            v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(word[i] >> 16));
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(w) + e0);
        const float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        amax = fmaxf(amax, fabsf(v[i]));
    amax = quad_max(amax);
    // amax / 8 is exact unless it is far below the binary16 range
    const _Float16 s16 = (_Float16)(amax * 0.125f);
    const float s = (float)s16;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t c = 8;
        if (s != 0.0f) {
            const float r = rintf(v[i] / s);
            c = (uint32_t)fminf(fmaxf(r + 8.0f, 0.0f), 15.0f);
        }
        word |= c << (4 * i);
    }
    reinterpret_cast<uint32_t *>(packed)[e0 >> 3] = word;
    if (part == 0)
        scales[grp] = __builtin_bit_cast(uint16_t, s16);
}

} // namespace

extern "C" q4_status q4_quantize(const void *w, int32_t w_dtype, uint8_t *packed,
                                 uint16_t *scales, int64_t N, int64_t K, hipStream_t stream) {
    if (!w || !packed || !scales)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_quantize: null pointer");
    if (w_dtype != Q4_DTYPE_F32 && w_dtype != Q4_DTYPE_F16)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_quantize: weight dtype %d", w_dtype);
    if (N < 1 || K < 32 || K % 32 != 0)
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_quantize: need N >= 1, K >= 32, K %% 32 == 0 (N=%lld K=%lld)",
                        (long long)N, (long long)K);
    if (N > ((int64_t)1 << 40) || K > ((int64_t)1 << 40) / N)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_quantize: N*K too large");
    if (!q4::aligned(w, 16) || !q4::aligned(packed, 16) || !q4::aligned(scales, 2))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_quantize: w and packed must be 16-byte, scales 2-byte aligned");
    const int64_t ngroups = N * (K / 32);
    const int64_t blocks = (ngroups * 4 + kQThreads - 1) / kQThreads;
    if (blocks > 0x7FFFFFFF)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_quantize: too many groups");
    if (w_dtype == Q4_DTYPE_F16)
        hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)blocks), dim3(kQThreads), 0,
                           stream, w, packed, scales, ngroups);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)blocks), dim3(kQThreads), 0,
                           stream, w, packed, scales, ngroups);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}
