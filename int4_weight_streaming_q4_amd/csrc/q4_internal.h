// Internal helpers of libq4stream (HIP, gfx950).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "q4.h"

namespace q4 {

// ------------------------------------------------------------------ status
// Records the message for q4_last_error() and returns the status.
q4_status fail(q4_status st, const char *fmt, ...)
    __attribute__((format(printf, 2, 3)));
q4_status ok();

#define Q4_HIP(call)                                                        \
    do {                                                                    \
        hipError_t e_ = (call);                                             \
        if (e_ != hipSuccess)                                               \
            return ::q4::fail(Q4_ERR_HIP, "%s failed: %s (%s:%d)", #call,   \
                              hipGetErrorString(e_), __FILE__, __LINE__);   \
    } while (0)

#define Q4_CHECK(st)                                                        \
    do {                                                                    \
        q4_status s_ = (st);                                                \
        if (s_ != Q4_OK)                                                    \
            return s_;                                                      \
    } while (0)

inline bool aligned(const void *p, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Validates the operands of one N x K product (shared by gemv, gemm and
// the decoder's matrices).
q4_status check_matrix(const void *packed, const void *scales, int64_t N,
                       int64_t K, const char *what);

// Number of compute units of the current device (cached per device).
int device_cus();

// ------------------------------------------------------------- kernels
// Epilogues of the product kernel.  `Mode` selects how output row units map
// to matrix rows and what is written.
enum class Epi : int {
    Store = 0,    // y[n] = acc
    Residual = 1, // h[n] += acc
    QkvGather = 2,// y[n] = acc; V rows also written as f16 per query head
    SiluPair = 3, // rows (j, j + dff): out_f16[j] = f16(silu(gate) * up)
};

struct EpiArgs {
    float *y;          // Store / QkvGather: f32 out; Residual: h
    uint16_t *out16;   // QkvGather: o_in f16[H*hd]; SiluPair: m f16[dff]
    int64_t v_off;     // QkvGather: first V row ((H + Hkv) * hd)
    int32_t hd;        // QkvGather: head dim
    int32_t group;     // QkvGather: query heads per key/value head
    int64_t pair_off;  // SiluPair: dff
};

// Launches the product kernel: rows of W (N x K) against the binary16
// vector x16 (u16[K]) with the chosen epilogue.
q4_status launch_gemv(const uint8_t *packed, const uint16_t *scales,
                      const uint16_t *x16, int64_t N, int64_t K, Epi epi,
                      const EpiArgs &ea, hipStream_t stream);

// Small-batch product with matrix cores (2 <= B <= 16).
q4_status launch_gemm_mfma(const uint8_t *packed, const uint16_t *scales,
                           const uint16_t *X16, float *Y, int64_t N, int64_t K,
                           int32_t B, hipStream_t stream);

// a = f16(h / sqrt(mean(h^2) + eps)) with one workgroup.
q4_status launch_rmsnorm_f16(const float *h, uint16_t *a, int32_t d, float eps,
                             hipStream_t stream);

} // namespace q4
