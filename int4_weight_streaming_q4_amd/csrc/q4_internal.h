// Internal helpers of libq4stream (HIP, gfx950).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "q4.h"
#include "q4_measure.h"

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

// Device loads through explicit global (address space 1) pointers: the
// compiler otherwise may emit flat loads, which also count against the LDS
// wait counter and serialise LDS reads behind outstanding HBM loads.
template <class T>
__device__ __forceinline__ T gload(const T *p) {
    typedef const __attribute__((address_space(1))) T global_t;
    return *(global_t *)(p);
}

// 16-byte variant (HIP's uint4 cannot be copied out of address space 1).
__device__ __forceinline__ uint4 gload16(const void *p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(1))) u32x4 global_t;
    const u32x4 v = *(global_t *)(p);
    return uint4{v.x, v.y, v.z, v.w};
}

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
    QkvRope = 4,  // rows (j, j + hd/2) of a head: y = both; query heads also
                  // rotated into qrot, key heads rotated and value heads as
                  // they are, in binary16, into row *pos_dev of the caches
};

// How the workgroup stages its activation vector.
enum class Pro : int {
    F16 = 0,     // binary16 x given
    RmsNorm = 1, // x = f16(h / sqrt(mean(h^2) + eps)) from the fp32 residual h
};

struct EpiArgs {
    float *y;          // Store / QkvGather: f32 out; Residual: h
    uint16_t *out16;   // QkvGather: o_in f16[H*hd]; SiluPair: m f16[dff]
    int64_t v_off;     // QkvGather: first V row ((H + Hkv) * hd)
    int32_t hd;        // QkvGather: head dim
    int32_t group;     // QkvGather: query heads per key/value head
    int64_t pair_off;  // SiluPair: dff
    float eps;         // RmsNorm prologue: epsilon
    uint16_t *norm_out;// RmsNorm prologue: workgroup 0 writes the normed f16 x here
    // QkvRope (hd, n_q_heads, n_kv_heads as the layer's): position word,
    // rotation table (cos, sin) [max_ctx][hd/2], rotated queries f32
    // [n_q_heads * hd], this layer's caches [n_kv_heads][max_ctx][hd]
    const int32_t *pos_dev;
    const float2 *rope;
    float *qrot;
    uint16_t *kc, *vc;
    int32_t n_q_heads, n_kv_heads, max_ctx;
};

// Launches the product kernel: rows of W (N x K) against the activation
// given by `xin` (binary16 u16[K] for Pro::F16, the fp32 residual f32[K] for
// Pro::RmsNorm) with the chosen epilogue.  launch_gemv picks the launch
// shape; launch_gemv_cfg takes it (R rows per 16-lane row, KS-way k split, U
// chunks per row in flight, NT non-temporal weight loads, pipe the
// software-pipelined loop, which needs U == 2 and NT).
q4_status launch_gemv(const uint8_t *packed, const uint16_t *scales, const void *xin, Pro pro,
                      int64_t N, int64_t K, Epi epi, const EpiArgs &ea, hipStream_t stream);
q4_status launch_gemv_cfg(const uint8_t *packed, const uint16_t *scales, const void *xin,
                          Pro pro, int64_t N, int64_t K, Epi epi, const EpiArgs &ea, int R,
                          int KS, int U, bool NT, bool pipe, hipStream_t stream);

// The row-per-wave kernels of q4_gemv_row.hip run every product for which
// use_row_kernels holds (K <= 4096, or any epilogue but SiluPair): each wave
// sweeps whole rows, its activation chunks in registers or read from LDS
// (batch 1) or the columns in LDS (batch 2..4, 8 for measurement), each
// column in the batch-1 order; launch_gemv_row picks the launch shape from
// the product's.  Paired rows with K > 4096 keep the product kernel of
// q4_gemv.hip.
bool use_row_kernels(Epi e, int64_t K);
q4_status launch_gemv_row(const uint8_t *packed, const uint16_t *scales, const void *xin,
                          Pro pro, int64_t N, int64_t K, Epi epi, const EpiArgs &ea,
                          hipStream_t stream);
q4_status launch_gemv_row_batch(const uint8_t *packed, const uint16_t *scales,
                                const uint16_t *X16, int64_t N, int64_t K, int32_t B, Epi epi,
                                const EpiArgs &ea, hipStream_t stream);

// Rows per slot and k split the batch-1 product uses for an N x K product
// with epilogue e (N counts both halves of paired rows).
void gemv_shape(Epi e, int64_t N, int64_t K, int *R, int *KS);

// Small-batch product on the vector ALUs (q4_gemv_batch.hip): B binary16
// columns X16[B][K] staged in LDS, each column computed exactly as the
// batch-1 product computes it.  Store / Residual: ea.y = Y f32 [B][N];
// SiluPair: ea.out16 = M binary16 [B][pair_off].  Kernels exist for B in
// {2, 3, 4} (and 8 for Store); the staged columns must fit kBatchStageBytes.
constexpr int kBatchStageBytes = 65536;
constexpr int kBatchMaxCols = 3; // widest batch the library sends to these kernels
bool gemv_batch_fits(int32_t B, int64_t K); // 2 <= B <= kBatchMaxCols, B * K * 2 <= kBatchStageBytes
q4_status launch_gemv_batch(const uint8_t *packed, const uint16_t *scales, const uint16_t *X16,
                            int64_t N, int64_t K, int32_t B, Epi epi, const EpiArgs &ea,
                            hipStream_t stream);

// Small-batch product with matrix cores (2 <= B <= 16).
q4_status launch_gemm_mfma(const uint8_t *packed, const uint16_t *scales,
                           const uint16_t *X16, float *Y, int64_t N, int64_t K,
                           int32_t B, hipStream_t stream, bool accumulate = false);
// The QKV product of B token columns (column b at position *pos_dev + b)
// whose epilogue, where the matrix-core row-tile launch takes the product,
// also stores what attention over the KV cache needs: the query heads
// rotated into qrot (f32 [B][nq * hd]), the rotated key and the value of
// every key/value head, in binary16, into cache rows *pos_dev + b (caches
// [nkv][max_ctx][hd]).  Y holds the unrotated rows either way; *stored
// tells whether the epilogue ran (otherwise the caller appends the rows).
struct GRope {
    const int32_t *pos_dev = nullptr;
    const float2 *rope = nullptr; // (cos, sin) [max_ctx][hd / 2]
    float *qrot = nullptr;
    uint16_t *kc = nullptr, *vc = nullptr;
    int32_t hd = 0, nq = 0, nkv = 0, max_ctx = 0;
};
q4_status launch_gemm_qkv_rope(const uint8_t *packed, const uint16_t *scales,
                               const uint16_t *X16, float *Y, int64_t N, int64_t K, int32_t B,
                               const GRope &rp, hipStream_t stream, bool *stored);
// Small-batch gate+up product with the SiLU gate fused: `packed` holds npair
// gate rows then npair up rows; M[b][u] = binary16(silu(gate) * up).
q4_status launch_gemm_silu_pair(const uint8_t *packed, const uint16_t *scales,
                                const uint16_t *X16, uint16_t *M, int64_t npair, int64_t K,
                                int32_t B, hipStream_t stream);

} // namespace q4
