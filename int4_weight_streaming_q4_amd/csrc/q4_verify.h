// Glue kernels of the batched (speculative-verify) decode step (internal).
#pragma once

#include "q4_internal.h"

namespace q4 {

// X[b] = f16(H[b] / sqrt(mean(H[b]^2) + eps)) for b < B; H f32[B][d],
// X u16[B][d].
q4_status launch_rmsnorm_batch(const float *H, uint16_t *X, int32_t B, int32_t d, float eps,
                               hipStream_t s);
// The product of RMSNorm'd columns as one launch (q4_gemv_row.hip): the
// vector-ALU batch kernel normalises H f32[B][K] in its prologue, each
// column exactly as the single-token prologue does, and multiplies (Store:
// ea.y = Y f32 [B][N]; SiluPair: ea.out16, ea.pair_off; ea.eps).  For the
// shapes batch_norm_fits accepts (two or three columns, K <= 4096).
bool batch_norm_fits(int64_t K, int32_t B);
// Whether the paired gate+up product of B columns (npair units) runs on the
// vector ALU (launch_gemm_silu_pair's choice; q4_gemm.hip).
bool silu_pair_on_valu(int64_t npair, int64_t K, int32_t B);
q4_status launch_batch_norm_product(const uint8_t *packed, const uint16_t *scales,
                                    const float *H, int64_t N, int64_t K, int32_t B, Epi epi,
                                    const EpiArgs &ea, hipStream_t stream);
// o[b][hq * hd + i] = f16(V[b][hq / group][i]), V the last Hkv * hd values
// of each row of qkv f32[B][nqkv].
q4_status launch_gather_batch(const float *qkv, uint16_t *o, int32_t B, int32_t H,
                              int32_t Hkv, int32_t hd, hipStream_t s);

} // namespace q4
