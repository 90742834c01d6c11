// Glue kernels of the batched (speculative-verify) decode step (internal).
#pragma once

#include "q4_internal.h"

namespace q4 {

// X[b] = f16(H[b] / sqrt(mean(H[b]^2) + eps)) for b < B; H f32[B][d],
// X u16[B][d].
q4_status launch_rmsnorm_batch(const float *H, uint16_t *X, int32_t B, int32_t d, float eps,
                               hipStream_t s);
// o[b][hq * hd + i] = f16(V[b][hq / group][i]), V the last Hkv * hd values
// of each row of qkv f32[B][nqkv].
q4_status launch_gather_batch(const float *qkv, uint16_t *o, int32_t B, int32_t H,
                              int32_t Hkv, int32_t hd, hipStream_t s);

} // namespace q4
