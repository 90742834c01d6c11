// Decode attention over binary16 KV caches (internal interface).
#pragma once

#include "q4_internal.h"

namespace q4 {

struct AttnArgs {
    const float *qkv;       // this token's Q | K | V (fp32)
    uint16_t *kc, *vc;      // this layer's caches, [Hkv][max_ctx][hd] binary16
                            // (one token: row pos already stored)
    const int32_t *pos_dev; // device word: position of the token (context - 1)
    int32_t max_ctx, H, Hkv, hd;
    const void *rope;       // rotation table, float2 [max_ctx][hd/2] (cos, sin)
    // rotated queries f32 [batch][H * hd]: one token reads those the QKV
    // product's epilogue stored with its key and value rows
    // (Epi::QkvRope); a batch has kv_append_batch write them
    const float *qrot = nullptr;
    float *part;            // partials, attention_partial_bytes()
    int32_t nchunk;         // chunks launched (covers the context bucket)
    uint16_t *out;          // binary16 [H * hd] attention output
    // token columns (1..16).  Above 1: qkv, partials and out hold one
    // block per column, column b sits at position *pos_dev + b, and all
    // key/value rows are stored before any column attends (causal batch).
    int32_t batch = 1;
    // a batch whose QKV product's epilogue already stored the key and value
    // rows and the rotated queries (launch_gemm_qkv_rope): no append kernel
    bool rows_stored = false;
};

bool attention_supported(int32_t H, int32_t Hkv, int32_t hd);
size_t attention_partial_bytes(int32_t H, int32_t Hkv, int32_t hd, int32_t max_ctx);
int attention_chunks(int32_t ctx_len);
size_t rope_table_bytes(int32_t max_ctx, int32_t hd);
// Fills the rotation table: entry [p][i] = (cos, sin) of p * base^(-2i/hd),
// evaluated in fp64 and rounded to fp32.
q4_status launch_rope_table(void *rope, int32_t max_ctx, int32_t hd, float base,
                            hipStream_t s);
q4_status launch_set_pos(int32_t *pos_dev, int32_t pos, hipStream_t s);
q4_status launch_attention(const AttnArgs &a, hipStream_t s);

} // namespace q4
