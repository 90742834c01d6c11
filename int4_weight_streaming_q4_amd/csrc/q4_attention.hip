// Decode attention over binary16 KV caches, inside the captured step.
//
// The decode step is captured once per context-length bucket and replayed
// per token (PipeLLM: Faster Local LLM Inference Than llama.cpp via
// System-Level Optimizations, "Layer 1: CUDA Graph Compilation"); attention
// over the cached keys and values of earlier tokens is what makes the bucket
// length matter, and the KV cache is the per-layer state an offloading
// pipeline loads and saves next to the weights (PIPO: Pipelined Offloading
// for Efficient Inference on Consumer Devices, "Method", "Pipeline design").
// The pages fix neither the attention arithmetic nor the positional
// encoding; this is the plain Llama-shaped reading: grouped-query heads,
// rotate-half rotary embedding, scores (q . k) / sqrt(hd), softmax, o =
// sum_j p_j v_j.
//
// One token: the QKV product's epilogue rotates the queries and the new key
// (a table of cos/sin per position, angles taken in fp64 once when the
// decoder is created) and stores the token's key and value rows into the
// caches (Epi::QkvRope); then two kernels per layer, split over the context
// like flash decoding:
//   attn_partial  one workgroup per (key/value head, chunk of 64 positions):
//                 scores on the matrix cores, a softmax over the chunk and
//                 the weighted value sum, written as a partial (chunk max,
//                 chunk sum, unnormalised output).
//   attn_merge    one wave per (query head, 64 dims): merges the partials
//                 of the chunks and writes the binary16 attention output the
//                 O product reads.
// The position comes from a device word, so one captured graph serves every
// context length of its bucket: chunks past the position write an empty
// partial.  Draft batches (several token columns) take kv_append_batch and
// attn_tile_mfma in place of attn_partial (the rows and rotated queries
// stored by the batched QKV product's epilogue, or by kv_append_batch after
// the launches that keep a plain epilogue), then the same merge.
#include <algorithm>
#include <cmath>

#include "q4_attention.h"
#include "q4_lanes.h"

namespace q4 {
namespace {

using namespace lanes;

constexpr int kAP = 64;        // positions per chunk
constexpr int kAThreads = 256;

__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__global__ void set_pos_kernel(int32_t *pos_dev, int32_t pos) { *pos_dev = pos; }

// Rotation table (cos, sin) of every position and frequency, angles in fp64
// rounded once to fp32: rope[p * half + i] at angle p * base^(-2i/hd).
__global__ void rope_table_kernel(float2 *rope, int32_t max_ctx, int32_t hd, double base) {
    const int half = hd / 2;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)max_ctx * half)
        return;
    const int p = (int)(i / half), f = (int)(i % half);
    const double ang = (double)p * pow(base, -2.0 * (double)f / (double)hd);
    rope[i] = make_float2((float)cos(ang), (float)sin(ang));
}

// QH query heads per key/value head, HD head dimension; four waves.  The
// QKV product before it stored the token's rotated queries (qrot) and its
// key and value rows (cache row pos), so every load here is known at
// launch: the queries first, then the cache tiles, all in flight while the
// position word is read; the position only masks.
//   scores   S = Q K^T on the matrix cores (v_mfma_f32_16x16x32_f16, fp32
//            accumulation): wave w takes positions 16w .. 16w + 15, whose
//            key rows it loads from the cache straight into the operand
//            layout (no LDS).  The rotated fp32 queries enter as two
//            binary16 halves (x = hi + lo, hi = f16(x), lo = f16(x - hi)),
//            so each product is two passes and agrees with an fp32
//            evaluation to about 2^-22 relative (queries beyond binary16
//            range are not supported); keys are binary16 already.
//   softmax  wave w takes heads w, w + 4; lane = position.  It runs before
//            the value tile is staged, while the value rows are in flight.
//   values   O = P V on the matrix cores the same way (weights as two
//            binary16 halves): wave w takes the 16-dimension tiles w,
//            w + 4, ...; the value tile is staged row-major in LDS and each
//            lane gathers its operand's eight positions of one dimension.
// A chunk past the position runs the same path with no position in the
// context: its partial is empty (max -inf, sum 0, o 0).
template <int QH, int HD>
__global__ void __launch_bounds__(kAThreads)
attn_partial(const float *__restrict__ qrot, const uint16_t *__restrict__ kc,
             const uint16_t *__restrict__ vc, const int32_t *__restrict__ pos_dev,
             int32_t max_ctx, float *__restrict__ part, int32_t nchunk) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int KT = HD / 32;                 // k steps of the scores
    constexpr int DB = HD / 8;                  // 16-byte blocks per row
    constexpr int TL = kAP * DB / kAThreads;    // value-tile blocks per thread
    constexpr int NW = kAThreads / 64;
    constexpr int QP = HD + 8;                  // query-half row stride (halves)
    constexpr int Q4N = QH * HD / 4;            // float4 blocks of the queries
    constexpr int SV = HD / 2 + 2;              // value row stride (dwords): rows
                                                // 8 apart 16 banks apart
    constexpr int EP = kAP + 4;                 // weight row stride (floats)
    static_assert(HD == 64 || HD == 128, "head dimension");
    static_assert(QH <= 8 && NW == 4 && kAP == 64 && TL >= 1, "layout");
    static_assert(Q4N <= kAThreads, "one query block per thread");
    __shared__ __align__(16) uint16_t qhi[QH][QP];
    __shared__ __align__(16) uint16_t qlo[QH][QP];
    __shared__ __align__(16) uint32_t vsh[kAP * SV];
    __shared__ __align__(16) float ssh[QH][kAP];
    __shared__ __align__(16) float esh[QH][EP];

    const int g = blockIdx.x, c = blockIdx.y;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int li = lane & 15, lk = lane >> 4;
    const int c0 = c * kAP;
    const size_t prow = (size_t)(HD + 2);
    float *pout = part + (((size_t)g * nchunk + c) * QH) * prow;
    const size_t gbase = (size_t)g * max_ctx + c0;
    const int rlim = max_ctx - 1 - c0;         // last cache row of the chunk

    // the group's queries (threads past the last block repeat it), then the
    // cache tiles: rows past the cache read its last row; rows past the
    // context, whatever the cache holds there, get masked scores and zero
    // value rows below.  Key rows in the operand layout: lane (li, lk) of
    // wave w holds row 16w + li, dimensions 32k + 8lk .. + 7 of step k.
    const int qb = t < Q4N ? t : Q4N - 1;
    const float4 qv = *reinterpret_cast<const float4 *>(qrot + (size_t)g * QH * HD + qb * 4);
    const int kr = w * 16 + li;
    uint4 kt[KT];
    {
        const uint16_t *krow = kc + (gbase + (kr < rlim ? kr : rlim)) * HD + lk * 8;
#pragma unroll
        for (int k = 0; k < KT; ++k)
            kt[k] = *reinterpret_cast<const uint4 *>(krow + k * 32);
    }
    uint4 vt[TL];
#pragma unroll
    for (int m = 0; m < TL; ++m) {
        const int blk = t + m * kAThreads;
        const int r = blk / DB, cb = blk % DB;
        vt[m] = *reinterpret_cast<const uint4 *>(vc + (gbase + (r < rlim ? r : rlim)) * HD +
                                                 cb * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    // positions of the chunk in the context (0 for a chunk past it)
    const int pos = *pos_dev;
    const int n = max(0, min(kAP, pos + 1 - c0));

    // queries as binary16 halves
    {
        const int h = (qb * 4) / HD, d = (qb * 4) % HD;
        const float qx[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const _Float16 hi = (_Float16)qx[e];
            qhi[h][d + e] = __builtin_bit_cast(uint16_t, hi);
            qlo[h][d + e] = f2h(qx[e] - (float)hi);
        }
    }
    __syncthreads();

    // scores: rows of the product are query heads (rows QH .. 15 zero),
    // columns the wave's 16 positions
    {
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        const bool qlive = li < QH;
        const int qrow = qlive ? li : 0;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const int d0 = k * 32 + lk * 8;
            const uint4 kk = make_uint4(kt[k].x, kt[k].y, kt[k].z, kt[k].w);
            const h8 bk = __builtin_bit_cast(h8, kk);
            uint4 uh = make_uint4(0u, 0u, 0u, 0u), ul = make_uint4(0u, 0u, 0u, 0u);
            if (qlive) {
                uh = *reinterpret_cast<const uint4 *>(&qhi[qrow][d0]);
                ul = *reinterpret_cast<const uint4 *>(&qlo[qrow][d0]);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, uh), bk, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, ul), bk, acc, 0, 0, 0);
        }
        // lane (li, lk) holds heads 4lk .. 4lk + 3 of position 16w + li
        const float scale = 1.0f / sqrtf((float)HD);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int h = 4 * lk + e;
            if (h < QH)
                ssh[h][kr] = kr < n ? acc[e] * scale : -INFINITY;
        }
    }
    __syncthreads();

    // softmax over the chunk: wave w takes heads w, w + 4; lane = position
    for (int h = w; h < QH; h += NW) {
        const float sv = ssh[h][lane];
        const float m = wave_max(sv);
        const float e = lane < n ? expf(sv - m) : 0.0f;
        const float l = wave_sum(e);
        esh[h][lane] = e;
        if (lane == 0) {
            pout[h * prow + HD] = m;
            pout[h * prow + HD + 1] = l;
        }
    }
    // value tile into LDS (row-major, 8-byte stores), rows past the context
    // zero (their weights are 0, whatever the cache holds there)
#pragma unroll
    for (int m = 0; m < TL; ++m) {
        const int blk = t + m * kAThreads;
        const int r = blk / DB, cb = blk % DB;
        const bool live = r < n;
        const uint2 v0 = make_uint2(live ? vt[m].x : 0u, live ? vt[m].y : 0u);
        const uint2 v1 = make_uint2(live ? vt[m].z : 0u, live ? vt[m].w : 0u);
        *reinterpret_cast<uint2 *>(vsh + r * SV + cb * 4) = v0;
        *reinterpret_cast<uint2 *>(vsh + r * SV + cb * 4 + 2) = v1;
    }
    __syncthreads();

    // O = P V: rows of the product are query heads (rows QH .. 15 zero),
    // columns the tile's 16 dimensions; lane (li, lk) takes positions
    // 32s + 8lk .. + 7 of step s
    {
        const bool plive = li < QH;
        const int prow_ = plive ? li : 0;
        h8 ph[2], pl[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            float4 p0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), p1 = p0;
            if (plive) {
                p0 = *reinterpret_cast<const float4 *>(&esh[prow_][k * 32 + lk * 8]);
                p1 = *reinterpret_cast<const float4 *>(&esh[prow_][k * 32 + lk * 8 + 4]);
            }
            const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ph[k][e] = (_Float16)pv[e];
                pl[k][e] = (_Float16)(pv[e] - (float)ph[k][e]);
            }
        }
        const uint16_t *vs16 = reinterpret_cast<const uint16_t *>(vsh);
        for (int dt = w; dt < HD / 16; dt += NW) {
            f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint16_t *col = vs16 + (k * 32 + lk * 8) * (2 * SV) + dt * 16 + li;
                h8 bv;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    bv[e] = __builtin_bit_cast(_Float16, col[e * 2 * SV]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[k], bv, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl[k], bv, acc, 0, 0, 0);
            }
            // lane (li, lk) holds heads 4lk .. 4lk + 3 of dimension 16dt + li
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int h = 4 * lk + e;
                if (h < QH)
                    pout[h * prow + dt * 16 + li] = acc[e];
            }
        }
    }
}

// One wave per (query head, 64 dims of it, token column) merges the chunk
// partials (chunk max m_c, chunk sum l_c, unnormalised o_c): o = sum_c o_c
// e^(m_c - M) / sum_c l_c e^(m_c - M), M the largest m_c.  Lane c takes
// chunk c's maximum and sum (64 chunks per round, a running maximum across
// rounds), so the weights are one exponential per lane; lane d's output
// dimension then sums o_c[d] times chunk c's weight, read from lane c.  A
// round's loads are all in flight at once; no LDS, no barrier.  One token
// (BATCH false) reads every chunk without waiting for the position word:
// attn_partial wrote those past the position as empty partials (max -inf,
// weight 0).  Column b of a batch reads the chunks up to its position.
template <int QH, int HD, bool BATCH>
__global__ void __launch_bounds__(64)
attn_merge(const float *__restrict__ part, const int32_t *__restrict__ pos_dev, int32_t nchunk,
           uint16_t *__restrict__ out) {
    static_assert(HD % 64 == 0, "dims per wave");
    const int hq = blockIdx.x, lane = threadIdx.x;
    const int d = blockIdx.y * 64 + lane;
    const int g = hq / QH, h = hq % QH;
    const size_t prow = (size_t)(HD + 2);
    const size_t cstride = (size_t)QH * prow;
    int nc = nchunk;
    if (BATCH) {
        const int col = (int)blockIdx.z;
        part += (size_t)col * (gridDim.x / QH) * nchunk * QH * prow;
        out += (size_t)col * gridDim.x * HD;
        nc = min(nchunk, (*pos_dev + col) / kAP + 1);
    }
    const float *base = part + ((size_t)g * nchunk * QH + h) * prow;
    const int last = nc - 1;
    float M = -INFINITY, L = 0.0f, O = 0.0f;
    for (int cb = 0; cb < nc; cb += 64) {
        // lanes and values past the last chunk: weight 0, and the clamped
        // loads read a written chunk
        const float2 ml =
            *reinterpret_cast<const float2 *>(base + (size_t)min(cb + lane, last) * cstride + HD);
        float ov[64];
#pragma unroll
        for (int k = 0; k < 64; ++k)
            ov[k] = base[(size_t)min(cb + k, last) * cstride + d];
        const float mc = cb + lane <= last ? ml.x : -INFINITY;
        const float Mn = fmaxf(M, wave_max(mc));
        // an empty chunk (max -inf) has weight 0, and a running max of -inf
        // means L = O = 0: the guards keep -inf - -inf out of expf
        const float r = M == -INFINITY ? 1.0f : expf(M - Mn);
        const float wc = mc == -INFINITY ? 0.0f : expf(mc - Mn);
        L = fmaf(L, r, wave_sum(ml.y * wc));
        O *= r;
#pragma unroll
        for (int k = 0; k < 64; ++k)
            O = fmaf(ov[k],
                     __builtin_bit_cast(float,
                                        __builtin_amdgcn_readlane(__builtin_bit_cast(int, wc), k)),
                     O);
        M = Mn;
    }
    out[(size_t)hq * HD + d] = f2h(O / L);
}

// Key and value rows of a batch of token columns: column b (blockIdx.y) at
// position *pos_dev + b, key rotated, both rounded to binary16; the
// column's query heads of the group rotated into qrot (f32 [b][H * hd]).
template <int QH, int HD>
__global__ void __launch_bounds__(HD / 2)
kv_append_batch(const float *__restrict__ qkv, uint16_t *__restrict__ kc,
                uint16_t *__restrict__ vc, const float2 *__restrict__ rope,
                const int32_t *__restrict__ pos_dev, int32_t max_ctx, int32_t H, int32_t Hkv,
                float *__restrict__ qrot) {
    constexpr int HALF = HD / 2;
    const int g = blockIdx.x, col = blockIdx.y, d = threadIdx.x;
    const int pos = *pos_dev + col;
    const float *row = qkv + (size_t)col * (H + 2 * Hkv) * HD;
    const float *k = row + (size_t)(H + g) * HD;
    const float *v = row + (size_t)(H + Hkv + g) * HD;
    const float2 cs = rope[(size_t)pos * HALF + d];
    const float a = k[d], b = k[d + HALF];
    uint16_t *krow = kc + ((size_t)g * max_ctx + pos) * HD;
    uint16_t *vrow = vc + ((size_t)g * max_ctx + pos) * HD;
    krow[d] = f2h(a * cs.x - b * cs.y);
    krow[d + HALF] = f2h(a * cs.y + b * cs.x);
    vrow[d] = f2h(v[d]);
    vrow[d + HALF] = f2h(v[d + HALF]);
    float *qo = qrot + (size_t)col * H * HD;
#pragma unroll
    for (int h = 0; h < QH; ++h) {
        const float *q = row + (size_t)(g * QH + h) * HD;
        const float x = q[d], y = q[d + HALF];
        qo[(size_t)(g * QH + h) * HD + d] = x * cs.x - y * cs.y;
        qo[(size_t)(g * QH + h) * HD + d + HALF] = x * cs.y + y * cs.x;
    }
}

// Matrix-core attention tile for draft batches: one workgroup per
// (key/value head, chunk of 64 positions) for all `batch` columns (column b
// at position *pos_dev + b; rows r = b * QH + h of the query matrix), the
// single-token pass extended to several row tiles.  kv_append_batch stored
// the columns' key and value rows and their rotated queries first, so
// every load is known at launch: the queries, the key rows (each wave the
// 16 positions 16w .. 16w + 15, straight into the operand layout) and the
// value tile go out before the position word is read.  S = Q K^T and O =
// P V are v_mfma_f32_16x16x32_f16 products with fp32 accumulation; the fp32
// queries and weights enter as two binary16 halves (x = hi + lo, hi =
// f16(x), lo = f16(x - hi)), so each product is two passes and agrees with
// an fp32 evaluation to about 2^-22 relative; keys and values are binary16
// already.  Scores are masked causally per column (position <= its own);
// a row with no position in the chunk gets an empty partial.  LDS: the
// query halves, the value tile (row-major, each lane gathering its
// operand's eight positions of one dimension), the scores/weights.
template <int QH, int HD>
__global__ void __launch_bounds__(kAThreads)
attn_tile_mfma(const float *__restrict__ qrot, const uint16_t *__restrict__ kc,
               const uint16_t *__restrict__ vc, const int32_t *__restrict__ pos_dev,
               int32_t max_ctx, int32_t H, int32_t Hkv, float *__restrict__ part,
               int32_t nchunk, int32_t batch) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int KT = HD / 32;                 // k steps of the scores
    constexpr int DB = HD / 8;                  // 16-byte blocks per row
    constexpr int TL = kAP * DB / kAThreads;    // value-tile blocks per thread
    constexpr int NW = kAThreads / 64;
    constexpr int QP = HD + 8;                  // query-half row stride (halves)
    constexpr int SV = HD / 2 + 2;              // value row stride (dwords)
    constexpr int SP = kAP + 4;                 // score row stride (floats)
    constexpr int QB = HD / 4;                  // float4 blocks per query row
    constexpr int QL = (Q4_MAX_BATCH * QH * QB + kAThreads - 1) / kAThreads; // per thread, at most
    static_assert(HD == 64 || HD == 128, "head dimension");
    static_assert(QH <= 8 && NW == 4 && kAP == 64 && TL >= 1, "layout");
    extern __shared__ __align__(16) unsigned char smem[];
    const int rows = batch * QH;
    const int RT = (rows + 15) / 16;
    const int RP = RT * 16;                     // padded rows
    uint16_t *qh = reinterpret_cast<uint16_t *>(smem);                 // [RP][QP]
    uint16_t *ql = qh + RP * QP;                                       // [RP][QP]
    uint32_t *vsh = reinterpret_cast<uint32_t *>(ql + RP * QP);        // [64][SV]
    float *ps = reinterpret_cast<float *>(vsh + kAP * SV);             // [RP][SP]

    const int g = blockIdx.x, c = blockIdx.y;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int li = lane & 15, lk = lane >> 4;
    const int c0 = c * kAP;
    const size_t prow = (size_t)(HD + 2);
    const size_t colstride = (size_t)Hkv * nchunk * QH * prow;
    const size_t gbase = (size_t)g * max_ctx + c0;
    const int rlim = max_ctx - 1 - c0;          // last cache row of the chunk

    // queries of the rows (r = b * QH + h, float4 blocks; padding rows and
    // blocks past them repeat the last block), key rows, value tile
    const int nqb = rows * QB;
    float4 qv[QL];
#pragma unroll
    for (int m = 0; m < QL; ++m) {
        const int i = t + m * kAThreads;
        const int ic = i < nqb ? i : nqb - 1;
        const int r = ic / QB, e = ic % QB;
        qv[m] = *reinterpret_cast<const float4 *>(
            qrot + (size_t)(r / QH) * H * HD + (size_t)(g * QH + r % QH) * HD + e * 4);
    }
    const int kr = w * 16 + li;
    uint4 kt[KT];
    {
        const uint16_t *krow = kc + (gbase + (kr < rlim ? kr : rlim)) * HD + lk * 8;
#pragma unroll
        for (int k = 0; k < KT; ++k)
            kt[k] = *reinterpret_cast<const uint4 *>(krow + k * 32);
    }
    uint4 vt[TL];
#pragma unroll
    for (int m = 0; m < TL; ++m) {
        const int blk = t + m * kAThreads;
        const int r = blk / DB, cb = blk % DB;
        vt[m] = *reinterpret_cast<const uint4 *>(vc + (gbase + (r < rlim ? r : rlim)) * HD +
                                                 cb * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int pos0 = *pos_dev;
    const int nrow = max(0, min(kAP, pos0 + batch - c0)); // rows any column reads

    // query halves; padding rows zero
#pragma unroll
    for (int m = 0; m < QL; ++m) {
        const int i = t + m * kAThreads;
        if (i < RP * QB) {
            const int r = i / QB, e = i % QB;
            const bool live = r < rows;
            const float qx[4] = {qv[m].x, qv[m].y, qv[m].z, qv[m].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float x = live ? qx[u] : 0.0f;
                const _Float16 hi = (_Float16)x;
                qh[r * QP + e * 4 + u] = __builtin_bit_cast(uint16_t, hi);
                ql[r * QP + e * 4 + u] = f2h(x - (float)hi);
            }
        }
    }
    __syncthreads();

    // scores of every row tile for the wave's 16 positions
    const float scale = 1.0f / sqrtf((float)HD);
    for (int rt = 0; rt < RT; ++rt) {
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const int d0 = k * 32 + lk * 8;
            const uint4 kk = make_uint4(kt[k].x, kt[k].y, kt[k].z, kt[k].w);
            const h8 bk = __builtin_bit_cast(h8, kk);
            const h8 ah = *reinterpret_cast<const h8 *>(qh + (rt * 16 + li) * QP + d0);
            const h8 al = *reinterpret_cast<const h8 *>(ql + (rt * 16 + li) * QP + d0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bk, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bk, acc, 0, 0, 0);
        }
        // lane (li, lk) holds rows rt * 16 + 4lk .. + 3 of position kr
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rt * 16 + 4 * lk + e;
            const bool live = r < rows && c0 + kr <= pos0 + r / QH;
            ps[r * SP + kr] = live ? acc[e] * scale : -INFINITY;
        }
    }
    __syncthreads();

    // softmax of each row over the chunk: rows w, w + 4, ...; lane = position
    for (int r = w; r < RP; r += NW) {
        const float sv = ps[r * SP + lane];
        const float m = wave_max(sv);
        const float e = m == -INFINITY ? 0.0f : expf(sv - m);
        const float l = wave_sum(e);
        ps[r * SP + lane] = e;
        if (lane == 0 && r < rows) {
            float *pout = part + (size_t)(r / QH) * colstride +
                          (((size_t)g * nchunk + c) * QH + r % QH) * prow;
            pout[HD] = m;
            pout[HD + 1] = l;
        }
    }
    // value tile into LDS (row-major, 8-byte stores), rows no column reads
    // zero
#pragma unroll
    for (int m = 0; m < TL; ++m) {
        const int blk = t + m * kAThreads;
        const int r = blk / DB, cb = blk % DB;
        const bool live = r < nrow;
        const uint2 v0 = make_uint2(live ? vt[m].x : 0u, live ? vt[m].y : 0u);
        const uint2 v1 = make_uint2(live ? vt[m].z : 0u, live ? vt[m].w : 0u);
        *reinterpret_cast<uint2 *>(vsh + r * SV + cb * 4) = v0;
        *reinterpret_cast<uint2 *>(vsh + r * SV + cb * 4 + 2) = v1;
    }
    __syncthreads();

    // O = P V: wave w takes the 16-dimension tiles w, w + 4 of every row
    // tile; the value operand of a (tile, k step) serves every row tile
    const uint16_t *vs16 = reinterpret_cast<const uint16_t *>(vsh);
    for (int dt = w; dt < HD / 16; dt += NW) {
        h8 bv[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint16_t *col = vs16 + (k * 32 + lk * 8) * (2 * SV) + dt * 16 + li;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                bv[k][e] = __builtin_bit_cast(_Float16, col[e * 2 * SV]);
        }
        for (int rt = 0; rt < RT; ++rt) {
            f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float *pr = ps + (rt * 16 + li) * SP + k * 32 + lk * 8;
                const float4 p0 = *reinterpret_cast<const float4 *>(pr);
                const float4 p1 = *reinterpret_cast<const float4 *>(pr + 4);
                const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                h8 ph, pl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ph[e] = (_Float16)pv[e];
                    pl[e] = (_Float16)(pv[e] - (float)ph[e]);
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bv[k], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, bv[k], acc, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = rt * 16 + 4 * lk + e;
                if (r < rows)
                    part[(size_t)(r / QH) * colstride +
                         (((size_t)g * nchunk + c) * QH + r % QH) * prow + dt * 16 + li] = acc[e];
            }
        }
    }
}

size_t tile_mfma_lds(int qh, int hd, int batch) {
    const int rp = (batch * qh + 15) / 16 * 16;
    return 2 * (size_t)rp * (hd + 8) * 2 + (size_t)kAP * (hd / 2 + 2) * 4 +
           (size_t)rp * (kAP + 4) * 4;
}

using AppendFn = void (*)(const float *, uint16_t *, uint16_t *, const float2 *, const int32_t *,
                          int32_t, int32_t, int32_t, float *);

using PartialFn = void (*)(const float *, const uint16_t *, const uint16_t *, const int32_t *,
                           int32_t, float *, int32_t);
using MergeFn = void (*)(const float *, const int32_t *, int32_t, uint16_t *);

using TileFn = void (*)(const float *, const uint16_t *, const uint16_t *, const int32_t *,
                        int32_t, int32_t, int32_t, float *, int32_t, int32_t);

struct AttnFns {
    PartialFn partial = nullptr;
    MergeFn merge = nullptr;
    AppendFn append = nullptr;
    TileFn tile = nullptr;
    size_t tile_lds_max = 0; // dynamic LDS the tile kernel may use (0: not usable)
};

// The tile kernel's dynamic LDS may exceed the default per-block limit:
// opt it into the device's maximum once.
template <int QH, int HD>
size_t tile_lds_limit() {
    static const size_t lim = [] {
        int dev = 0, max_lds = 0, optin = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return (size_t)0;
        if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess)
            max_lds = 0;
        if (hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev) !=
            hipSuccess)
            optin = 0;
        const int lds = std::max(max_lds, optin);
        if (lds <= 0 || hipFuncSetAttribute((const void *)attn_tile_mfma<QH, HD>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize,
                                            lds) != hipSuccess)
            return (size_t)0;
        return (size_t)lds;
    }();
    return lim;
}

template <int QH, int HD>
bool pick(int qh, int hd, bool batch, AttnFns &f) {
    if (qh != QH || hd != HD)
        return false;
    f.partial = attn_partial<QH, HD>;
    f.merge = batch ? attn_merge<QH, HD, true> : attn_merge<QH, HD, false>;
    f.append = kv_append_batch<QH, HD>;
    f.tile = attn_tile_mfma<QH, HD>;
    f.tile_lds_max = tile_lds_limit<QH, HD>();
    return true;
}

} // namespace

bool attention_supported(int32_t H, int32_t Hkv, int32_t hd) {
    if (Hkv < 1 || H % Hkv != 0)
        return false;
    const int qh = H / Hkv;
    return (qh == 1 || qh == 2 || qh == 4 || qh == 8) && (hd == 64 || hd == 128);
}

size_t attention_partial_bytes(int32_t H, int32_t Hkv, int32_t hd, int32_t max_ctx) {
    const size_t nchunk = ((size_t)max_ctx + kAP - 1) / kAP;
    return (size_t)H * nchunk * (size_t)(hd + 2) * sizeof(float);
}

int attention_chunks(int32_t ctx_len) { return (ctx_len + kAP - 1) / kAP; }

size_t rope_table_bytes(int32_t max_ctx, int32_t hd) {
    return (size_t)max_ctx * (size_t)(hd / 2) * sizeof(float2);
}

q4_status launch_rope_table(void *rope, int32_t max_ctx, int32_t hd, float base,
                            hipStream_t s) {
    const int64_t n = (int64_t)max_ctx * (hd / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<float2 *>(rope), max_ctx, hd, (double)base);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

q4_status launch_set_pos(int32_t *pos_dev, int32_t pos, hipStream_t s) {
    hipLaunchKernelGGL(set_pos_kernel, dim3(1), dim3(1), 0, s, pos_dev, pos);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

q4_status launch_attention(const AttnArgs &a, hipStream_t s) {
    AttnFns f;
    const int qh = a.H / a.Hkv;
    const bool bt = a.batch > 1;
    if (a.batch < 1 || a.batch > 16)
        return fail(Q4_ERR_INVALID_ARG, "attention: batch %d", a.batch);
    if (!(pick<1, 64>(qh, a.hd, bt, f) || pick<2, 64>(qh, a.hd, bt, f) ||
          pick<4, 64>(qh, a.hd, bt, f) || pick<8, 64>(qh, a.hd, bt, f) ||
          pick<1, 128>(qh, a.hd, bt, f) || pick<2, 128>(qh, a.hd, bt, f) ||
          pick<4, 128>(qh, a.hd, bt, f) || pick<8, 128>(qh, a.hd, bt, f)))
        return fail(Q4_ERR_UNSUPPORTED, "attention: %d query heads per group, head dim %d", qh,
                    a.hd);
    if (a.nchunk < 1 || a.nchunk * kAP > a.max_ctx + kAP - 1)
        return fail(Q4_ERR_INVALID_ARG, "attention: %d chunks for max_ctx %d", a.nchunk,
                    a.max_ctx);
    if (bt) {
        const size_t lds = tile_mfma_lds(qh, a.hd, a.batch);
        if (lds > f.tile_lds_max)
            return fail(Q4_ERR_UNSUPPORTED, "attention: tile needs %zu bytes of LDS, %zu available",
                        lds, f.tile_lds_max);
        if (!a.qrot)
            return fail(Q4_ERR_INVALID_ARG, "attention: no rotated-query buffer");
        if (!a.rows_stored) {
            hipLaunchKernelGGL(f.append, dim3((unsigned)a.Hkv, (unsigned)a.batch),
                               dim3(a.hd / 2), 0, s, a.qkv, a.kc, a.vc,
                               static_cast<const float2 *>(a.rope), a.pos_dev, a.max_ctx, a.H,
                               a.Hkv, const_cast<float *>(a.qrot));
            Q4_HIP(hipGetLastError());
        }
        hipLaunchKernelGGL(f.tile, dim3((unsigned)a.Hkv, (unsigned)a.nchunk), dim3(kAThreads), lds,
                           s, a.qrot, a.kc, a.vc, a.pos_dev, a.max_ctx, a.H, a.Hkv, a.part,
                           a.nchunk, a.batch);
    } else {
        if (!a.qrot)
            return fail(Q4_ERR_INVALID_ARG, "attention: no rotated queries");
        hipLaunchKernelGGL(f.partial, dim3((unsigned)a.Hkv, (unsigned)a.nchunk), dim3(kAThreads),
                           0, s, a.qrot, a.kc, a.vc, a.pos_dev, a.max_ctx, a.part, a.nchunk);
    }
    Q4_HIP(hipGetLastError());
    hipLaunchKernelGGL(f.merge, dim3((unsigned)a.H, (unsigned)(a.hd / 64), (unsigned)a.batch),
                       dim3(64), 0, s, a.part, a.pos_dev, a.nchunk, a.out);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace q4
