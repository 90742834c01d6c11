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
// Two kernels per layer, split over the context like flash decoding:
//   attn_partial  one workgroup per (key/value head, chunk of 64 positions):
//                 loads its cache tile, rotates the group's queries (a
//                 table of cos/sin per position, angles taken in fp64 once
//                 when the decoder is created), the chunk that holds the
//                 current position also rotates the new key and stores it
//                 and the new value into the caches; then scores, a softmax
//                 over the chunk and the weighted value sum, written as a
//                 partial (chunk max, chunk sum, unnormalised output).
//   attn_combine  one workgroup per query head: merges the partials of the
//                 chunks up to the current position and writes the
//                 binary16 attention output the O product reads.
// The position comes from a device word, so one captured graph serves every
// context length of its bucket: chunks past the position write an empty
// partial.
#include <algorithm>
#include <cmath>

#include "q4_attention.h"
#include "q4_lanes.h"

namespace q4 {
namespace {

using namespace lanes;

constexpr int kAP = 64;        // positions per chunk
constexpr int kAThreads = 256;
constexpr int kCThreads = 1024; // combine workgroup

__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

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

__device__ __forceinline__ void unpack8(const uint4 &u, float *f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = h2f((uint16_t)(w[e] & 0xFFFFu));
        f[2 * e + 1] = h2f((uint16_t)(w[e] >> 16));
    }
}

// QH query heads per key/value head, HD head dimension.  The workgroup's
// cache tile (64 K rows and 64 V rows of its group) is loaded into
// registers first, so its latency overlaps the rotation of the queries.
template <int QH, int HD>
__global__ void __launch_bounds__(kAThreads)
attn_partial(const float *__restrict__ qkv, uint16_t *__restrict__ kc, uint16_t *__restrict__ vc,
             const float2 *__restrict__ rope, const int32_t *__restrict__ pos_dev,
             int32_t max_ctx, int32_t H, int32_t Hkv, float *__restrict__ part, int32_t nchunk) {
    constexpr int HALF = HD / 2;
    constexpr int QD = HD / 4;                 // dims per lane in the scores
    constexpr int KL = QD / 8;                 // 16-byte K loads per lane
    constexpr int DB = HD / 8;                 // 16-byte blocks per row
    constexpr int PG = kAThreads / DB;         // position groups in the value sum
    constexpr int VL = kAP / PG;               // V rows per lane
    constexpr int NW = kAThreads / 64;
    static_assert(HD % 32 == 0 && HD <= 256, "head dimension");
    static_assert(kAThreads % DB == 0 && kAP % PG == 0 && (DB == 8 || DB == 16), "value-sum layout");
    __shared__ float qr[QH][HD];               // rotated queries
    __shared__ __align__(16) uint16_t knew[HD];
    __shared__ __align__(16) uint16_t vnew[HD];
    __shared__ float sc[QH][kAP];              // scores, then weights
    __shared__ float mx[QH], sm[QH];
    __shared__ float vred[NW][QH][HD];

    const int g = blockIdx.x, c = blockIdx.y;
    const int t = threadIdx.x;
    const int pos = *pos_dev;
    const int c0 = c * kAP;
    const size_t prow = (size_t)(HD + 2);
    float *pout = part + (((size_t)g * nchunk + c) * QH) * prow;
    if (c0 > pos) {
        // empty partial: no positions of this chunk are in the context
        for (int i = t; i < QH * (HD + 2); i += kAThreads) {
            const int h = i / (HD + 2), e = i % (HD + 2);
            pout[h * prow + e] = e == HD ? -INFINITY : 0.0f;
        }
        return;
    }
    const int n = min(kAP, pos + 1 - c0);
    const int jn = pos - c0;                   // row of the new token (>= kAP: not here)
    const size_t gbase = (size_t)g * max_ctx + c0;

    // The operands of this thread's first query rotation are loaded first,
    // then the cache tile, so the rotation waits only for its own operands
    // while the tile is in flight.  Every one of these loads is issued
    // unconditionally (indices clamped into valid rows and elements): a
    // load behind a per-lane branch makes the compiler's next wait cover
    // every load in flight, which had the value tile wait for the key tile
    // and the rotation for both.  Rows past the context (r >= n) load row
    // n - 1, a written row: their scores are masked out of the softmax and
    // their weights are 0, so the results are those of zero rows.
    const float2 *rp = rope + (size_t)pos * HALF;
    const int i0 = t < QH * HALF ? t : QH * HALF - 1;
    const float *q0 = qkv + (size_t)(g * QH + i0 / HALF) * HD;
    const float2 cs0 = rp[i0 % HALF];
    const float qa0 = q0[i0 % HALF], qb0 = q0[i0 % HALF + HALF];
    // the new token's key and value operands (used by the chunk holding its
    // row; every workgroup loads them, clamped, so no load is conditional)
    const int dk = t < HALF ? t : HALF - 1, dv = t < HD ? t : HD - 1;
    const float *kq = qkv + (size_t)(H + g) * HD;
    const float *vq = qkv + (size_t)(H + Hkv + g) * HD;
    const float2 csk = rp[dk];
    const float ka0 = kq[dk], kb0 = kq[dk + HALF], v0 = vq[dv];
    __builtin_amdgcn_sched_barrier(0); // keep these loads ahead of the tile's

    // cache tile loads; the row of the new token is replaced from LDS below
    const int jj = t >> 2, qq = t & 3;
    uint4 kreg[KL];
    {
        const uint16_t *kr = kc + (gbase + (jj < n ? jj : n - 1)) * HD + qq * QD;
#pragma unroll
        for (int b = 0; b < KL; ++b)
            kreg[b] = *reinterpret_cast<const uint4 *>(kr + b * 8);
    }
    const int db = t % DB, pg = t / DB;
    uint4 vreg[VL];
#pragma unroll
    for (int i = 0; i < VL; ++i) {
        const int r = pg + i * PG;
        vreg[i] = *reinterpret_cast<const uint4 *>(vc + (gbase + (r < n ? r : n - 1)) * HD +
                                                   db * 8);
    }
    // The new token's operands are consumed here, so the compiler cannot
    // sink their loads into the branch below, behind the tile's.
    asm volatile("" ::"v"(ka0), "v"(kb0), "v"(v0), "v"(csk.x), "v"(csk.y));

    // rotate the group's queries; the chunk of the new token also rotates
    // its key and stores key and value into row pos of the caches
    {   // threads past QH * HALF repeat the last element: the same values
        // to the same place
        const int h = i0 / HALF, d = i0 % HALF;
        qr[h][d] = qa0 * cs0.x - qb0 * cs0.y;
        qr[h][d + HALF] = qa0 * cs0.y + qb0 * cs0.x;
    }
    for (int i = t + kAThreads; i < QH * HALF; i += kAThreads) {
        const int h = i / HALF, d = i % HALF;
        const float *q = qkv + (size_t)(g * QH + h) * HD;
        const float2 cs = rp[d];
        const float a = q[d], b = q[d + HALF];
        qr[h][d] = a * cs.x - b * cs.y;
        qr[h][d + HALF] = a * cs.y + b * cs.x;
    }
    if (jn < kAP) {
        uint16_t *krow = kc + (gbase + jn) * HD;
        uint16_t *vrow = vc + (gbase + jn) * HD;
        if (t < HALF) {
            const uint16_t r0 = f2h(ka0 * csk.x - kb0 * csk.y);
            const uint16_t r1 = f2h(ka0 * csk.y + kb0 * csk.x);
            knew[t] = r0;
            knew[t + HALF] = r1;
            krow[t] = r0;
            krow[t + HALF] = r1;
        }
        if (t < HD) {
            const uint16_t r = f2h(v0);
            vnew[t] = r;
            vrow[t] = r;
        }
    }
    __syncthreads();

    // scores: four lanes per position, each a quarter of the head dimension
    {
        if (jj == jn) {
#pragma unroll
            for (int b = 0; b < KL; ++b)
                kreg[b] = *reinterpret_cast<const uint4 *>(knew + qq * QD + b * 8);
        }
        float acc[QH];
#pragma unroll
        for (int h = 0; h < QH; ++h)
            acc[h] = 0.0f;
#pragma unroll
        for (int b = 0; b < KL; ++b) {
            const int d0 = qq * QD + b * 8;
            float kf[8];
            unpack8(kreg[b], kf);
#pragma unroll
            for (int e = 0; e < 8; e += 2)
#pragma unroll
                for (int h = 0; h < QH; ++h)
                    acc[h] = fmaf(qr[h][d0 + e], kf[e], fmaf(qr[h][d0 + e + 1], kf[e + 1], acc[h]));
        }
        const float scale = 1.0f / sqrtf((float)HD);
#pragma unroll
        for (int h = 0; h < QH; ++h) {
            float v = acc[h];
            v += dpp<kQuadXor1>(v);
            v += dpp<kQuadXor2>(v);
            if (qq == 0)
                sc[h][jj] = v * scale;
        }
    }
    __syncthreads();

    // softmax over the chunk: one wave per head
    {
        const int w = t >> 6, lane = t & 63;
        for (int h = w; h < QH; h += NW) {
            const float s = lane < n ? sc[h][lane] : -INFINITY;
            const float m = wave_max(s);
            const float e = lane < n ? expf(s - m) : 0.0f;
            const float l = wave_sum(e);
            sc[h][lane] = e;
            if (lane == 0) {
                mx[h] = m;
                sm[h] = l;
            }
        }
    }
    __syncthreads();

    // weighted value sum: lane = (16-byte block of the row, position group);
    // rows past the context have weight 0 and zero values
    {
        float acc[QH][8];
#pragma unroll
        for (int h = 0; h < QH; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[h][e] = 0.0f;
#pragma unroll
        for (int i = 0; i < VL; ++i) {
            const int r = pg + i * PG;
            if (r == jn)
                vreg[i] = *reinterpret_cast<const uint4 *>(vnew + db * 8);
            float vf[8];
            unpack8(vreg[i], vf);
#pragma unroll
            for (int h = 0; h < QH; ++h) {
                const float p = sc[h][r];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[h][e] = fmaf(p, vf[e], acc[h][e]);
            }
        }
        // position groups of one wave (lanes DB, 2 DB, ... apart): half
        // rows for 8 blocks per row, then rows, then wave halves
#pragma unroll
        for (int h = 0; h < QH; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = acc[h][e];
                if (DB == 8)
                    x += dpp<kRowRor8>(x);
                const Rows16 r(x);
                x = fa(r.a) + fa(r.b);
                const Halves32 hh(x);
                acc[h][e] = fa(hh.a) + fa(hh.b);
            }
        const int w = t >> 6, lane = t & 63;
        if (lane < DB) {
#pragma unroll
            for (int h = 0; h < QH; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    vred[w][h][db * 8 + e] = acc[h][e];
        }
        __syncthreads();
        for (int i = t; i < QH * HD; i += kAThreads) {
            const int h = i / HD, d = i % HD;
            float s = 0.0f;
#pragma unroll
            for (int q = 0; q < NW; ++q)
                s += vred[q][h][d];
            pout[h * prow + d] = s;
        }
        if (t < QH) {
            pout[t * prow + HD] = mx[t];
            pout[t * prow + HD + 1] = sm[t];
        }
    }
}

// One workgroup per (query head, 64 dims of it) merges the chunk partials
// (chunk max m_c, chunk sum l_c, unnormalised o_c): o = sum_c o_c e^(m_c -
// M) / sum_c l_c e^(m_c - M), M the largest m_c.  Wave s merges chunks s,
// s + S, ... with a running maximum, U chunks per round, then the S waves
// merge through LDS.
constexpr int kCDims = 64;
template <int QH, int HD, bool BATCH>
__global__ void __launch_bounds__(kCThreads)
attn_combine(const float *__restrict__ part, const int32_t *__restrict__ pos_dev,
             int32_t nchunk, uint16_t *__restrict__ out) {
    constexpr int S = kCThreads / kCDims;
    static_assert(HD % kCDims == 0, "dims per workgroup");
    constexpr int U = 4;
    __shared__ float ored[S][kCDims];
    __shared__ float ms[S], ls[S];
    const int hq = blockIdx.x, t = threadIdx.x;
    const int d = blockIdx.y * kCDims + t % kCDims;
    // the wave index is the slice: every chunk index is wave-uniform, so
    // chunk max and sum come from scalar loads
    const int s = __builtin_amdgcn_readfirstlane(t / kCDims);
    const int g = hq / QH, h = hq % QH;
    const int col = BATCH ? (int)blockIdx.z : 0;
    if (BATCH) {
        part += (size_t)col * (gridDim.x / QH) * nchunk * QH * (HD + 2);
        out += (size_t)col * gridDim.x * HD;
    }
    // One token: attn_partial wrote every chunk, those past the position as
    // empty partials (max -inf, sum 0, o 0), whose merge changes nothing
    // bitwise (weight exp(-inf) = 0, rescale exp(0) = 1), so all nchunk are
    // read and the loads need not wait for the position word.  A batch reads
    // only its column's chunks.
    const int nc = BATCH ? min(nchunk, (*pos_dev + col) / kAP + 1) : nchunk;
    const size_t prow = (size_t)(HD + 2);
    const size_t cstride = (size_t)QH * prow;
    const float *base = part + ((size_t)g * nchunk * QH + h) * prow;
    float m = -INFINITY, l = 0.0f, o = 0.0f;
    for (int c1 = s; c1 < nc; c1 += S * U) {
        float mv[U], lv[U], ov[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = c1 + u * S;
            mv[u] = -INFINITY;
            lv[u] = 0.0f;
            ov[u] = 0.0f;
            if (cc < nc) {
                const float *pc = base + (size_t)cc * cstride;
                mv[u] = pc[HD];
                lv[u] = pc[HD + 1];
                ov[u] = pc[d];
            }
        }
        float mn = m;
#pragma unroll
        for (int u = 0; u < U; ++u)
            mn = fmaxf(mn, mv[u]);
        // an empty chunk (max -inf) has weight 0, and a running max of -inf
        // means l = o = 0: the guards keep -inf - -inf out of expf and give
        // the same bits as expf wherever that difference is defined
        const float r = m == -INFINITY ? 1.0f : expf(m - mn);
        l *= r;
        o *= r;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = mv[u] == -INFINITY ? 0.0f : expf(mv[u] - mn);
            l = fmaf(lv[u], w, l);
            o = fmaf(ov[u], w, o);
        }
        m = mn;
    }
    ored[s][t % kCDims] = o;
    if (t % kCDims == 0) {
        ms[s] = m;
        ls[s] = l;
    }
    __syncthreads();
    if (s == 0) {
        float M = ms[0];
#pragma unroll
        for (int q = 1; q < S; ++q)
            M = fmaxf(M, ms[q]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int q = 0; q < S; ++q) {
            const float w = expf(ms[q] - M);
            L = fmaf(ls[q], w, L);
            O = fmaf(ored[q][t], w, O);
        }
        out[(size_t)hq * HD + d] = f2h(O / L);
    }
}

// Key and value rows of a batch of token columns: column b (blockIdx.y) at
// position *pos_dev + b, key rotated, both rounded to binary16.
template <int HD>
__global__ void __launch_bounds__(HD / 2)
kv_append_batch(const float *__restrict__ qkv, uint16_t *__restrict__ kc,
                uint16_t *__restrict__ vc, const float2 *__restrict__ rope,
                const int32_t *__restrict__ pos_dev, int32_t max_ctx, int32_t H, int32_t Hkv) {
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
}

// Matrix-core attention tile: one workgroup per (key/value head, chunk of
// 64 positions) for all `batch` columns (column b at position *pos_dev + b;
// rows r = b * QH + h of the query matrix).  Scores S = Q K^T and outputs
// O = P V are v_mfma_f32_16x16x32_f16 products with fp32 accumulation; the
// fp32 queries and weights enter as two binary16 halves (x = hi + lo, hi =
// f16(x), lo = f16(x - hi)), so each product is two passes and agrees with
// an fp32 evaluation to about 2^-22 relative; keys and values are binary16
// already.  LDS: the K rows (row-major) and the V rows transposed (so both
// operands are 16-byte reads), the query halves, the scores/weights.  Every
// row comes from the caches: kv_append_batch stored the columns' rows
// first.  Used for draft batches; a single token takes attn_partial, whose
// loads overlap its arithmetic (this tile's fixed staging costs more there).
template <int QH, int HD>
__global__ void __launch_bounds__(kAThreads)
attn_tile_mfma(const float *__restrict__ qkv, const uint16_t *__restrict__ kc,
               const uint16_t *__restrict__ vc, const float2 *__restrict__ rope,
               const int32_t *__restrict__ pos_dev, int32_t max_ctx, int32_t H, int32_t Hkv,
               float *__restrict__ part, int32_t nchunk, int32_t batch) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int HALF = HD / 2;
    constexpr int HP = HD + 8;     // K tile / query row stride, halves
    constexpr int VP = kAP + 8;    // transposed V row stride, halves
    constexpr int SP = kAP + 4;    // score row stride, floats
    constexpr int KT = HD / 32;    // k tiles of the scores
    constexpr int DT = HD / 16;    // output column tiles
    constexpr int NW = kAThreads / 64;
    static_assert(HD == 64 || HD == 128, "head dimension");
    extern __shared__ __align__(16) unsigned char smem[];
    const int rows = batch * QH;
    const int RT = (rows + 15) / 16;
    const int RP = RT * 16;        // padded rows
    uint16_t *kt = reinterpret_cast<uint16_t *>(smem);                 // [64][HP]
    uint16_t *vt = kt + kAP * HP;                                      // [HD][VP]
    uint16_t *qh = vt + HD * VP;                                       // [RP][HP]
    uint16_t *ql = qh + RP * HP;                                       // [RP][HP]
    float *ps = reinterpret_cast<float *>(ql + RP * HP);               // [RP][SP]
    float *mrow = ps + RP * SP;                                        // [RP]
    float *lrow = mrow + RP;                                           // [RP]

    const int g = blockIdx.x, c = blockIdx.y;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int pos0 = *pos_dev;
    const int pmax = pos0 + batch - 1;
    const int c0 = c * kAP;
    const size_t prow = (size_t)(HD + 2);
    const size_t nqkv = (size_t)(H + 2 * Hkv) * HD;
    const size_t colstride = (size_t)Hkv * nchunk * QH * prow;
    if (c0 > pmax) {
        for (int i = t; i < rows * (HD + 2); i += kAThreads) {
            const int r = i / (HD + 2), e = i % (HD + 2);
            const int b = r / QH, h = r % QH;
            part[b * colstride + (((size_t)g * nchunk + c) * QH + h) * prow + e] =
                e == HD ? -INFINITY : 0.0f;
        }
        return;
    }
    const int nrow = min(kAP, pmax + 1 - c0);   // rows any column reads
    const size_t gbase = ((size_t)g * max_ctx + c0) * HD;

    // stage K (row-major) and V (transposed) of the chunk
    {
        constexpr int CPR = HD / 8;
        for (int i = t; i < kAP * CPR; i += kAThreads) {
            const int r = i / CPR, cb = i % CPR;
            uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
            if (r < nrow) {
                kv = *reinterpret_cast<const uint4 *>(kc + gbase + (size_t)r * HD + cb * 8);
                vv = *reinterpret_cast<const uint4 *>(vc + gbase + (size_t)r * HD + cb * 8);
            }
            *reinterpret_cast<uint4 *>(kt + r * HP + cb * 8) = kv;
            const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vt[(cb * 8 + 2 * e) * VP + r] = (uint16_t)(vw[e] & 0xFFFFu);
                vt[(cb * 8 + 2 * e + 1) * VP + r] = (uint16_t)(vw[e] >> 16);
            }
        }
    }
    // rotated queries as binary16 halves; padding rows are zero
    for (int i = t; i < RP * HALF; i += kAThreads) {
        const int r = i / HALF, d = i % HALF;
        float a0 = 0.0f, a1 = 0.0f;
        if (r < rows) {
            const int b = r / QH, h = r % QH;
            const float *q = qkv + (size_t)b * nqkv + (size_t)(g * QH + h) * HD;
            const float2 cs = rope[(size_t)(pos0 + b) * HALF + d];
            const float x = q[d], y = q[d + HALF];
            a0 = x * cs.x - y * cs.y;
            a1 = x * cs.y + y * cs.x;
        }
        const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1;
        qh[r * HP + d] = __builtin_bit_cast(uint16_t, h0);
        qh[r * HP + d + HALF] = __builtin_bit_cast(uint16_t, h1);
        ql[r * HP + d] = f2h(a0 - (float)h0);
        ql[r * HP + d + HALF] = f2h(a1 - (float)h1);
    }
    __syncthreads();

    // scores: wave w takes positions 16w .. 16w + 15 of every row tile
    const float scale = 1.0f / sqrtf((float)HD);
    const int li = lane & 15, lk = lane >> 4;
    for (int rt = 0; rt < RT; ++rt) {
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const int d0 = k * 32 + lk * 8;
            const h8 bk = *reinterpret_cast<const h8 *>(kt + (w * 16 + li) * HP + d0);
            const h8 ah = *reinterpret_cast<const h8 *>(qh + (rt * 16 + li) * HP + d0);
            const h8 al = *reinterpret_cast<const h8 *>(ql + (rt * 16 + li) * HP + d0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bk, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bk, acc, 0, 0, 0);
        }
        // lane holds rows rt*16 + 4*lk + e of position column w*16 + li
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rt * 16 + 4 * lk + e;
            const int j = w * 16 + li;
            const bool live = r < rows && c0 + j <= pos0 + r / QH;
            ps[r * SP + j] = live ? acc[e] * scale : -INFINITY;
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
        if (lane == 0) {
            mrow[r] = m;
            lrow[r] = l;
        }
    }
    __syncthreads();

    // outputs: wave w takes column tiles w, w + 4, ... of every row tile
    for (int dt = w; dt < DT; dt += NW) {
        for (int rt = 0; rt < RT; ++rt) {
            f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < kAP / 32; ++k) {
                const int j0 = k * 32 + lk * 8;
                const float *pr = ps + (rt * 16 + li) * SP + j0;
                const float4 p0 = *reinterpret_cast<const float4 *>(pr);
                const float4 p1 = *reinterpret_cast<const float4 *>(pr + 4);
                const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                h8 ph, pl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ph[e] = (_Float16)pv[e];
                    pl[e] = (_Float16)(pv[e] - (float)ph[e]);
                }
                const h8 bv = *reinterpret_cast<const h8 *>(vt + (dt * 16 + li) * VP + j0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bv, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, bv, acc, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = rt * 16 + 4 * lk + e;
                if (r < rows) {
                    const int b = r / QH, h = r % QH;
                    float *pout = part + b * colstride + (((size_t)g * nchunk + c) * QH + h) * prow;
                    pout[dt * 16 + li] = acc[e];
                }
            }
        }
    }
    for (int r = t; r < rows; r += kAThreads) {
        const int b = r / QH, h = r % QH;
        float *pout = part + b * colstride + (((size_t)g * nchunk + c) * QH + h) * prow;
        pout[HD] = mrow[r];
        pout[HD + 1] = lrow[r];
    }
}

size_t tile_mfma_lds(int qh, int hd, int batch) {
    const int rp = (batch * qh + 15) / 16 * 16;
    return (size_t)kAP * (hd + 8) * 2 + (size_t)hd * (kAP + 8) * 2 + 2 * (size_t)rp * (hd + 8) * 2 +
           (size_t)rp * (kAP + 4) * 4 + 2 * (size_t)rp * 4;
}

using AppendFn = void (*)(const float *, uint16_t *, uint16_t *, const float2 *, const int32_t *,
                          int32_t, int32_t, int32_t);

using PartialFn = void (*)(const float *, uint16_t *, uint16_t *, const float2 *,
                           const int32_t *, int32_t, int32_t, int32_t, float *, int32_t);
using CombineFn = void (*)(const float *, const int32_t *, int32_t, uint16_t *);

using TileFn = void (*)(const float *, const uint16_t *, const uint16_t *, const float2 *,
                        const int32_t *, int32_t, int32_t, int32_t, float *, int32_t, int32_t);

struct AttnFns {
    PartialFn partial = nullptr;
    CombineFn combine = nullptr;
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
    f.combine = batch ? attn_combine<QH, HD, true> : attn_combine<QH, HD, false>;
    f.append = kv_append_batch<HD>;
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
        hipLaunchKernelGGL(f.append, dim3((unsigned)a.Hkv, (unsigned)a.batch), dim3(a.hd / 2), 0,
                           s, a.qkv, a.kc, a.vc, static_cast<const float2 *>(a.rope), a.pos_dev,
                           a.max_ctx, a.H, a.Hkv);
        Q4_HIP(hipGetLastError());
        hipLaunchKernelGGL(f.tile, dim3((unsigned)a.Hkv, (unsigned)a.nchunk), dim3(kAThreads), lds,
                           s, a.qkv, a.kc, a.vc, static_cast<const float2 *>(a.rope), a.pos_dev,
                           a.max_ctx, a.H, a.Hkv, a.part, a.nchunk, a.batch);
    } else {
        hipLaunchKernelGGL(f.partial, dim3((unsigned)a.Hkv, (unsigned)a.nchunk), dim3(kAThreads),
                           0, s, a.qkv, a.kc, a.vc, static_cast<const float2 *>(a.rope),
                           a.pos_dev, a.max_ctx, a.H, a.Hkv, a.part, a.nchunk);
    }
    Q4_HIP(hipGetLastError());
    hipLaunchKernelGGL(f.combine, dim3((unsigned)a.H, (unsigned)(a.hd / kCDims), (unsigned)a.batch),
                       dim3(kCThreads), 0, s,
                       a.part, a.pos_dev, a.nchunk, a.out);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace q4
