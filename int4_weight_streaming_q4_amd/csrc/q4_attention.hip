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
//                 rotates the group's queries (angles in fp64), the chunk
//                 that holds the current position also rotates the new key
//                 and stores it and the new value into the caches; then
//                 scores, a softmax over the chunk and the weighted value
//                 sum, written as a partial (chunk max, chunk sum,
//                 unnormalised output).
//   attn_combine  one workgroup per query head: merges the partials of the
//                 chunks up to the current position and writes the
//                 binary16 attention output the O product reads.
// The position comes from a device word, so one captured graph serves every
// context length of its bucket: chunks past the position write an empty
// partial.
#include <cmath>

#include "q4_attention.h"

namespace q4 {
namespace {

constexpr int kAP = 64;        // positions per chunk
constexpr int kAThreads = 256;

__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__global__ void set_pos_kernel(int32_t *pos_dev, int32_t pos) { *pos_dev = pos; }

// QH query heads per key/value head, HD head dimension.
template <int QH, int HD>
__global__ void __launch_bounds__(kAThreads)
attn_partial(const float *__restrict__ qkv, uint16_t *__restrict__ kc, uint16_t *__restrict__ vc,
             const int32_t *__restrict__ pos_dev, int32_t max_ctx, int32_t H, int32_t Hkv,
             float rope_base, float *__restrict__ part, int32_t nchunk) {
    constexpr int HALF = HD / 2;
    constexpr int DB = HD / 8;                 // 16-byte blocks per head row
    constexpr int PG = kAThreads / DB;         // position groups in the value sum
    static_assert(HD % 32 == 0 && HD <= 256, "head dimension");
    static_assert(kAThreads % DB == 0, "value-sum layout");
    __shared__ float qr[QH][HD];               // rotated queries
    __shared__ float cs[HALF], sn[HALF];
    __shared__ __align__(16) uint16_t knew[HD];
    __shared__ __align__(16) uint16_t vnew[HD];
    __shared__ float sc[QH][kAP];              // scores, then weights
    __shared__ float mx[QH], sm[QH];

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
    const bool has_new = pos < c0 + kAP;

    // rotation angles of this position, in fp64 then rounded
    if (t < HALF) {
        const double inv = pow((double)rope_base, -2.0 * (double)t / (double)HD);
        const double ang = (double)pos * inv;
        cs[t] = (float)cos(ang);
        sn[t] = (float)sin(ang);
    }
    __syncthreads();
    for (int i = t; i < QH * HALF; i += kAThreads) {
        const int h = i / HALF, d = i % HALF;
        const float *q = qkv + (size_t)(g * QH + h) * HD;
        const float a = q[d], b = q[d + HALF];
        qr[h][d] = a * cs[d] - b * sn[d];
        qr[h][d + HALF] = a * sn[d] + b * cs[d];
    }
    if (has_new) {
        const float *k = qkv + (size_t)(H + g) * HD;
        const float *v = qkv + (size_t)(H + Hkv + g) * HD;
        uint16_t *krow = kc + ((size_t)g * max_ctx + pos) * HD;
        uint16_t *vrow = vc + ((size_t)g * max_ctx + pos) * HD;
        for (int d = t; d < HALF; d += kAThreads) {
            const float a = k[d], b = k[d + HALF];
            const uint16_t r0 = f2h(a * cs[d] - b * sn[d]);
            const uint16_t r1 = f2h(a * sn[d] + b * cs[d]);
            knew[d] = r0;
            knew[d + HALF] = r1;
            krow[d] = r0;
            krow[d + HALF] = r1;
        }
        for (int d = t; d < HD; d += kAThreads) {
            const uint16_t r = f2h(v[d]);
            vnew[d] = r;
            vrow[d] = r;
        }
    }
    __syncthreads();

    // scores: four lanes per position, each a quarter of the head dimension
    {
        constexpr int QD = HD / 4;
        const int jj = t >> 2, qq = t & 3;
        float acc[QH];
#pragma unroll
        for (int h = 0; h < QH; ++h)
            acc[h] = 0.0f;
        if (jj < n) {
            const int j = c0 + jj;
            const uint16_t *kr = (j == pos) ? knew : kc + ((size_t)g * max_ctx + j) * HD;
#pragma unroll
            for (int b = 0; b < QD / 8; ++b) {
                const int d0 = qq * QD + b * 8;
                const uint4 kv = *reinterpret_cast<const uint4 *>(kr + d0);
                const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float k0 = h2f((uint16_t)(w[e] & 0xFFFFu));
                    const float k1 = h2f((uint16_t)(w[e] >> 16));
#pragma unroll
                    for (int h = 0; h < QH; ++h)
                        acc[h] = fmaf(qr[h][d0 + 2 * e], k0, fmaf(qr[h][d0 + 2 * e + 1], k1, acc[h]));
                }
            }
        }
        const float scale = 1.0f / sqrtf((float)HD);
#pragma unroll
        for (int h = 0; h < QH; ++h) {
            float v = acc[h];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            if (qq == 0 && jj < kAP)
                sc[h][jj] = v * scale;
        }
    }
    __syncthreads();

    // softmax over the chunk: one wave per head
    {
        const int w = t >> 6, lane = t & 63;
        for (int h = w; h < QH; h += kAThreads / 64) {
            const float s = lane < n ? sc[h][lane] : -INFINITY;
            float m = s;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1)
                m = fmaxf(m, __shfl_xor(m, o));
            const float e = lane < n ? expf(s - m) : 0.0f;
            float l = e;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1)
                l += __shfl_xor(l, o);
            sc[h][lane] = e;
            if (lane == 0) {
                mx[h] = m;
                sm[h] = l;
            }
        }
    }
    __syncthreads();

    // weighted value sum: thread = (16-byte block of the row, position group)
    {
        const int db = t % DB, pg = t / DB;
        float acc[QH][8];
#pragma unroll
        for (int h = 0; h < QH; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[h][e] = 0.0f;
        for (int jj = pg; jj < n; jj += PG) {
            const int j = c0 + jj;
            const uint16_t *vr = (j == pos) ? vnew : vc + ((size_t)g * max_ctx + j) * HD;
            const uint4 vv = *reinterpret_cast<const uint4 *>(vr + db * 8);
            const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
            float vf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vf[2 * e] = h2f((uint16_t)(w[e] & 0xFFFFu));
                vf[2 * e + 1] = h2f((uint16_t)(w[e] >> 16));
            }
#pragma unroll
            for (int h = 0; h < QH; ++h) {
                const float p = sc[h][jj];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[h][e] = fmaf(p, vf[e], acc[h][e]);
            }
        }
        // reduce over the position groups through LDS, in a fixed order
        __shared__ float vred[PG][QH][8 * DB];
#pragma unroll
        for (int h = 0; h < QH; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                vred[pg][h][db * 8 + e] = acc[h][e];
        __syncthreads();
        for (int i = t; i < QH * HD; i += kAThreads) {
            const int h = i / HD, d = i % HD;
            float s = 0.0f;
            for (int q = 0; q < PG; ++q)
                s += vred[q][h][d];
            pout[h * prow + d] = s;
        }
        if (t < QH) {
            pout[t * prow + HD] = mx[t];
            pout[t * prow + HD + 1] = sm[t];
        }
    }
}

// One workgroup per query head: merges the chunk partials.
template <int QH, int HD>
__global__ void __launch_bounds__(HD)
attn_combine(const float *__restrict__ part, const int32_t *__restrict__ pos_dev,
             int32_t nchunk, uint16_t *__restrict__ out) {
    const int hq = blockIdx.x, d = threadIdx.x;
    const int g = hq / QH, h = hq % QH;
    const int pos = *pos_dev;
    const int last = min(nchunk - 1, pos / kAP);
    const size_t prow = (size_t)(HD + 2);
    const float *base = part + ((size_t)g * nchunk * QH + h) * prow;
    float M = -INFINITY;
    for (int c = 0; c <= last; ++c)
        M = fmaxf(M, base[(size_t)c * QH * prow + HD]);
    float L = 0.0f, o = 0.0f;
    for (int c = 0; c <= last; ++c) {
        const float *pc = base + (size_t)c * QH * prow;
        const float w = expf(pc[HD] - M);
        L = fmaf(pc[HD + 1], w, L);
        o = fmaf(pc[d], w, o);
    }
    out[(size_t)hq * HD + d] = f2h(o / L);
}

using PartialFn = void (*)(const float *, uint16_t *, uint16_t *, const int32_t *, int32_t,
                           int32_t, int32_t, float, float *, int32_t);
using CombineFn = void (*)(const float *, const int32_t *, int32_t, uint16_t *);

template <int QH, int HD>
bool pick(int qh, int hd, PartialFn &p, CombineFn &c) {
    if (qh != QH || hd != HD)
        return false;
    p = attn_partial<QH, HD>;
    c = attn_combine<QH, HD>;
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

q4_status launch_set_pos(int32_t *pos_dev, int32_t pos, hipStream_t s) {
    hipLaunchKernelGGL(set_pos_kernel, dim3(1), dim3(1), 0, s, pos_dev, pos);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

q4_status launch_attention(const AttnArgs &a, hipStream_t s) {
    PartialFn pf = nullptr;
    CombineFn cf = nullptr;
    const int qh = a.H / a.Hkv;
    if (!(pick<1, 64>(qh, a.hd, pf, cf) || pick<2, 64>(qh, a.hd, pf, cf) ||
          pick<4, 64>(qh, a.hd, pf, cf) || pick<8, 64>(qh, a.hd, pf, cf) ||
          pick<1, 128>(qh, a.hd, pf, cf) || pick<2, 128>(qh, a.hd, pf, cf) ||
          pick<4, 128>(qh, a.hd, pf, cf) || pick<8, 128>(qh, a.hd, pf, cf)))
        return fail(Q4_ERR_UNSUPPORTED, "attention: %d query heads per group, head dim %d", qh,
                    a.hd);
    if (a.nchunk < 1 || a.nchunk * kAP > a.max_ctx + kAP - 1)
        return fail(Q4_ERR_INVALID_ARG, "attention: %d chunks for max_ctx %d", a.nchunk,
                    a.max_ctx);
    hipLaunchKernelGGL(pf, dim3((unsigned)a.Hkv, (unsigned)a.nchunk), dim3(kAThreads), 0, s,
                       a.qkv, a.kc, a.vc, a.pos_dev, a.max_ctx, a.H, a.Hkv, a.rope_base, a.part,
                       a.nchunk);
    Q4_HIP(hipGetLastError());
    hipLaunchKernelGGL(cf, dim3((unsigned)a.H), dim3((unsigned)a.hd), 0, s, a.part, a.pos_dev,
                       a.nchunk, a.out);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace q4
