// Device code of the INT4 product, shared by the standalone product kernel
// (q4_gemv.hip) and the persistent decode kernel (q4_persistent.hip).
//
// Operation: PIPO: Pipelined Offloading for Efficient Inference on Consumer
// Devices, "Method", bullet "Computation optimization" -- the vector is
// multiplied directly by the 4-bit weights; no dequantized matrix is ever
// written.  The decomposition and unpack are described in q4_gemv.hip.
#pragma once

#include "q4_internal.h"
#include "q4_lanes.h"

namespace q4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlots = 4; // 16-lane rows per wave

__device__ __forceinline__ half2_t as_h2(uint32_t v) {
    return __builtin_bit_cast(half2_t, v);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total
// (the adds are commutative pairs, so all lanes hold the same bits).
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);  // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);  // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v); // row_half_mirror
    v += dpp_f<0x140>(v); // row_mirror
    return v;
}

// A loop-invariant constant held in a VGPR.  gfx9 VOP3 instructions take no
// literal and at most one SGPR, so `(v & mask) | bias` fuses into one
// v_and_or_b32 only when one of the two constants sits in a VGPR.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
    return r;
}

// One chunk (32 codes, 16 bytes) against its 32 permuted activations.
__device__ __forceinline__ float chunk_acc(uint4 w, const uint4 (&xq)[4], float s,
                                           float acc, uint32_t bias) {
    const half2_t off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2_t off_hi = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    float tlo = 0.0f, thi = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t v = wd[i];
        const uint32_t u = v >> 8;
        half2_t a = as_h2((v & 0x000F000Fu) | bias) - off_lo;
        half2_t b = as_h2((v & 0x00F000F0u) | bias) - off_hi;
        half2_t c = as_h2((u & 0x000F000Fu) | bias) - off_lo;
        half2_t d = as_h2((u & 0x00F000F0u) | bias) - off_hi;
        tlo = __builtin_amdgcn_fdot2(a, as_h2(xq[i].x), tlo, false);
        thi = __builtin_amdgcn_fdot2(b, as_h2(xq[i].y), thi, false);
        tlo = __builtin_amdgcn_fdot2(c, as_h2(xq[i].z), tlo, false);
        thi = __builtin_amdgcn_fdot2(d, as_h2(xq[i].w), thi, false);
    }
    return fmaf(s, fmaf(thi, 0.0625f, tlo), acc);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <Epi E, int R>
__device__ __forceinline__ int64_t row_of(int64_t unit, int r, const EpiArgs &ea) {
    if constexpr (E == Epi::SiluPair)
        return unit + r * ea.pair_off;
    else
        return unit * R + r;
}

// Activation accesses.  COH = false: ordinary loads and stores (one kernel
// per product; the kernel boundary publishes the data).  COH = true: the
// persistent kernels, where workgroups on different XCDs exchange the small
// activation vectors inside one launch: every store and every load of such
// a vector is an agent-scope atomic access, which goes to the coherence
// point instead of an XCD's own L2, so no cache writeback or invalidation
// is needed at the grid barriers (each of those is a whole-L2 operation).
template <bool COH>
__device__ __forceinline__ uint4 act_load16(const void *p) {
    if constexpr (COH) {
        const uint64_t *q = static_cast<const uint64_t *>(p);
        const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return uint4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
    } else {
        return gload16(p);
    }
}

template <bool COH>
__device__ __forceinline__ void act_store16(void *p, uint4 v) {
    if constexpr (COH) {
        uint64_t *q = static_cast<uint64_t *>(p);
        __hip_atomic_store(q, (uint64_t)v.x | ((uint64_t)v.y << 32), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q + 1, (uint64_t)v.z | ((uint64_t)v.w << 32), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *static_cast<uint4 *>(p) = v;
    }
}

template <bool COH>
__device__ __forceinline__ float act_load_f32(const float *p) {
    if constexpr (COH)
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        return gload(p);
}

template <bool COH>
__device__ __forceinline__ void act_store_f32(float *p, float v) {
    if constexpr (COH)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

template <bool COH>
__device__ __forceinline__ void act_store_u16(uint16_t *p, uint16_t v) {
    if constexpr (COH)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

// 8 binary16 values in natural order -> the four activation pairs in unpack
// order: (x0,x4), (x1,x5), (x2,x6), (x3,x7).
__device__ __forceinline__ uint4 permute8(uint4 v) {
    uint4 o;
    o.x = (v.x & 0xFFFFu) | (v.z << 16);
    o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    o.z = (v.y & 0xFFFFu) | (v.w << 16);
    o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return o;
}

// Stage x (binary16, K values) into LDS as xs[p * C + c] = the four
// activation pairs of 8-block p of chunk c, in unpack order.
template <bool COH>
__device__ __forceinline__ void stage_x(const uint16_t *__restrict__ x16, uint4 *xs, int K) {
    const int C = K >> 5;
    for (int b = threadIdx.x; b < (K >> 3); b += kThreads)
        xs[(b & 3) * C + (b >> 2)] = permute8(act_load16<COH>(x16 + 8 * (size_t)b));
}

__device__ __forceinline__ float eps_of(const EpiArgs &ea) { return ea.eps; }

// Sum over the 64 lanes of a wave; every lane gets the total.  After the
// row sums, the rows pair up as with lane xor 16 and the half-waves as with
// lane xor 32, through gfx950's row and half-wave swaps (VALU operations,
// not LDS permutes); each add takes the same two operands either way, so
// the bits are those of the xor form.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    const lanes::Rows16 r(v);
    v = lanes::fa(r.a) + lanes::fa(r.b);
    const lanes::Halves32 h(v);
    return lanes::fa(h.a) + lanes::fa(h.b);
}

template <bool COH>
__device__ __forceinline__ void load_f32x8(const float *p, float (&f)[8]) {
    const uint4 lo = act_load16<COH>(p);
    const uint4 hi = act_load16<COH>(p + 4);
    f[0] = __uint_as_float(lo.x);
    f[1] = __uint_as_float(lo.y);
    f[2] = __uint_as_float(lo.z);
    f[3] = __uint_as_float(lo.w);
    f[4] = __uint_as_float(hi.x);
    f[5] = __uint_as_float(hi.y);
    f[6] = __uint_as_float(hi.z);
    f[7] = __uint_as_float(hi.w);
}

// Stage a = f16(h / sqrt(mean(h^2) + eps)) (RMSNorm with unit gain) from the
// fp32 residual h.  Every workgroup computes the same sum in the same order,
// so all of them stage identical bits.  Workgroup 0 also writes `a` (natural
// order) to norm_out when given.
template <bool COH>
__device__ __forceinline__ void stage_rmsnorm(const float *__restrict__ h, uint4 *xs, int K,
                                              float eps, uint16_t *norm_out, float *wsum) {
    // Up to kKeep 8-value blocks per thread stay in registers between the
    // sum of squares and the scaling (K <= 8192 with 256 threads); larger K
    // rereads the rest.
    constexpr int kKeep = 4;
    const int C = K >> 5;
    const int nb8 = K >> 3;
    float keep[kKeep][8];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < kKeep; ++j) {
        const int b = threadIdx.x + j * kThreads;
        if (b < nb8) {
            load_f32x8<COH>(h + 8 * (size_t)b, keep[j]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ss = fmaf(keep[j][i], keep[j][i], ss);
        }
    }
    for (int b = threadIdx.x + kKeep * kThreads; b < nb8; b += kThreads) {
        float f[8];
        load_f32x8<COH>(h + 8 * (size_t)b, f);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ss = fmaf(f[i], f[i], ss);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0)
        wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = wsum[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        tot += wsum[w];
    const float r = 1.0f / sqrtf(tot / (float)K + eps);
    auto emit = [&](int b, const float (&f)[8]) {
        uint32_t p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            p[i] = (uint32_t)f32_to_f16(f[2 * i] * r) |
                   ((uint32_t)f32_to_f16(f[2 * i + 1] * r) << 16);
        const uint4 v = {p[0], p[1], p[2], p[3]};
        xs[(b & 3) * C + (b >> 2)] = permute8(v);
        if (norm_out && blockIdx.x == 0)
            act_store16<COH>(norm_out + 8 * (size_t)b, v);
    };
#pragma unroll
    for (int j = 0; j < kKeep; ++j) {
        const int b = threadIdx.x + j * kThreads;
        if (b < nb8)
            emit(b, keep[j]);
    }
    for (int b = threadIdx.x + kKeep * kThreads; b < nb8; b += kThreads) {
        float f[8];
        load_f32x8<COH>(h + 8 * (size_t)b, f);
        emit(b, f);
    }
}

// Two-step staging.  Loads of one wave return in issue order, so activation
// loads issued after a batch of weight loads would wait for that batch: the
// activation is therefore loaded first (stage_issue, up to kXR 16-byte
// values per thread held in registers), the weight prefetch goes out next,
// and stage_finish then reduces, normalises, permutes and writes LDS.
constexpr int kXR = 8;

struct XStage {
    uint4 v[kXR];
};

// Every thread issues all kXR loads (indices past the end wrap around to
// blocks other threads load anyway -- one common address for all of them
// would queue the whole grid on one cache channel; stage_finish ignores
// them): a load under a per-lane branch would make the compiler wait for
// every load in flight, the weight prefetch included, before the first use
// of the activation.
// The RMSNorm prologue (UNIFORM) skips the rows of blocks past the end on a
// workgroup-uniform test instead (issuing them all made its products slower:
// gate+up 15.05 vs 14.55 us, QKV 7.06 vs 6.88); without UNIFORM it skips
// them per lane, so the staging waits for the first weight batch as well,
// which measured faster for the paired gate+up rows (14.47 vs 15.45 us).
template <Pro P, bool COH, bool UNIFORM = true>
__device__ __forceinline__ void stage_issue(const void *xin, int K, XStage &st) {
    if constexpr (P == Pro::F16) {
        const uint16_t *x16 = static_cast<const uint16_t *>(xin);
        const int nb = K >> 3;
#pragma unroll
        for (int j = 0; j < kXR; ++j) {
            const int b = threadIdx.x + j * kThreads;
            st.v[j] = act_load16<COH>(x16 + 8 * (size_t)(b < nb ? b : b % nb));
        }
    } else {
        const float *h = static_cast<const float *>(xin);
        const int nb8 = K >> 3;
#pragma unroll
        for (int j = 0; j < kXR / 2; ++j) {
            // UNIFORM: a workgroup-uniform bound (the whole group loads block
            // row j or none of it; the last threads of a partial row wrap
            // around), so no load sits behind a per-lane branch
            const int b = threadIdx.x + j * kThreads;
            if (UNIFORM ? j * kThreads < nb8 : b < nb8) {
                const size_t o = 8 * (size_t)(b < nb8 ? b : b % nb8);
                st.v[2 * j] = act_load16<COH>(h + o);
                st.v[2 * j + 1] = act_load16<COH>(h + o + 4);
            } else {
                st.v[2 * j] = st.v[2 * j + 1] = uint4{0u, 0u, 0u, 0u};
            }
        }
    }
}

__device__ __forceinline__ void unpack_f32x8(const uint4 &lo, const uint4 &hi, float (&f)[8]) {
    f[0] = __uint_as_float(lo.x);
    f[1] = __uint_as_float(lo.y);
    f[2] = __uint_as_float(lo.z);
    f[3] = __uint_as_float(lo.w);
    f[4] = __uint_as_float(hi.x);
    f[5] = __uint_as_float(hi.y);
    f[6] = __uint_as_float(hi.z);
    f[7] = __uint_as_float(hi.w);
}

template <Pro P, bool COH>
__device__ __forceinline__ void stage_finish(const void *xin, uint4 *xs, int K, const EpiArgs &ea,
                                             float *wsum, const XStage &st) {
    const int C = K >> 5;
    if constexpr (P == Pro::F16) {
        const uint16_t *x16 = static_cast<const uint16_t *>(xin);
        const int nb = K >> 3;
#pragma unroll
        for (int j = 0; j < kXR; ++j) {
            const int b = threadIdx.x + j * kThreads;
            if (b < nb)
                xs[(b & 3) * C + (b >> 2)] = permute8(st.v[j]);
        }
        for (int b = threadIdx.x + kXR * kThreads; b < nb; b += kThreads)
            xs[(b & 3) * C + (b >> 2)] = permute8(act_load16<COH>(x16 + 8 * (size_t)b));
    } else {
        // a = f16(h / sqrt(mean(h^2) + eps)), unit gain; every workgroup sums
        // in the same order, so all stage identical bits.
        const float *h = static_cast<const float *>(xin);
        const int nb8 = K >> 3;
        constexpr int kKeep = kXR / 2;
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < kKeep; ++j) {
            if (threadIdx.x + j * kThreads < nb8) {
                float f[8];
                unpack_f32x8(st.v[2 * j], st.v[2 * j + 1], f);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    ss = fmaf(f[i], f[i], ss);
            }
        }
        for (int b = threadIdx.x + kKeep * kThreads; b < nb8; b += kThreads) {
            float f[8];
            load_f32x8<COH>(h + 8 * (size_t)b, f);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ss = fmaf(f[i], f[i], ss);
        }
        ss = wave_sum(ss);
        if ((threadIdx.x & 63) == 0)
            wsum[threadIdx.x >> 6] = ss;
        __syncthreads();
        float tot = wsum[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            tot += wsum[w];
        const float r = 1.0f / sqrtf(tot / (float)K + eps_of(ea));
        auto emit = [&](int b, const float (&f)[8]) {
            uint32_t p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p[i] = (uint32_t)f32_to_f16(f[2 * i] * r) |
                       ((uint32_t)f32_to_f16(f[2 * i + 1] * r) << 16);
            const uint4 v = {p[0], p[1], p[2], p[3]};
            xs[(b & 3) * C + (b >> 2)] = permute8(v);
            if (ea.norm_out && blockIdx.x == 0)
                act_store16<COH>(ea.norm_out + 8 * (size_t)b, v);
        };
#pragma unroll
        for (int j = 0; j < kKeep; ++j) {
            const int b = threadIdx.x + j * kThreads;
            if (b < nb8) {
                float f[8];
                unpack_f32x8(st.v[2 * j], st.v[2 * j + 1], f);
                emit(b, f);
            }
        }
        for (int b = threadIdx.x + kKeep * kThreads; b < nb8; b += kThreads) {
            float f[8];
            load_f32x8<COH>(h + 8 * (size_t)b, f);
            emit(b, f);
        }
    }
}

// Weight loads: each byte is read exactly once per call, so NT marks them
// non-temporal (streamed past the caches' retention policy).
template <bool NT>
__device__ __forceinline__ uint4 wload16(const void *p) {
    if constexpr (NT) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        typedef const __attribute__((address_space(1))) u32x4 global_t;
        const u32x4 v = __builtin_nontemporal_load((global_t *)p);
        return uint4{v.x, v.y, v.z, v.w};
    } else {
        return gload16(p);
    }
}

template <bool NT>
__device__ __forceinline__ uint16_t wload2(const uint16_t *p) {
    if constexpr (NT) {
        typedef const __attribute__((address_space(1))) uint16_t global_t;
        return __builtin_nontemporal_load((global_t *)p);
    } else {
        return gload(p);
    }
}

// Loads of one group of U chunks of R rows.  ALL: every load is issued,
// chunks past this lane's count loading the lane's last chunk again (or its
// row's first chunk when it has none) and never used -- for the first batch
// of a product, so that the wait before the activation staging covers only
// the activation loads (a load behind a per-lane branch makes the next wait
// cover every load in flight).  Otherwise chunks past the count are skipped
// (in the steady loop, issuing them all lets the compiler reuse in-flight
// loads' address registers as destinations and wait inside the issue
// sequence).
template <int U, int R, bool NT, bool ALL = false>
__device__ __forceinline__ void load_chunks(uint4 (&w)[U][R], uint16_t (&s)[U][R],
                                            const uint8_t *const (&wp)[R],
                                            const uint16_t *const (&sp)[R], int first, int nl,
                                            int cstep) {
    const int last = nl > 0 ? nl - 1 : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool ok = first + u < nl;
        const int c = ok ? first + u : last;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (ALL || ok) {
                w[u][r] = wload16<NT>(wp[r] + (size_t)c * cstep * 16);
                s[u][r] = wload2<NT>(sp[r] + (size_t)c * cstep);
            } else {
                w[u][r] = uint4{0u, 0u, 0u, 0u};
                s[u][r] = 0;
            }
        }
    }
}

template <Epi E, int R, int KS>
struct Geometry {
    static constexpr int kRowGroups = kWaves / KS;
    static constexpr int kUnitsPerBlock = kRowGroups * kSlots;
};

// Points wp/sp at this lane's first chunk of the R rows of row block `blk`
// (units past the end use the last unit; a lane with no chunk in its row,
// cfirst >= C, points at the row's last chunk, which it loads but never
// uses, so every address stays inside the matrix).
template <int R, int KS, Epi E>
__device__ __forceinline__ void setup_rows(const uint8_t *W, const uint16_t *S, int64_t N, int C,
                                           int64_t n_units, const EpiArgs &ea, int64_t blk,
                                           const uint8_t *(&wp)[R], const uint16_t *(&sp)[R]) {
    constexpr int kUnitsPerBlock = Geometry<E, R, KS>::kUnitsPerBlock;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slot = lane >> 4;
    const int rgroup = wave / KS;
    const int cf = (wave % KS) * 16 + (lane & 15);
    const int cfirst = cf < C ? cf : C - 1;
    const int64_t unit = blk * kUnitsPerBlock + rgroup * kSlots + slot;
    const int64_t lunit = unit < n_units ? unit : n_units - 1;
    const size_t row_bytes = (size_t)(C * 16);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int64_t row = row_of<E, R>(lunit, r, ea);
        row = row < N ? row : N - 1;
        wp[r] = W + (size_t)row * row_bytes + (size_t)cfirst * 16;
        sp[r] = S + (size_t)row * C + cfirst;
    }
}

// Number of row blocks of a product and this lane's chunk count.
template <int R, int KS, Epi E>
__device__ __forceinline__ int64_t row_blocks(int64_t n_units) {
    constexpr int kUnitsPerBlock = Geometry<E, R, KS>::kUnitsPerBlock;
    return (n_units + kUnitsPerBlock - 1) / kUnitsPerBlock;
}

template <int KS>
__device__ __forceinline__ int lane_chunks(int C) {
    const int cstep = 16 * KS;
    const int cfirst = ((threadIdx.x >> 6) % KS) * 16 + (threadIdx.x & 15);
    return cfirst < C ? (C - cfirst + cstep - 1) / cstep : 0;
}

// Issues the first chunk loads of row block `blk`.  GUARD: skip them when
// the block does not exist (the persistent kernels prefetch a product whose
// row blocks may be fewer than the workgroups), and skip chunks past a
// lane's count per lane; without GUARD (the per-product kernels, which
// launch at most one workgroup per row block) every load is issued, so the
// staging that follows waits only for the activation.
template <int R, int KS, int U, bool NT, Epi E, bool GUARD = true>
__device__ __forceinline__ void prefetch_block(const uint8_t *W, const uint16_t *S, int64_t N,
                                               int K, int64_t n_units, const EpiArgs &ea,
                                               int64_t blk, uint4 (&w)[U][R],
                                               uint16_t (&s)[U][R], const uint8_t *(&wp)[R],
                                               const uint16_t *(&sp)[R]) {
    const int C = K >> 5;
    if (!GUARD || blk < row_blocks<R, KS, E>(n_units)) {
        setup_rows<R, KS, E>(W, S, N, C, n_units, ea, blk, wp, sp);
        load_chunks<U, R, NT, !GUARD>(w, s, wp, sp, 0, lane_chunks<KS>(C), 16 * KS);
    }
}

// Sums a row's partials over its 16 lanes and then over the KS waves that
// split its k range (LDS, fixed order).  Afterwards lane 0 of each slot of
// the first wave of a row group holds the row totals.  KS > 1 synchronises
// the workgroup twice, so every thread must call it.
template <int R, int KS>
__device__ __forceinline__ void reduce_rows(float (&acc)[R], float (*red)[kSlots][R]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sl = lane & 15;
    const int slot = lane >> 4;
    const int kpart = wave % KS;
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = row16_sum(acc[r]);
    if constexpr (KS > 1) {
        if (sl == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                red[wave][slot][r] = acc[r];
        }
        __syncthreads();
        if (kpart == 0 && sl == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float t = red[wave][slot][r];
                for (int k = 1; k < KS; ++k)
                    t += red[wave + k][slot][r];
                acc[r] = t;
            }
        }
        __syncthreads();
    }
}

// Writes the totals of output unit `unit` (lane 0 of its slot in the first
// wave of the row group) through the epilogue E.
template <int R, int KS, Epi E, bool COH>
__device__ __forceinline__ void store_unit(const float (&acc)[R], int64_t unit, int64_t N,
                                           int64_t n_units, const EpiArgs &ea) {
    const int lane = threadIdx.x & 63;
    const int kpart = (threadIdx.x >> 6) % KS;
    if (kpart == 0 && (lane & 15) == 0 && unit < n_units) {
        if constexpr (E == Epi::SiluPair) {
            static_assert(R == 2, "paired rows need two rows per slot");
            const float g = acc[0], up = acc[1];
            const float silu = g / (1.0f + expf(-g));
            act_store_u16<COH>(ea.out16 + unit, f32_to_f16(silu * up));
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t row = unit * R + r;
                if (row < N) {
                    if constexpr (E == Epi::Residual) {
                        act_store_f32<COH>(ea.y + row, act_load_f32<COH>(ea.y + row) + acc[r]);
                    } else {
                        act_store_f32<COH>(ea.y + row, acc[r]);
                        if constexpr (E == Epi::QkvGather) {
                            if (row >= ea.v_off) {
                                const int64_t v = row - ea.v_off;
                                const int64_t g = v / ea.hd, i = v % ea.hd;
                                const uint16_t h16 = f32_to_f16(acc[r]);
                                for (int q = 0; q < ea.group; ++q)
                                    act_store_u16<COH>(
                                        ea.out16 + (g * ea.group + q) * ea.hd + i, h16);
                            }
                        }
                    }
                }
            }
        }
    }
}

// Residual epilogue with the rows' old values already loaded (hv): the same
// sum as store_unit's h[row] + acc.
template <int R, int KS>
__device__ __forceinline__ void store_residual(const float (&acc)[R], const float (&hv)[R],
                                               int64_t unit, int64_t N, int64_t n_units,
                                               const EpiArgs &ea) {
    const int lane = threadIdx.x & 63;
    const int kpart = (threadIdx.x >> 6) % KS;
    if (kpart == 0 && (lane & 15) == 0 && unit < n_units) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = unit * R + r;
            if (row < N)
                ea.y[row] = hv[r] + acc[r];
        }
    }
}

// Loads the residual values of this lane's rows in row block blk (rows past
// the end read row N - 1; every lane loads, so no load sits behind a
// branch).
template <int R, int KS, Epi E>
__device__ __forceinline__ void load_residual(const EpiArgs &ea, int64_t N, int64_t blk,
                                              float (&hv)[R]) {
    constexpr int kUnitsPerBlock = Geometry<E, R, KS>::kUnitsPerBlock;
    const int wave = threadIdx.x >> 6;
    const int64_t unit = blk * kUnitsPerBlock + (wave / KS) * kSlots + ((threadIdx.x & 63) >> 4);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = unit * R + r;
        hv[r] = gload(ea.y + (row < N ? row : N - 1));
    }
}

// Processes row blocks blk, blk + stride, ... of one product with the
// activation already staged in LDS.  Precondition: the first chunk loads of
// `blk` are in w/s (prefetch_block), and, for the Residual epilogue of the
// per-product kernels (COH false), hv holds the old values of blk's rows
// (load_residual).  Every thread of the workgroup must call this (the
// k-split reduction synchronises the workgroup).
template <int R, int KS, int U, bool NT, Epi E, bool COH = false>
__device__ __forceinline__ void run_units(const uint8_t *W, const uint16_t *S, int64_t N, int K,
                                          int64_t n_units, const EpiArgs &ea, int64_t blk,
                                          int64_t stride, const uint4 *xs,
                                          float (*red)[kSlots][R], uint4 (&w)[U][R],
                                          uint16_t (&s)[U][R], const uint8_t *(&wp)[R],
                                          const uint16_t *(&sp)[R], uint32_t bias,
                                          float (&hv)[R]) {
    constexpr int kUnitsPerBlock = Geometry<E, R, KS>::kUnitsPerBlock;
    const int C = K >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sl = lane & 15;
    const int slot = lane >> 4;
    const int rgroup = wave / KS;
    const int kpart = wave % KS;
    const int64_t nblk = row_blocks<R, KS, E>(n_units);
    const int cstep = 16 * KS;
    const int cfirst = kpart * 16 + sl;
    const int nl = lane_chunks<KS>(C);
    const int niter = (nl + U - 1) / U;
    // Residual epilogue, one kernel per product: the rows' old values are
    // loaded ahead of the row block's weights instead of after the multiply
    // (a kernel starts with cold caches, so that read would cost a full
    // memory round trip at the end of every block).  The persistent kernels
    // keep the late read.
    constexpr bool kEarlyRes = E == Epi::Residual && !COH;

    for (; blk < nblk; blk += stride) {
        const int64_t unit = blk * kUnitsPerBlock + rgroup * kSlots + slot;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = 0.0f;

        for (int it = 0; it < niter; ++it) {
            if (it > 0)
                load_chunks<U, R, NT>(w, s, wp, sp, it * U, nl, cstep);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = it * U + u;
                if (j < nl) {
                    uint4 xq[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        xq[p] = xs[p * C + cfirst + j * cstep];
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[r] = chunk_acc(w[u][r], xq, f16_to_f32(s[u][r]), acc[r], bias);
                }
            }
        }
        reduce_rows<R, KS>(acc, red);

        // The next row block's first loads go out before this epilogue.
        float hcur[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            hcur[r] = hv[r];
        if (blk + stride < nblk) {
            if constexpr (kEarlyRes)
                load_residual<R, KS, E>(ea, N, blk + stride, hv);
            setup_rows<R, KS, E>(W, S, N, C, n_units, ea, blk + stride, wp, sp);
            load_chunks<U, R, NT>(w, s, wp, sp, 0, nl, cstep);
        }
        if constexpr (kEarlyRes)
            store_residual<R, KS>(acc, hcur, unit, N, n_units, ea);
        else
            store_unit<R, KS, E, COH>(acc, unit, N, n_units, ea);
    }
}

// ------------------------------------------------ software-pipelined loop
// The same products with every lane's chunk loads kept in flight across row
// blocks: two register buffers of U chunks x R rows alternate, and the loads
// of batch q + 2 are issued as soon as batch q has been multiplied, so one
// batch is always on its way while the other is in use.  A batch is U chunks
// of one row block; with C = K / 32 chunks per row, a row block is
// C / (16 KS U) batches.  Requires C % (16 KS U) == 0 (every lane then has
// the same chunk count and no chunk is out of range) and at least one row
// block per workgroup.  Chunks are accumulated in the same order as
// run_units, so both give bitwise-equal results for the same KS.
//
// Scales are held one per 32-bit register: two binary16 scales packed into
// one register would make the wave wait for a batch right after issuing it.
template <int R, int KS, int U, bool NT, Epi E>
__device__ __forceinline__ void load_batch(const uint8_t *W, const uint16_t *S, int64_t N, int C,
                                           int64_t n_units, const EpiArgs &ea, int64_t blk,
                                           int it, uint4 (&w)[U][R], uint32_t (&s)[U][R]) {
    const uint8_t *wp[R];
    const uint16_t *sp[R];
    setup_rows<R, KS, E>(W, S, N, C, n_units, ea, blk, wp, sp);
    const size_t c0 = (size_t)it * U * 16 * KS;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            w[u][r] = wload16<NT>(wp[r] + (c0 + (size_t)u * 16 * KS) * 16);
            s[u][r] = wload2<NT>(sp[r] + c0 + (size_t)u * 16 * KS);
        }
    }
}

template <int R, int KS, int U>
__device__ __forceinline__ void mul_batch(const uint4 (&w)[U][R], const uint32_t (&s)[U][R],
                                          const uint4 *xs, int C, int it, float (&acc)[R],
                                          uint32_t bias) {
    const int cfirst = ((threadIdx.x >> 6) % KS) * 16 + (threadIdx.x & 15);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = cfirst + (it * U + u) * 16 * KS;
        uint4 xq[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
            xq[p] = xs[p * C + c];
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = chunk_acc(w[u][r], xq, f16_to_f32((uint16_t)s[u][r]), acc[r], bias);
    }
}

// Batches of this workgroup: row blocks blk0, blk0 + stride, ... (blk0 <
// nblk), C / (16 KS U) batches each.
template <int R, int KS, int U, Epi E>
__device__ __forceinline__ int64_t pipe_batches(int C, int64_t n_units, int64_t blk0,
                                                int64_t stride) {
    const int64_t nblk = row_blocks<R, KS, E>(n_units);
    return (nblk - blk0 + stride - 1) / stride * (C / (16 * KS * U));
}

// Issues batch q of this workgroup: row block blk0 + (q / niter) * stride,
// batch q % niter within it.
template <int R, int KS, int U, bool NT, Epi E>
__device__ __forceinline__ void load_batch_q(const uint8_t *W, const uint16_t *S, int64_t N,
                                             int C, int64_t n_units, const EpiArgs &ea,
                                             int64_t blk0, int64_t stride, int niter, int64_t q,
                                             uint4 (&w)[U][R], uint32_t (&s)[U][R]) {
    load_batch<R, KS, U, NT, E>(W, S, N, C, n_units, ea, blk0 + (q / niter) * stride,
                                (int)(q % niter), w, s);
}

// Issues batches 0 and 1 of this workgroup into A and B (a workgroup with
// a single batch loads it into both, so B is always in flight).
template <int R, int KS, int U, bool NT, Epi E>
__device__ __forceinline__ void prefetch_pipe(const uint8_t *W, const uint16_t *S, int64_t N,
                                              int K, int64_t n_units, const EpiArgs &ea,
                                              int64_t blk0, int64_t stride, uint4 (&wA)[U][R],
                                              uint32_t (&sA)[U][R], uint4 (&wB)[U][R],
                                              uint32_t (&sB)[U][R]) {
    const int C = K >> 5;
    const int niter = C / (16 * KS * U);
    const int64_t Q = pipe_batches<R, KS, U, E>(C, n_units, blk0, stride);
    load_batch_q<R, KS, U, NT, E>(W, S, N, C, n_units, ea, blk0, stride, niter, 0, wA, sA);
    load_batch_q<R, KS, U, NT, E>(W, S, N, C, n_units, ea, blk0, stride, niter, Q > 1 ? 1 : 0,
                                  wB, sB);
}

// Precondition: prefetch_pipe issued batches 0 and 1.  The main loop runs
// while batches q .. q + 3 all exist, so its loads are unconditional and
// the compiler's wait before each multiply covers only that buffer's
// loads; the last one to three batches follow in a short tail.  Every
// thread of the workgroup must call this.
template <int R, int KS, int U, bool NT, Epi E>
__device__ __forceinline__ void run_units_pipe(const uint8_t *W, const uint16_t *S, int64_t N,
                                               int K, int64_t n_units, const EpiArgs &ea,
                                               int64_t blk0, int64_t stride, const uint4 *xs,
                                               float (*red)[kSlots][R], uint4 (&wA)[U][R],
                                               uint32_t (&sA)[U][R], uint4 (&wB)[U][R],
                                               uint32_t (&sB)[U][R], uint32_t bias) {
    constexpr int kUnitsPerBlock = Geometry<E, R, KS>::kUnitsPerBlock;
    const int C = K >> 5;
    const int niter = C / (16 * KS * U);
    const int64_t Q = pipe_batches<R, KS, U, E>(C, n_units, blk0, stride);
    const int wave = threadIdx.x >> 6;
    const int64_t my_unit = (wave / KS) * kSlots + ((threadIdx.x & 63) >> 4);
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0.0f;
    auto finish = [&](int64_t q) {
        if ((int)(q % niter) == niter - 1) {
            reduce_rows<R, KS>(acc, red);
            store_unit<R, KS, E, false>(acc, (blk0 + (q / niter) * stride) * kUnitsPerBlock +
                                                 my_unit,
                                        N, n_units, ea);
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[r] = 0.0f;
        }
    };
    int64_t q = 0;
    for (; q + 3 < Q; q += 2) {
        mul_batch<R, KS, U>(wA, sA, xs, C, (int)(q % niter), acc, bias);
        finish(q);
        load_batch_q<R, KS, U, NT, E>(W, S, N, C, n_units, ea, blk0, stride, niter, q + 2, wA,
                                      sA);
        mul_batch<R, KS, U>(wB, sB, xs, C, (int)((q + 1) % niter), acc, bias);
        finish(q + 1);
        load_batch_q<R, KS, U, NT, E>(W, S, N, C, n_units, ea, blk0, stride, niter, q + 3, wB,
                                      sB);
    }
    // Q - q batches remain (1 to 3): q in A, q + 1 in B.
    mul_batch<R, KS, U>(wA, sA, xs, C, (int)(q % niter), acc, bias);
    finish(q);
    if (q + 2 < Q)
        load_batch_q<R, KS, U, NT, E>(W, S, N, C, n_units, ea, blk0, stride, niter, q + 2, wA,
                                      sA);
    if (q + 1 < Q) {
        mul_batch<R, KS, U>(wB, sB, xs, C, (int)((q + 1) % niter), acc, bias);
        finish(q + 1);
    }
    if (q + 2 < Q) {
        mul_batch<R, KS, U>(wA, sA, xs, C, (int)((q + 2) % niter), acc, bias);
        finish(q + 2);
    }
}

// Stages the activation of a product into LDS.
template <Pro P, bool COH = false>
__device__ __forceinline__ void stage_activation(const void *xin, uint4 *xs, int K,
                                                 const EpiArgs &ea, float *wsum) {
    if constexpr (P == Pro::RmsNorm)
        stage_rmsnorm<COH>(static_cast<const float *>(xin), xs, K, ea.eps, ea.norm_out, wsum);
    else
        stage_x<COH>(static_cast<const uint16_t *>(xin), xs, K);
}

} // namespace
} // namespace q4
