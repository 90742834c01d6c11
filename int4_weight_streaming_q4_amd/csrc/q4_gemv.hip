// Dequantization-free INT4 matrix-vector product for gfx950.
//
// Operation: PIPO: Pipelined Offloading for Efficient Inference on Consumer
// Devices, "Method", bullet "Computation optimization" -- the vector is
// multiplied directly by the 4-bit weights; no dequantized matrix is ever
// written.  The design below is our own for CDNA4 and is HBM-bound: every
// weight byte is read once with 128-bit loads, everything else is registers
// and LDS.
//
// Work decomposition
//   * A 16-lane DPP row of a wavefront owns one output row at a time; a
//     wave therefore works on 4 "slots", each on R rows.  Lane l of a slot
//     reads the 16-byte chunks l, l+16, ... of its rows (a chunk is one group
//     of 32 codes), so each load instruction covers four 256-byte runs.
//   * KS waves may split one slot's chunks between them (k-split); their
//     partial sums meet in LDS in a fixed order.
//   * The binary16 activation vector is staged once per workgroup into LDS,
//     already permuted so that the halves of each LDS dword pair up with the
//     nibble pairs the unpack produces (see below).
//
// Unpack (per 32-bit word v of 8 codes k0..k7, byte b holds k(2b), k(2b+1)):
//   (v & 0x000F000F) | 0x64006400 is the binary16 pair (1024+k0, 1024+k4);
//   (v & 0x00F000F0) | 0x64006400 is (1024+16*k1, 1024+16*k5);
//   the same on v >> 8 gives (k2, k6) and (16*k3, 16*k7).
// Subtracting 1032 (resp. 1152) is exact and leaves (k-8) (resp.
// 16*(k-8)); one v_dot2_f32_f16 per pair multiplies them with the matching
// activation pair exactly and sums in fp32.  The x16 sums are folded in with
// an exact 1/16, and each group's sum is scaled by its fp32 scale.
#include <map>
#include <mutex>
#include <utility>

#include "q4_internal.h"

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
__device__ __forceinline__ void stage_x(const uint16_t *__restrict__ x16, uint4 *xs, int K) {
    const int C = K >> 5;
    for (int b = threadIdx.x; b < (K >> 3); b += kThreads)
        xs[(b & 3) * C + (b >> 2)] = permute8(gload16(x16 + 8 * (size_t)b));
}

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ void load_f32x8(const float *p, float (&f)[8]) {
    const uint4 lo = gload16(p);
    const uint4 hi = gload16(p + 4);
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
__device__ __forceinline__ void stage_rmsnorm(const float *__restrict__ h, uint4 *xs, int K,
                                              float eps, uint16_t *norm_out, float *wsum) {
    const int C = K >> 5;
    float ss = 0.0f;
    for (int b = threadIdx.x; b < (K >> 3); b += kThreads) {
        float f[8];
        load_f32x8(h + 8 * (size_t)b, f);
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
    for (int b = threadIdx.x; b < (K >> 3); b += kThreads) {
        float f[8];
        load_f32x8(h + 8 * (size_t)b, f);
        uint32_t p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            p[i] = (uint32_t)f32_to_f16(f[2 * i] * r) |
                   ((uint32_t)f32_to_f16(f[2 * i + 1] * r) << 16);
        const uint4 v = {p[0], p[1], p[2], p[3]};
        xs[(b & 3) * C + (b >> 2)] = permute8(v);
        if (norm_out && blockIdx.x == 0)
            *reinterpret_cast<uint4 *>(norm_out + 8 * (size_t)b) = v;
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

// Loads of one group of U chunks of R rows; chunks past this lane's count
// are not loaded (their registers are zeroed and never used).
template <int U, int R, bool NT>
__device__ __forceinline__ void load_chunks(uint4 (&w)[U][R], uint16_t (&s)[U][R],
                                            const uint8_t *const (&wp)[R],
                                            const uint16_t *const (&sp)[R], int first, int nl,
                                            int cstep) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool ok = first + u < nl;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (ok) {
                w[u][r] = wload16<NT>(wp[r] + (size_t)(first + u) * cstep * 16);
                s[u][r] = wload2<NT>(sp[r] + (size_t)(first + u) * cstep);
            } else {
                w[u][r] = uint4{0u, 0u, 0u, 0u};
                s[u][r] = 0;
            }
        }
    }
}

// R rows per 16-lane row, KS waves per row's k range, U chunks of each row
// loaded per lane before use, NT non-temporal weight loads.
template <int R, int KS, int U, bool NT, Epi E, Pro P>
__global__ void __launch_bounds__(kThreads)
gemv_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
            const void *__restrict__ xin, int64_t N, int K, int64_t n_units, EpiArgs ea) {
    constexpr int kRowGroups = kWaves / KS;
    constexpr int kUnitsPerBlock = kRowGroups * kSlots;
    extern __shared__ uint4 xs[];
    __shared__ float red[kWaves][kSlots][R];
    __shared__ float wsum[kWaves];

    const int C = K >> 5;
    const uint32_t bias = vgpr_const(0x64006400u);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sl = lane & 15;
    const int slot = lane >> 4;
    const int rgroup = wave / KS;
    const int kpart = wave % KS;
    const int64_t nblk = (n_units + kUnitsPerBlock - 1) / kUnitsPerBlock;
    const size_t row_bytes = (size_t)K >> 1;
    // This lane's chunks: cfirst, cfirst + cstep, ... < C  (nl of them).
    const int cstep = 16 * KS;
    const int cfirst = kpart * 16 + sl;
    const int nl = cfirst < C ? (C - cfirst + cstep - 1) / cstep : 0;
    const int niter = (nl + U - 1) / U;

    const uint8_t *wp[R];
    const uint16_t *sp[R];
    uint4 w[U][R];
    uint16_t s[U][R];
    auto setup_rows = [&](int64_t b) {
        const int64_t unit = b * kUnitsPerBlock + rgroup * kSlots + slot;
        const int64_t lunit = unit < n_units ? unit : n_units - 1;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t row = row_of<E, R>(lunit, r, ea);
            row = row < N ? row : N - 1;
            wp[r] = W + (size_t)row * row_bytes + (size_t)cfirst * 16;
            sp[r] = S + (size_t)row * C + cfirst;
        }
    };

    // The first weight loads go out before the activation is staged, so
    // their HBM latency overlaps the prologue.
    int64_t blk = blockIdx.x;
    if (blk < nblk) {
        setup_rows(blk);
        load_chunks<U, R, NT>(w, s, wp, sp, 0, nl, cstep);
    }
    if constexpr (P == Pro::RmsNorm)
        stage_rmsnorm(static_cast<const float *>(xin), xs, K, ea.eps, ea.norm_out, wsum);
    else
        stage_x(static_cast<const uint16_t *>(xin), xs, K);
    __syncthreads();

    for (; blk < nblk; blk += gridDim.x) {
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

        // The next row block's first loads go out before this epilogue.
        if (blk + gridDim.x < nblk) {
            setup_rows(blk + gridDim.x);
            load_chunks<U, R, NT>(w, s, wp, sp, 0, nl, cstep);
        }

        if (kpart == 0 && sl == 0 && unit < n_units) {
            if constexpr (E == Epi::SiluPair) {
                static_assert(R == 2, "paired rows need two rows per slot");
                const float g = acc[0], up = acc[1];
                const float silu = g / (1.0f + expf(-g));
                ea.out16[unit] = f32_to_f16(silu * up);
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int64_t row = unit * R + r;
                    if (row < N) {
                        if constexpr (E == Epi::Residual) {
                            ea.y[row] += acc[r];
                        } else {
                            ea.y[row] = acc[r];
                            if constexpr (E == Epi::QkvGather) {
                                if (row >= ea.v_off) {
                                    const int64_t v = row - ea.v_off;
                                    const int64_t g = v / ea.hd, i = v % ea.hd;
                                    const uint16_t h16 = f32_to_f16(acc[r]);
                                    for (int q = 0; q < ea.group; ++q)
                                        ea.out16[(g * ea.group + q) * ea.hd + i] = h16;
                                }
                            }
                        }
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launch
using KernelFn = void (*)(const uint8_t *, const uint16_t *, const void *, int64_t, int,
                          int64_t, EpiArgs);

// Launch shape of one product kernel.
struct Cfg {
    int R, KS, U;
    bool NT;
};

template <Epi E, Pro P, int R, int KS>
KernelFn pick_ut(const Cfg &c) {
    if (c.U == 4)
        return c.NT ? gemv_kernel<R, KS, 4, true, E, P> : gemv_kernel<R, KS, 4, false, E, P>;
    if (c.U == 8)
        return c.NT ? gemv_kernel<R, KS, 8, true, E, P> : gemv_kernel<R, KS, 8, false, E, P>;
    return nullptr;
}

template <Epi E, Pro P>
KernelFn pick(const Cfg &c) {
#define Q4_PICK(r, ks)                                                           \
    if (c.R == r && c.KS == ks)                                                  \
        return pick_ut<E, P, r, ks>(c);
    if constexpr (E == Epi::SiluPair) {
        Q4_PICK(2, 1) Q4_PICK(2, 2) Q4_PICK(2, 4)
    } else if constexpr (E == Epi::Store) {
        Q4_PICK(1, 1) Q4_PICK(1, 2) Q4_PICK(1, 4)
        Q4_PICK(2, 1) Q4_PICK(2, 2) Q4_PICK(2, 4)
        Q4_PICK(4, 1) Q4_PICK(4, 2) Q4_PICK(4, 4)
    } else {
        Q4_PICK(1, 2) Q4_PICK(1, 4)
        Q4_PICK(2, 1) Q4_PICK(2, 2) Q4_PICK(2, 4)
    }
#undef Q4_PICK
    return nullptr;
}

KernelFn pick_kernel(Epi e, Pro p, const Cfg &c) {
    if (p == Pro::RmsNorm) {
        switch (e) {
        case Epi::QkvGather: return pick<Epi::QkvGather, Pro::RmsNorm>(c);
        case Epi::SiluPair: return pick<Epi::SiluPair, Pro::RmsNorm>(c);
        default: return nullptr;
        }
    }
    switch (e) {
    case Epi::Store: return pick<Epi::Store, Pro::F16>(c);
    case Epi::Residual: return pick<Epi::Residual, Pro::F16>(c);
    case Epi::QkvGather: return pick<Epi::QkvGather, Pro::F16>(c);
    case Epi::SiluPair: return pick<Epi::SiluPair, Pro::F16>(c);
    }
    return nullptr;
}

int resident_blocks(KernelFn fn, size_t lds) {
    static std::mutex mu;
    static std::map<std::pair<int, std::pair<void *, size_t>>, int> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    auto key = std::make_pair(dev, std::make_pair((void *)fn, lds));
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end())
        return it->second;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kThreads, lds) != hipSuccess ||
        nb < 1)
        nb = 1;
    int total = nb * device_cus();
    cache[key] = total;
    return total;
}

// Default launch shape, from rocprofv3 kernel traces of every shape on the
// decode matrices (non-temporal loads won or tied everywhere):
//   * two rows per 16-lane row with a 4-way k split is best or within 3% on
//     every 4096-wide product and on the largest ones (57344 x 8192);
//   * K = 8192 with 8192..12288 rows prefers one row per 16-lane row
//     (10240 x 8192: 12.2 vs 14.5 us; 8192 x 8192 with 8 chunks in flight:
//     11.0 vs 12.6 us);
//   * K = 28672 prefers a 2-way split (27.4 vs 28.2 us).
// The epilogue variant (paired rows) needs two rows per slot.
Cfg choose_config(Epi e, int64_t N, int64_t K) {
    const int64_t C = K / 32;
    Cfg c{2, 4, 4, true};
    if (e != Epi::SiluPair && K >= 8192 && K < 12288 && N <= 12288) {
        c.R = 1;
        if (N > 8192) {
            c.KS = 2;
        } else {
            c.KS = 4;
            c.U = 8;
        }
    } else if (K >= 16384) {
        c.KS = 2;
    }
    while (c.KS > 1 && C < 16 * c.KS)
        c.KS /= 2;
    return c;
}

} // namespace

q4_status launch_gemv_cfg(const uint8_t *packed, const uint16_t *scales, const void *xin,
                          Pro pro, int64_t N, int64_t K, Epi epi, const EpiArgs &ea, int R,
                          int KS, int U, bool NT, hipStream_t stream) {
    Cfg cfg{R, KS, U, NT};
    KernelFn fn = pick_kernel(epi, pro, cfg);
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED,
                    "gemv: no kernel for rows_per_slot=%d k_split=%d chunks=%d", R, KS, U);
    int64_t n_units;
    if (epi == Epi::SiluPair) {
        if (ea.pair_off * 2 != N)
            return fail(Q4_ERR_INVALID_ARG, "gemv: paired rows need N == 2*pair_off");
        n_units = ea.pair_off;
    } else {
        n_units = (N + R - 1) / R;
    }
    const int units_per_block = (kWaves / KS) * kSlots;
    const int64_t nblk = (n_units + units_per_block - 1) / units_per_block;
    const size_t lds = (size_t)K * 2;
    const int64_t grid = std::min<int64_t>(nblk, resident_blocks(fn, lds));
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kThreads), lds, stream, packed, scales,
                       xin, N, (int)K, n_units, ea);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

q4_status launch_gemv(const uint8_t *packed, const uint16_t *scales, const void *xin, Pro pro,
                      int64_t N, int64_t K, Epi epi, const EpiArgs &ea, hipStream_t stream) {
    const Cfg c = choose_config(epi, epi == Epi::SiluPair ? 2 * ea.pair_off : N, K);
    return launch_gemv_cfg(packed, scales, xin, pro, N, K, epi, ea, c.R, c.KS, c.U, c.NT, stream);
}

} // namespace q4

extern "C" q4_status q4_gemv(const uint8_t *packed, const uint16_t *scales,
                             const uint16_t *x_f16, float *y, int64_t N, int64_t K,
                             hipStream_t stream) {
    Q4_CHECK(q4::check_matrix(packed, scales, N, K, "q4_gemv"));
    if (!x_f16 || !y)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_gemv: null x or y");
    if (!q4::aligned(x_f16, 16) || !q4::aligned(y, 4))
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_gemv: x must be 16-byte and y 4-byte aligned");
    q4::EpiArgs ea{};
    ea.y = y;
    return q4::launch_gemv(packed, scales, x_f16, q4::Pro::F16, N, K, q4::Epi::Store, ea,
                            stream);
}

extern "C" q4_status q4_gemv_tuned(const uint8_t *packed, const uint16_t *scales,
                                   const uint16_t *x_f16, float *y, int64_t N, int64_t K,
                                   int32_t rows_per_slot, int32_t k_split,
                                   int32_t chunks_in_flight, int32_t nontemporal,
                                   hipStream_t stream) {
    Q4_CHECK(q4::check_matrix(packed, scales, N, K, "q4_gemv_tuned"));
    if (!x_f16 || !y)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_gemv_tuned: null x or y");
    if (!q4::aligned(x_f16, 16) || !q4::aligned(y, 4))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_gemv_tuned: x must be 16-byte and y 4-byte aligned");
    if (!(rows_per_slot == 1 || rows_per_slot == 2 || rows_per_slot == 4) ||
        !(k_split == 1 || k_split == 2 || k_split == 4) ||
        !(chunks_in_flight == 4 || chunks_in_flight == 8))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_gemv_tuned: rows_per_slot and k_split must be 1, 2 or 4, "
                        "chunks_in_flight 4 or 8");
    q4::EpiArgs ea{};
    ea.y = y;
    return q4::launch_gemv_cfg(packed, scales, x_f16, q4::Pro::F16, N, K, q4::Epi::Store, ea,
                               rows_per_slot, k_split, chunks_in_flight, nontemporal != 0,
                               stream);
}
