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

// One chunk (32 codes, 16 bytes) against its 32 permuted activations.
__device__ __forceinline__ float chunk_acc(uint4 w, const uint4 (&xq)[4], float s,
                                           float acc) {
    const half2_t off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2_t off_hi = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    float tlo = 0.0f, thi = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t v = wd[i];
        const uint32_t u = v >> 8;
        half2_t a = as_h2((v & 0x000F000Fu) | 0x64006400u) - off_lo;
        half2_t b = as_h2((v & 0x00F000F0u) | 0x64006400u) - off_hi;
        half2_t c = as_h2((u & 0x000F000Fu) | 0x64006400u) - off_lo;
        half2_t d = as_h2((u & 0x00F000F0u) | 0x64006400u) - off_hi;
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

// Stage x (binary16, K values) into LDS as xs[p * C + c] = the four
// activation pairs of 8-block p of chunk c, in unpack order.
__device__ __forceinline__ void stage_x(const uint16_t *__restrict__ x16, uint4 *xs,
                                        int K) {
    const int C = K >> 5;
    for (int b = threadIdx.x; b < (K >> 3); b += blockDim.x) {
        const uint4 v = *reinterpret_cast<const uint4 *>(x16 + 8 * (size_t)b);
        uint4 o;
        o.x = (v.x & 0xFFFFu) | (v.z << 16);          // (x0, x4)
        o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);      // (x1, x5)
        o.z = (v.y & 0xFFFFu) | (v.w << 16);          // (x2, x6)
        o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);      // (x3, x7)
        xs[(b & 3) * C + (b >> 2)] = o;
    }
}

template <int R, int KS, Epi E>
__global__ void __launch_bounds__(kThreads)
gemv_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
            const uint16_t *__restrict__ x16, int64_t N, int K, int64_t n_units,
            EpiArgs ea) {
    constexpr int U = (8 / R) > 1 ? (8 / R) : 1; // chunks in flight per row
    constexpr int kRowGroups = kWaves / KS;
    constexpr int kUnitsPerBlock = kRowGroups * kSlots;
    extern __shared__ uint4 xs[];
    __shared__ float red[kWaves][kSlots][R];

    const int C = K >> 5;
    stage_x(x16, xs, K);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sl = lane & 15;
    const int slot = lane >> 4;
    const int rgroup = wave / KS;
    const int kpart = wave % KS;
    const int64_t nblk = (n_units + kUnitsPerBlock - 1) / kUnitsPerBlock;
    const size_t row_bytes = (size_t)K >> 1;

    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int64_t unit = blk * kUnitsPerBlock + rgroup * kSlots + slot;
        const int64_t lunit = unit < n_units ? unit : n_units - 1;
        const uint8_t *wrow[R];
        const uint16_t *srow[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t row = row_of<E, R>(lunit, r, ea);
            row = row < N ? row : N - 1;
            wrow[r] = W + (size_t)row * row_bytes;
            srow[r] = S + (size_t)row * C;
        }
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = 0.0f;

        const int cstep = 16 * KS;
        for (int c0 = kpart * 16 + sl; c0 < C; c0 += cstep * U) {
            uint4 w[U][R];
            uint16_t s[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * cstep;
                const int cc = c < C ? c : c0;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    w[u][r] = *reinterpret_cast<const uint4 *>(wrow[r] + (size_t)cc * 16);
                    s[u][r] = srow[r][cc];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * cstep;
                if (c < C) {
                    uint4 xq[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        xq[p] = xs[p * C + c];
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[r] = chunk_acc(w[u][r], xq, f16_to_f32(s[u][r]), acc[r]);
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

// RMSNorm of one vector by one workgroup, fixed summation order.
constexpr int kNormThreads = 1024;

__global__ void __launch_bounds__(kNormThreads)
rmsnorm_f16_kernel(const float *__restrict__ h, uint16_t *__restrict__ a, int d, float eps) {
    __shared__ float part[kNormThreads];
    float ss = 0.0f;
    for (int i = threadIdx.x; i < d; i += kNormThreads)
        ss = fmaf(h[i], h[i], ss);
    part[threadIdx.x] = ss;
    __syncthreads();
    for (int w = kNormThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w)
            part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    const float r = 1.0f / sqrtf(part[0] / (float)d + eps);
    for (int i = threadIdx.x; i < d; i += kNormThreads)
        a[i] = f32_to_f16(h[i] * r);
}

// ---------------------------------------------------------------- launch
using KernelFn = void (*)(const uint8_t *, const uint16_t *, const uint16_t *, int64_t,
                          int, int64_t, EpiArgs);

template <Epi E>
KernelFn pick(int R, int KS) {
#define Q4_PICK(r, ks)                                                           \
    if (R == r && KS == ks)                                                      \
        return gemv_kernel<r, ks, E>;
    Q4_PICK(1, 1) Q4_PICK(1, 2) Q4_PICK(1, 4)
    Q4_PICK(2, 1) Q4_PICK(2, 2) Q4_PICK(2, 4)
    Q4_PICK(4, 1) Q4_PICK(4, 2) Q4_PICK(4, 4)
#undef Q4_PICK
    return nullptr;
}

KernelFn pick_kernel(Epi e, int R, int KS) {
    switch (e) {
    case Epi::Store: return pick<Epi::Store>(R, KS);
    case Epi::Residual: return pick<Epi::Residual>(R, KS);
    case Epi::QkvGather: return pick<Epi::QkvGather>(R, KS);
    case Epi::SiluPair:
        if (R != 2)
            return nullptr;
        if (KS == 1) return gemv_kernel<2, 1, Epi::SiluPair>;
        if (KS == 2) return gemv_kernel<2, 2, Epi::SiluPair>;
        if (KS == 4) return gemv_kernel<2, 4, Epi::SiluPair>;
        return nullptr;
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

// Shape heuristic: enough waves to cover the chip several times over, rows
// per slot raised only when rows are plentiful, k-split when they are not.
void choose_config(Epi e, int64_t n_units_r1, int64_t K, int *R, int *KS) {
    const int64_t want_waves = 8LL * device_cus();
    const int64_t C = K / 32;
    if (e == Epi::SiluPair) {
        *R = 2;
    } else {
        *R = 1;
    }
    int64_t units = (e == Epi::SiluPair) ? n_units_r1 : (n_units_r1 + *R - 1) / *R;
    int ks = 1;
    while (ks < 4 && (units / kSlots) * ks < want_waves && C / (16 * ks * 2) >= 2)
        ks *= 2;
    *KS = ks;
}

} // namespace

q4_status launch_gemv_cfg(const uint8_t *packed, const uint16_t *scales,
                          const uint16_t *x16, int64_t N, int64_t K, Epi epi,
                          const EpiArgs &ea, int R, int KS, hipStream_t stream) {
    KernelFn fn = pick_kernel(epi, R, KS);
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED, "gemv: no kernel for rows_per_slot=%d k_split=%d", R,
                    KS);
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
                       x16, N, (int)K, n_units, ea);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

q4_status launch_gemv(const uint8_t *packed, const uint16_t *scales, const uint16_t *x16,
                      int64_t N, int64_t K, Epi epi, const EpiArgs &ea,
                      hipStream_t stream) {
    int R, KS;
    choose_config(epi, epi == Epi::SiluPair ? ea.pair_off : N, K, &R, &KS);
    return launch_gemv_cfg(packed, scales, x16, N, K, epi, ea, R, KS, stream);
}

q4_status launch_rmsnorm_f16(const float *h, uint16_t *a, int32_t d, float eps,
                             hipStream_t stream) {
    hipLaunchKernelGGL(rmsnorm_f16_kernel, dim3(1), dim3(kNormThreads), 0, stream, h, a, d,
                       eps);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
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
    return q4::launch_gemv(packed, scales, x_f16, N, K, q4::Epi::Store, ea, stream);
}

extern "C" q4_status q4_gemv_tuned(const uint8_t *packed, const uint16_t *scales,
                                   const uint16_t *x_f16, float *y, int64_t N, int64_t K,
                                   int32_t rows_per_slot, int32_t k_split,
                                   hipStream_t stream) {
    Q4_CHECK(q4::check_matrix(packed, scales, N, K, "q4_gemv_tuned"));
    if (!x_f16 || !y)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_gemv_tuned: null x or y");
    if (!q4::aligned(x_f16, 16) || !q4::aligned(y, 4))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_gemv_tuned: x must be 16-byte and y 4-byte aligned");
    if (!(rows_per_slot == 1 || rows_per_slot == 2 || rows_per_slot == 4) ||
        !(k_split == 1 || k_split == 2 || k_split == 4))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_gemv_tuned: rows_per_slot and k_split must be 1, 2 or 4");
    q4::EpiArgs ea{};
    ea.y = y;
    return q4::launch_gemv_cfg(packed, scales, x_f16, N, K, q4::Epi::Store, ea, rows_per_slot,
                               k_split, stream);
}
