// INT4 matrix-vector product with one row per wave instruction (K <= 4096 by
// default; up to 8192 for measurement).
//
// Operation: PIPO: Pipelined Offloading for Efficient Inference on Consumer
// Devices, "Method", bullet "Computation optimization" -- the vector is
// multiplied directly by the 4-bit weights; no dequantized matrix is ever
// written.  Unpack and per-chunk arithmetic are those of q4_gemv.hip.
//
// Work decomposition (our own for CDNA4).  Every wave works alone: no LDS,
// no workgroup barrier.  A wave takes R rows at a time; lane l reads the
// 16-byte chunks (groups of 32 codes) l, l + 64, ... of each row, so one
// load instruction covers 1 KB of one row -- a linear sweep, which the HBM
// streams faster than several shorter runs of different rows.  The lane
// needs only the activations of its own chunks (at most four, K <= 8192),
// so it holds them in registers, already in the unpack's pair order (the
// workgroup stages the activation, or its RMSNorm, in LDS once with linear
// loads; each lane then copies its chunks), or, with three or four chunks
// per lane, reads them from LDS as it goes; a row total is a 64-lane
// DPP/permlane sum.
//
// Summation order of one output: per lane, its chunks in increasing order
// (each chunk: exact binary16 products summed by v_dot2_f32_f16, then the
// group scale in fp32), then the fixed 64-lane sum.  The batch kernel below
// keeps exactly this order per column, so each column of a 2..4-column
// product equals q4_gemv of that column bitwise.
#include <algorithm>

#include "q4_gemv_core.h"
#include "q4_lanes.h"

namespace q4 {
namespace {

constexpr int kRowWaves = 4;
constexpr int kRowThreads = 64 * kRowWaves;

// Sum over the 64 lanes with identical bits in every lane: every step adds
// a value and its partner's in the same order on both sides (quad xor
// pairs, half-row and row mirrors, then the row and half-wave swaps), so a
// row total can be stored from any lane -- the batch kernel stores column b
// of row r from another lane than the batch-1 kernel does.
__device__ __forceinline__ float wave_total(float x) {
    x = row16_sum(x);
    const lanes::Rows16 r(x);
    x = lanes::fa(r.a) + lanes::fa(r.b);
    const lanes::Halves32 h(x);
    return lanes::fa(h.a) + lanes::fa(h.b);
}

// Chunk j of this lane: index lane + 64 j, clamped into the row (loads stay
// in bounds); `valid` marks the real ones (a clamped chunk gets scale 0, so
// it adds exactly nothing).
template <int NC>
struct RowChunks {
    int c[NC];
    bool valid[NC];
};

template <int NC>
__device__ __forceinline__ RowChunks<NC> row_chunks(int lane, int C) {
    RowChunks<NC> g;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = lane + 64 * j;
        g.valid[j] = c < C;
        g.c[j] = c < C ? c : C - 1;
    }
    return g;
}

// Output units per group of R rows: SiluPair pairs gate row u with up row
// u + pair_off, so R rows hold R / 2 units.
template <Epi E, int R>
constexpr int units_per_group() {
    return E == Epi::SiluPair ? R / 2 : R;
}

// Matrix row of row slot r of group g (units past the end repeat the last).
template <Epi E, int R>
__device__ __forceinline__ int64_t group_row(int64_t g, int r, int64_t n_units,
                                             const EpiArgs &ea) {
    constexpr int UP = units_per_group<E, R>();
    int64_t unit = g * UP + r % UP;
    unit = unit < n_units ? unit : n_units - 1;
    if constexpr (E == Epi::SiluPair)
        return unit + (r / UP) * ea.pair_off;
    else
        return unit;
}

template <int NC, int R, Epi E>
__device__ __forceinline__ void group_loads(const uint8_t *W, const uint16_t *S, int C,
                                            int64_t n_units, const EpiArgs &ea, int64_t g,
                                            const RowChunks<NC> &ch, uint4 (&w)[R][NC],
                                            uint16_t (&s)[R][NC]) {
    const size_t row_bytes = (size_t)C * 16;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = group_row<E, R>(g, r, n_units, ea);
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            w[r][j] = wload16<true>(W + (size_t)row * row_bytes + (size_t)ch.c[j] * 16);
            s[r][j] = gload(S + (size_t)row * C + ch.c[j]);
        }
    }
}

template <int NC>
__device__ __forceinline__ float row_acc(const uint4 (&w)[NC], const uint16_t (&s)[NC],
                                         const uint4 (&xq)[NC][4], const RowChunks<NC> &ch,
                                         uint32_t bias) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NC; ++j)
        acc = chunk_acc(w[j], xq[j], ch.valid[j] ? f16_to_f32(s[j]) : 0.0f, acc, bias);
    return acc;
}

// NC chunks per lane (K <= 64 NC * 32), R rows per group, epilogue E,
// prologue P.  Grid: waves take groups wave, wave + total waves, ...
// The activation is staged once per workgroup exactly as the other product
// kernel stages it (linear loads, the same RMSNorm sums, so the same bits),
// then every lane copies its own chunks from LDS into registers; after that
// the waves never meet again.
template <int NC, int R, Epi E, Pro P, bool XREG>
__global__ void __launch_bounds__(kRowThreads)
gemv_row_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
                const void *__restrict__ xin, int64_t N, int K, int64_t n_units, EpiArgs ea) {
    static_assert(E != Epi::SiluPair || R % 2 == 0, "paired rows come in pairs");
    static_assert(kRowThreads == kThreads, "the staging code assumes the product's workgroup");
    constexpr int UP = units_per_group<E, R>();
    extern __shared__ uint4 xs[];
    __shared__ float wsum[kWaves];
    const int lane = threadIdx.x & 63;
    const int64_t wave =
        __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kRowWaves + (threadIdx.x >> 6)));
    const int64_t nwaves = (int64_t)gridDim.x * kRowWaves;
    const int C = K >> 5;
    const int64_t ngroups = (n_units + UP - 1) / UP;
    int64_t g = wave;
    const uint32_t bias = vgpr_const(0x64006400u);
    const RowChunks<NC> ch = row_chunks<NC>(lane, C);

    // activation loads first, then the first group's weights, then the
    // staging arithmetic while the weights are in flight
    XStage st;
    stage_issue<P, false>(xin, K, st);
    uint4 w[R][NC];
    uint16_t s[R][NC];
    float hv = 0.0f; // Residual: old value of this lane's row (lane r: row r)
    const int64_t g0 = g < ngroups ? g : ngroups - 1;
    group_loads<NC, R, E>(W, S, C, n_units, ea, g0, ch, w, s);
    if constexpr (E == Epi::Residual)
        hv = gload(ea.y + group_row<E, R>(g0, lane < R ? lane : 0, n_units, ea));
    stage_finish<P, false>(xin, xs, K, ea, wsum, st);
    __syncthreads();
    if (g >= ngroups)
        return; // no barrier below: a wave without rows simply leaves
    // XREG: the lane's activation chunks stay in registers (NC <= 2);
    // otherwise they are read from LDS chunk by chunk (the same values, so
    // the same bits, with far fewer registers).
    uint4 xq[XREG ? NC : 1][4];
    if constexpr (XREG) {
#pragma unroll
        for (int j = 0; j < NC; ++j)
#pragma unroll
            for (int p = 0; p < 4; ++p)
                xq[j][p] = xs[p * C + ch.c[j]];
    }

    while (true) {
        float acc[R];
        if constexpr (XREG) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[r] = row_acc<NC>(w[r], s[r], xq, ch, bias);
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[r] = 0.0f;
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                uint4 xj[4];
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    xj[p] = xs[p * C + ch.c[j]];
#pragma unroll
                for (int r = 0; r < R; ++r)
                    acc[r] = chunk_acc(w[r][j], xj, ch.valid[j] ? f16_to_f32(s[r][j]) : 0.0f,
                                       acc[r], bias);
            }
        }
        const int64_t gn = g + nwaves;
        float hcur = hv;
        float tot[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            tot[r] = wave_total(acc[r]);
        if constexpr (E == Epi::SiluPair) {
#pragma unroll
            for (int i = 0; i < UP; ++i) {
                const int64_t unit = g * UP + i;
                if (lane == i && unit < n_units) {
                    const float gt = tot[i], up = tot[i + UP];
                    const float silu = gt / (1.0f + expf(-gt));
                    ea.out16[unit] = f32_to_f16(silu * up);
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t row = g * R + r;
                if (lane == r && row < N) {
                    if constexpr (E == Epi::Residual) {
                        ea.y[row] = hcur + tot[r];
                    } else {
                        ea.y[row] = tot[r];
                        if constexpr (E == Epi::QkvGather) {
                            if (row >= ea.v_off) {
                                const int64_t v = row - ea.v_off;
                                const int64_t gi = v / ea.hd, i = v % ea.hd;
                                const uint16_t h16 = f32_to_f16(tot[r]);
                                for (int q = 0; q < ea.group; ++q)
                                    ea.out16[(gi * ea.group + q) * ea.hd + i] = h16;
                            }
                        }
                    }
                }
            }
        }
        if (gn >= ngroups)
            break;
        g = gn;
        group_loads<NC, R, E>(W, S, C, n_units, ea, g, ch, w, s);
        if constexpr (E == Epi::Residual)
            hv = gload(ea.y + group_row<E, R>(g, lane < R ? lane : 0, n_units, ea));
    }
}

// B binary16 columns X16[B][K] staged in LDS (pair order, [B][4][C]); per
// column the batch-1 kernel's arithmetic and order.  Store / Residual:
// ea.y = Y f32 [B][N]; SiluPair: ea.out16 = M binary16 [B][pair_off].
template <int NC, int R, int B, Epi E>
__global__ void __launch_bounds__(kRowThreads)
gemv_row_batch_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
                      const uint16_t *__restrict__ X16, int64_t N, int K, int64_t n_units,
                      EpiArgs ea) {
    static_assert(E != Epi::SiluPair || R % 2 == 0, "paired rows come in pairs");
    constexpr int UP = units_per_group<E, R>();
    extern __shared__ uint4 xs[];
    const int lane = threadIdx.x & 63;
    const int64_t wave =
        __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kRowWaves + (threadIdx.x >> 6)));
    const int64_t nwaves = (int64_t)gridDim.x * kRowWaves;
    const int C = K >> 5;
    const int nb = K >> 3; // 8-value blocks per column
    const int64_t ngroups = (n_units + UP - 1) / UP;
    const RowChunks<NC> ch = row_chunks<NC>(lane, C);
    uint4 w[R][NC];
    uint16_t s[R][NC];
    int64_t g = wave;
    if (g < ngroups)
        group_loads<NC, R, E>(W, S, C, n_units, ea, g, ch, w, s);
    for (int i = threadIdx.x; i < B * nb; i += kRowThreads) {
        const int b = i / nb, k8 = i - b * nb;
        xs[(size_t)b * 4 * C + (k8 & 3) * C + (k8 >> 2)] = permute8(gload16(X16 + 8 * (size_t)i));
    }
    __syncthreads();
    if (g >= ngroups)
        return;
    const uint32_t bias = vgpr_const(0x64006400u);
    while (true) {
        float acc[R][B];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b)
                acc[r][b] = 0.0f;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            half2_t q[R][16];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint4 wv = w[r][j];
                const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
                const half2_t off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
                const half2_t off_hi = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t v = wd[i], u = v >> 8;
                    q[r][4 * i + 0] = as_h2((v & 0x000F000Fu) | bias) - off_lo;
                    q[r][4 * i + 1] = as_h2((v & 0x00F000F0u) | bias) - off_hi;
                    q[r][4 * i + 2] = as_h2((u & 0x000F000Fu) | bias) - off_lo;
                    q[r][4 * i + 3] = as_h2((u & 0x00F000F0u) | bias) - off_hi;
                }
            }
#pragma unroll
            for (int b = 0; b < B; ++b) {
                uint4 xq[4];
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    xq[p] = xs[(size_t)b * 4 * C + p * C + ch.c[j]];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float sc = ch.valid[j] ? f16_to_f32(s[r][j]) : 0.0f;
                    float tlo = 0.0f, thi = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        tlo = __builtin_amdgcn_fdot2(q[r][4 * i + 0], as_h2(xq[i].x), tlo, false);
                        thi = __builtin_amdgcn_fdot2(q[r][4 * i + 1], as_h2(xq[i].y), thi, false);
                        tlo = __builtin_amdgcn_fdot2(q[r][4 * i + 2], as_h2(xq[i].z), tlo, false);
                        thi = __builtin_amdgcn_fdot2(q[r][4 * i + 3], as_h2(xq[i].w), thi, false);
                    }
                    acc[r][b] = fmaf(sc, fmaf(thi, 0.0625f, tlo), acc[r][b]);
                }
            }
        }
        const int64_t gn = g + nwaves;
        if (gn < ngroups)
            group_loads<NC, R, E>(W, S, C, n_units, ea, gn, ch, w, s);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b)
                acc[r][b] = wave_total(acc[r][b]);
        if constexpr (E == Epi::SiluPair) {
#pragma unroll
            for (int i = 0; i < UP; ++i)
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const int64_t unit = g * UP + i;
                    if (lane == i * B + b && unit < n_units) {
                        const float gt = acc[i][b], up = acc[i + UP][b];
                        const float silu = gt / (1.0f + expf(-gt));
                        ea.out16[(size_t)b * ea.pair_off + unit] = f32_to_f16(silu * up);
                    }
                }
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const int64_t row = g * R + r;
                    if (lane == r * B + b && row < N) {
                        float *y = ea.y + (size_t)b * N + row;
                        if constexpr (E == Epi::Residual)
                            *y = *y + acc[r][b];
                        else
                            *y = acc[r][b];
                    }
                }
        }
        if (gn >= ngroups)
            break;
        g = gn;
    }
}

using RowFn = void (*)(const uint8_t *, const uint16_t *, const void *, int64_t, int, int64_t,
                       EpiArgs);
using RowBatchFn = void (*)(const uint8_t *, const uint16_t *, const uint16_t *, int64_t, int,
                            int64_t, EpiArgs);

template <int NC, Epi E, Pro P>
RowFn pick_row_r(int R) {
    constexpr bool kReg = NC <= 2;
    if (R == 2)
        return gemv_row_kernel<NC, 2, E, P, kReg>;
    if (R == 4)
        return gemv_row_kernel<NC, 4, E, P, kReg>;
    return nullptr;
}

// Chunks per lane with a row kernel: up to four (K <= 8192).  A wave holds
// all of a group's chunks in flight, so wider rows (the down products, K =
// 14336 and 28672: 7 and 14 chunks per lane) would need 220 to 256+ VGPRs;
// they keep the product kernel of q4_gemv.hip.
template <Epi E, Pro P>
RowFn pick_row_nc(int NC, int R) {
    switch (NC) {
    case 1: return pick_row_r<1, E, P>(R);
    case 2: return pick_row_r<2, E, P>(R);
    case 3: return pick_row_r<3, E, P>(R);
    case 4: return pick_row_r<4, E, P>(R);
    default: return nullptr;
    }
}

RowFn pick_row(Epi e, Pro p, int NC, int R) {
    if (p == Pro::RmsNorm) {
        switch (e) {
        case Epi::QkvGather: return pick_row_nc<Epi::QkvGather, Pro::RmsNorm>(NC, R);
        case Epi::SiluPair: return pick_row_nc<Epi::SiluPair, Pro::RmsNorm>(NC, R);
        default: return nullptr;
        }
    }
    switch (e) {
    case Epi::Store: return pick_row_nc<Epi::Store, Pro::F16>(NC, R);
    case Epi::Residual: return pick_row_nc<Epi::Residual, Pro::F16>(NC, R);
    case Epi::QkvGather: return pick_row_nc<Epi::QkvGather, Pro::F16>(NC, R);
    case Epi::SiluPair: return pick_row_nc<Epi::SiluPair, Pro::F16>(NC, R);
    }
    return nullptr;
}

template <int NC, Epi E>
RowBatchFn pick_row_batch_b(int B) {
    switch (B) {
    case 2: return gemv_row_batch_kernel<NC, 2, 2, E>;
    case 3: return gemv_row_batch_kernel<NC, 2, 3, E>;
    case 4: return gemv_row_batch_kernel<NC, 2, 4, E>;
    case 8:
        if constexpr (E == Epi::Store)
            return gemv_row_batch_kernel<NC, 2, 8, E>;
        return nullptr;
    default: return nullptr;
    }
}

template <Epi E>
RowBatchFn pick_row_batch(int NC, int B) {
    switch (NC) {
    case 1: return pick_row_batch_b<1, E>(B);
    case 2: return pick_row_batch_b<2, E>(B);
    case 3: return pick_row_batch_b<3, E>(B);
    case 4: return pick_row_batch_b<4, E>(B);
    default: return nullptr;
    }
}

// Rows per group: four for the tall products (N >= 16384: 28672 x 4096
// 13.1 us against 13.7 with two; 57344 x 8192 46.0 against 47.2), two
// otherwise (4096 x 4096 4.1 against 4.4; 10240 x 8192 11.7 against 12.0).
int row_rows(int64_t rows) { return rows >= 16384 ? 4 : 2; }

// Workgroups: one group per wave, at most four workgroups per compute unit
// (10240 x 8192: 11.7 us at 1024 workgroups against 12.6 at 1280).
int64_t row_grid(int64_t ngroups, int grid) {
    const int64_t need = (ngroups + kRowWaves - 1) / kRowWaves;
    const int64_t cap = grid > 0 ? grid : 4 * (int64_t)device_cus();
    return std::max<int64_t>(1, std::min(need, cap));
}

q4_status row_units(Epi epi, int64_t N, const EpiArgs &ea, int64_t *n_units, const char *what) {
    if (epi == Epi::SiluPair) {
        if (ea.pair_off * 2 != N)
            return fail(Q4_ERR_INVALID_ARG, "%s: paired rows need N == 2*pair_off", what);
        *n_units = ea.pair_off;
    } else {
        *n_units = N;
    }
    return Q4_OK;
}

} // namespace

// The default dispatch uses the row kernels up to K = 4096 (two chunks per
// lane): there they beat the product kernel of q4_gemv.hip (8B decode:
// gate+up 13.6 against 14.5 us, QKV 5.7 against 6.0, O 4.6 against 4.9);
// at K = 8192 they lose (70B gate+up 47.8 against the pipelined loop's 44.6
// us, O 10.7 against 9.4), so wider products keep that kernel.
bool gemv_row_fits(int64_t K) { return K / 32 <= 128; }

q4_status launch_gemv_row(const uint8_t *packed, const uint16_t *scales, const void *xin,
                          Pro pro, int64_t N, int64_t K, Epi epi, const EpiArgs &ea, int R,
                          int grid, hipStream_t stream) {
    const int C = (int)(K / 32);
    const int NC = (C + 63) / 64;
    if (R == 0)
        R = row_rows(N);
    RowFn fn = pick_row(epi, pro, NC, R);
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED, "gemv rows: no kernel for K=%lld rows_per_wave=%d",
                    (long long)K, R);
    int64_t n_units = 0;
    Q4_CHECK(row_units(epi, N, ea, &n_units, "gemv rows"));
    const int UP = epi == Epi::SiluPair ? R / 2 : R;
    const int64_t blocks = row_grid((n_units + UP - 1) / UP, grid);
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kRowThreads), (size_t)K * 2, stream,
                       packed, scales, xin, N, (int)K, n_units, ea);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

q4_status launch_gemv_row_batch(const uint8_t *packed, const uint16_t *scales,
                                const uint16_t *X16, int64_t N, int64_t K, int32_t B, Epi epi,
                                const EpiArgs &ea, hipStream_t stream) {
    const int C = (int)(K / 32);
    const int NC = (C + 63) / 64;
    RowBatchFn fn = epi == Epi::SiluPair  ? pick_row_batch<Epi::SiluPair>(NC, B)
                    : epi == Epi::Residual ? pick_row_batch<Epi::Residual>(NC, B)
                    : epi == Epi::Store    ? pick_row_batch<Epi::Store>(NC, B)
                                           : nullptr;
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED, "gemv rows batch: no kernel for B=%d K=%lld", B,
                    (long long)K);
    int64_t n_units = 0;
    Q4_CHECK(row_units(epi, N, ea, &n_units, "gemv rows batch"));
    const int UP = epi == Epi::SiluPair ? 1 : 2;
    const int64_t blocks = row_grid((n_units + UP - 1) / UP, 0);
    const size_t lds = (size_t)B * 4 * C * 16;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kRowThreads), lds, stream, packed, scales,
                       X16, N, (int)K, n_units, ea);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace q4

extern "C" q4_status q4_gemv_rows_tuned(const uint8_t *packed, const uint16_t *scales,
                                        const uint16_t *x_f16, float *y, int64_t N, int64_t K,
                                        int32_t rows_per_wave, int32_t workgroups,
                                        hipStream_t stream) {
    Q4_CHECK(q4::check_matrix(packed, scales, N, K, "q4_gemv_rows_tuned"));
    if (!x_f16 || !y)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_gemv_rows_tuned: null x or y");
    if (!q4::aligned(x_f16, 16) || !q4::aligned(y, 4))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_gemv_rows_tuned: x must be 16-byte and y 4-byte aligned");
    if (!(rows_per_wave == 2 || rows_per_wave == 4) || workgroups < 0)
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_gemv_rows_tuned: rows_per_wave must be 2 or 4, workgroups >= 0");
    if (K / 32 > 256)
        return q4::fail(Q4_ERR_UNSUPPORTED,
                        "q4_gemv_rows_tuned: no row kernel for K=%lld above 8192",
                        (long long)K);
    q4::EpiArgs ea{};
    ea.y = y;
    return q4::launch_gemv_row(packed, scales, x_f16, q4::Pro::F16, N, K, q4::Epi::Store, ea,
                               rows_per_wave, workgroups, stream);
}
