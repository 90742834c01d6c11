// Small-batch INT4 product on the vector ALUs: Y[b] = W X[b] for a few
// activation columns (a speculative-verify batch of two to four tokens).
//
// Operation: PIPO: Pipelined Offloading for Efficient Inference on Consumer
// Devices, "Method", bullets "Computation optimization" and "Automatic
// configuration" -- the 4-bit kernel serves small batches, and a batch
// reuses every unpacked weight for each of its vectors.
//
// Same decomposition as the batch-1 product (q4_gemv.hip): 16-lane rows own
// output rows, each lane streams 16-byte chunks (one group of 32 codes), KS
// waves split a row's k range.  A chunk is unpacked once into sixteen exact
// binary16 pairs (code - 8, or 16 (code - 8)) and then multiplied with the
// matching activation pairs of each of the B columns by v_dot2_f32_f16; the
// B columns are staged in LDS in the unpack's pair order.  Per column the
// arithmetic and its order are exactly those of the batch-1 kernel at the
// same k split, so each column equals q4_gemv of that column bitwise.
//
// Measured on the 8B shapes (back-to-back launches): gate+up 18.0 us at B =
// 2 and 24.2 at B = 4 against 26.4 and 26.9 us on the matrix cores; at B = 8
// the dot products take over the VALU (39.8 vs 28.2 us), so wider batches
// stay on the matrix-core kernel.
#include "q4_gemv_core.h"

namespace q4 {
namespace {

// Exact binary16 pairs of one chunk in unpack order: for word i,
// q[4i] = (k0-8, k4-8), q[4i+1] = 16 (k1-8, k5-8), q[4i+2] = (k2-8, k6-8),
// q[4i+3] = 16 (k3-8, k7-8).
__device__ __forceinline__ void unpack_chunk(uint4 w, uint32_t bias, half2_t (&q)[16]) {
    const half2_t off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2_t off_hi = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t v = wd[i];
        const uint32_t u = v >> 8;
        q[4 * i + 0] = as_h2((v & 0x000F000Fu) | bias) - off_lo;
        q[4 * i + 1] = as_h2((v & 0x00F000F0u) | bias) - off_hi;
        q[4 * i + 2] = as_h2((u & 0x000F000Fu) | bias) - off_lo;
        q[4 * i + 3] = as_h2((u & 0x00F000F0u) | bias) - off_hi;
    }
}

// One unpacked chunk against one column's 32 permuted activations: the sums
// and their order are those of chunk_acc.
__device__ __forceinline__ float dot_chunk(const half2_t (&q)[16], const uint4 (&xq)[4], float s,
                                           float acc) {
    float tlo = 0.0f, thi = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tlo = __builtin_amdgcn_fdot2(q[4 * i + 0], as_h2(xq[i].x), tlo, false);
        thi = __builtin_amdgcn_fdot2(q[4 * i + 1], as_h2(xq[i].y), thi, false);
        tlo = __builtin_amdgcn_fdot2(q[4 * i + 2], as_h2(xq[i].z), tlo, false);
        thi = __builtin_amdgcn_fdot2(q[4 * i + 3], as_h2(xq[i].w), thi, false);
    }
    return fmaf(s, fmaf(thi, 0.0625f, tlo), acc);
}

// X16: binary16 [B][K]; Store / Residual: ea.y = Y f32 [B][N] (written /
// added to); SiluPair: ea.out16 = M binary16 [B][pair_off], rows (j, j +
// pair_off) give M[b][j] = f16(silu(gate) * up).
template <int R, int KS, int U, int B, Epi E>
__global__ void __launch_bounds__(kThreads)
gemv_batch_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
                  const uint16_t *__restrict__ X16, int64_t N, int K, int64_t n_units,
                  EpiArgs ea) {
    extern __shared__ uint4 xs[];
    __shared__ float red[kWaves][kSlots][R * B];
    const uint32_t bias = vgpr_const(0x64006400u);
    const int C = K >> 5;
    const int nb = K >> 3;  // 8-value blocks per column
    const int xcol = K >> 3; // uint4 per staged column
    const uint8_t *wp[R];
    const uint16_t *sp[R];
    uint4 w[U][R];
    uint16_t s[U][R];

    // Activation loads first (up to kXR per thread in registers), then the
    // first weight batch, then the LDS writes.
    // (unconditional loads, indices past the end wrapping around, so the
    // wait before the LDS writes covers only these loads)
    uint4 xr[kXR];
#pragma unroll
    for (int j = 0; j < kXR; ++j) {
        const int i = threadIdx.x + j * kThreads;
        xr[j] = gload16(X16 + 8 * (size_t)(i < B * nb ? i : i % (B * nb)));
    }
    prefetch_block<R, KS, U, true, E, false>(W, S, N, K, n_units, ea, blockIdx.x, w, s, wp, sp);
    auto put = [&](int i, uint4 v) {
        const int b = i / nb, k8 = i - b * nb;
        xs[b * xcol + (k8 & 3) * C + (k8 >> 2)] = permute8(v);
    };
#pragma unroll
    for (int j = 0; j < kXR; ++j) {
        const int i = threadIdx.x + j * kThreads;
        if (i < B * nb)
            put(i, xr[j]);
    }
    for (int i = threadIdx.x + kXR * kThreads; i < B * nb; i += kThreads)
        put(i, gload16(X16 + 8 * (size_t)i));
    __syncthreads();

    constexpr int kUnitsPerBlock = Geometry<E, R, KS>::kUnitsPerBlock;
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

    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int64_t unit = blk * kUnitsPerBlock + rgroup * kSlots + slot;
        float acc[R][B];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b)
                acc[r][b] = 0.0f;
        for (int it = 0; it < niter; ++it) {
            if (it > 0)
                load_chunks<U, R, true>(w, s, wp, sp, it * U, nl, cstep);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = it * U + u;
                if (j < nl) {
                    half2_t q[R][16];
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        unpack_chunk(w[u][r], bias, q[r]);
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        uint4 xq[4];
#pragma unroll
                        for (int p = 0; p < 4; ++p)
                            xq[p] = xs[b * xcol + p * C + cfirst + j * cstep];
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            acc[r][b] = dot_chunk(q[r], xq, f16_to_f32(s[u][r]), acc[r][b]);
                    }
                }
            }
        }
        // Row sums over the 16 lanes, then over the k-split waves in a
        // fixed order (the batch-1 kernel's order).
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b)
                acc[r][b] = row16_sum(acc[r][b]);
        if constexpr (KS > 1) {
            if (sl == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        red[wave][slot][r * B + b] = acc[r][b];
            }
            __syncthreads();
            if (kpart == 0 && sl == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        float t = red[wave][slot][r * B + b];
                        for (int k = 1; k < KS; ++k)
                            t += red[wave + k][slot][r * B + b];
                        acc[r][b] = t;
                    }
            }
            __syncthreads();
        }
        if (blk + gridDim.x < nblk) {
            setup_rows<R, KS, E>(W, S, N, C, n_units, ea, blk + gridDim.x, wp, sp);
            load_chunks<U, R, true>(w, s, wp, sp, 0, nl, cstep);
        }
        if (kpart == 0 && sl == 0 && unit < n_units) {
            if constexpr (E == Epi::SiluPair) {
                static_assert(R == 2, "paired rows need two rows per slot");
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const float g = acc[0][b], up = acc[1][b];
                    const float silu = g / (1.0f + expf(-g));
                    ea.out16[(size_t)b * ea.pair_off + unit] = f32_to_f16(silu * up);
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int64_t row = unit * R + r;
                    if (row < N) {
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            float *y = ea.y + (size_t)b * N + row;
                            if constexpr (E == Epi::Residual)
                                *y = *y + acc[r][b];
                            else
                                *y = acc[r][b];
                        }
                    }
                }
            }
        }
    }
}

using BatchFn = void (*)(const uint8_t *, const uint16_t *, const uint16_t *, int64_t, int,
                         int64_t, EpiArgs);

template <int R, int KS, int U, Epi E>
BatchFn pick_b(int B) {
    switch (B) {
    case 2: return gemv_batch_kernel<R, KS, U, 2, E>;
    case 3: return gemv_batch_kernel<R, KS, U, 3, E>;
    case 4: return gemv_batch_kernel<R, KS, U, 4, E>;
    case 8:
        if constexpr (E == Epi::Store)
            return gemv_batch_kernel<R, KS, U, 8, E>;
        return nullptr;
    default: return nullptr;
    }
}

// Four chunks in flight per lane, or two when a lane has no more per row
// (the loads are unconditional, so extra ones would be wasted).
template <Epi E>
BatchFn pick_batch(int R, int KS, int B, int nl) {
#define Q4_PICK(r, ks)                                                           \
    if (R == r && KS == ks)                                                      \
        return nl <= 2 ? pick_b<r, ks, 2, E>(B) : pick_b<r, ks, 4, E>(B);
    if constexpr (E == Epi::SiluPair) {
        Q4_PICK(2, 1) Q4_PICK(2, 2) Q4_PICK(2, 4)
    } else {
        Q4_PICK(1, 1) Q4_PICK(1, 2) Q4_PICK(1, 4)
        Q4_PICK(2, 1) Q4_PICK(2, 2) Q4_PICK(2, 4)
    }
#undef Q4_PICK
    return nullptr;
}

int batch_resident_blocks(BatchFn fn, size_t lds) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kThreads, lds) != hipSuccess ||
        nb < 1)
        nb = 1;
    return nb * device_cus();
}

} // namespace

// Up to three columns.  From four the matrix cores win or tie on the 8B
// shapes (B = 4, vector ALU / the library's matrix-core launch, us: 6144 x
// 4096 8.49 / 8.63, 4096 x 4096 6.48 / 5.86, 28672 x 4096 24.7 / 20.0); at
// three 7.13 / 8.66, 5.31 / 6.59 and 20.9 / 24.6 (row-tile launch).
bool gemv_batch_fits(int32_t B, int64_t K) {
    return B >= 2 && B <= kBatchMaxCols && (int64_t)B * K * 2 <= kBatchStageBytes;
}

q4_status launch_gemv_batch(const uint8_t *packed, const uint16_t *scales, const uint16_t *X16,
                            int64_t N, int64_t K, int32_t B, Epi epi, const EpiArgs &ea,
                            hipStream_t stream) {
    if ((int64_t)B * K * 2 > kBatchStageBytes)
        return fail(Q4_ERR_UNSUPPORTED, "gemv batch: %d columns of K=%lld exceed %d LDS bytes",
                    B, (long long)K, kBatchStageBytes);
    // Where the batch-1 product is a row-per-wave kernel, so is this.
    if (use_row_kernels(epi, K))
        return launch_gemv_row_batch(packed, scales, X16, N, K, B, epi, ea, stream);
    // The batch-1 kernel's rows per slot and k split for this shape, so each
    // column's summation order is the batch-1 product's.
    int R = 0, KS = 0;
    gemv_shape(epi, epi == Epi::SiluPair ? 2 * ea.pair_off : N, K, &R, &KS);
    const int nl = (int)((K / 32 + 16 * KS - 1) / (16 * KS));
    BatchFn fn = epi == Epi::SiluPair  ? pick_batch<Epi::SiluPair>(R, KS, B, nl)
                 : epi == Epi::Residual ? pick_batch<Epi::Residual>(R, KS, B, nl)
                 : epi == Epi::Store    ? pick_batch<Epi::Store>(R, KS, B, nl)
                                        : nullptr;
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED, "gemv batch: no kernel for B=%d R=%d KS=%d", B, R, KS);
    int64_t n_units;
    if (epi == Epi::SiluPair) {
        if (ea.pair_off * 2 != N)
            return fail(Q4_ERR_INVALID_ARG, "gemv batch: paired rows need N == 2*pair_off");
        n_units = ea.pair_off;
    } else {
        n_units = (N + R - 1) / R;
    }
    const int units_per_block = (kWaves / KS) * kSlots;
    const int64_t nblk = (n_units + units_per_block - 1) / units_per_block;
    const size_t lds = (size_t)B * K * 2;
    const int64_t grid = std::min<int64_t>(nblk, batch_resident_blocks(fn, lds));
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kThreads), lds, stream, packed, scales,
                       X16, N, (int)K, n_units, ea);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace q4
