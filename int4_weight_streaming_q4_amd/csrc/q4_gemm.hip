// Small-batch INT4 product Y[b] = W X[b] (2 <= B <= 16) on gfx950 matrix
// cores.
//
// Operation: PIPO: Pipelined Offloading for Efficient Inference on Consumer
// Devices, "Method", bullets "Computation optimization" and "Automatic
// configuration" -- the 4-bit kernel serves batches below 16; a batch of B
// activation vectors (e.g. a speculative-verify batch) reuses every unpacked
// weight B times.  Up to four columns (whose binary16 copies fit 64 KB of
// LDS) the dot2 kernel of q4_gemv_batch.hip is faster; beyond that its dot
// products take over the VALU, so the multiply-adds go to
// v_mfma_f32_16x16x32_f16 here and the VALU only unpacks.
//
// One MFMA covers 16 weight rows x 32 k x 16 batch columns (B padded with
// zeros).  Lane l supplies row (l % 16) / column (l % 16) and the 8-value k
// block l / 16.  Lane l holds one whole 16-byte group (32 codes) of its row
// for the group g0 + l/16 of a "quad" of four groups (loaded by lane
// 4 * (l % 16) + l / 16 and passed over by ds_bpermute); word p of that
// group feeds MFMA p.  Because an MFMA then spans four different groups, each
// weight is scaled on the A side: (code - 8) * scale rounded once to
// binary16, a relative change below 2^-11 per weight.  The k order inside a
// word is the unpack order (k0,k4,k1,k5,k2,k6,k3,k7); the activation block is
// permuted in registers to match.
#include <algorithm>

#include "q4_internal.h"

namespace q4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2_t as_h2(uint32_t v) {
    return __builtin_bit_cast(half2_t, v);
}

__device__ __forceinline__ uint32_t as_u32(half2_t v) {
    return __builtin_bit_cast(uint32_t, v);
}

// Natural-order block of 8 halves -> unpack order.
__device__ __forceinline__ uint4 permute_block(uint4 v) {
    uint4 o;
    o.x = (v.x & 0xFFFFu) | (v.z << 16);
    o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    o.z = (v.y & 0xFFFFu) | (v.w << 16);
    o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return o;
}

__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
    return r;
}

// 8 codes of one 32-bit word -> 8 scaled binary16 weights in unpack order.
// `bias` (0x64006400) lives in a VGPR so each pair is one v_and_or_b32.
__device__ __forceinline__ half8_t dequant_word(uint32_t v, half2_t s2, uint32_t bias) {
    const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
    half2_t p0 = (as_h2((v & 0x000F000Fu) | bias) - off) * s2;
    half2_t p1 = (as_h2(((v >> 4) & 0x000F000Fu) | bias) - off) * s2;
    half2_t p2 = (as_h2(((v >> 8) & 0x000F000Fu) | bias) - off) * s2;
    half2_t p3 = (as_h2(((v >> 12) & 0x000F000Fu) | bias) - off) * s2;
    uint4 u = {as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)};
    return __builtin_bit_cast(half8_t, u);
}

__device__ __forceinline__ uint4 ntload16(const void *p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(1))) u32x4 global_t;
    const u32x4 v = __builtin_nontemporal_load((global_t *)p);
    return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ uint16_t ntload2(const uint16_t *p) {
    typedef const __attribute__((address_space(1))) uint16_t global_t;
    return __builtin_nontemporal_load((global_t *)p);
}

// Operands of one group quad as this lane loaded them: for each row tile a
// 16-byte group of codes and its scale (handed to their matrix-op lane by
// ds_bpermute before the multiply), and four 16-byte blocks of activations
// (rearranged through LDS before the multiply).
template <int RT>
struct Quad {
    uint4 w[RT];
    uint32_t s[RT]; // binary16 bits, zero-extended (keeps the struct in registers)
    uint4 x[4];
    bool live;      // this lane's matrix-op group exists (false: scale taken as 0)
};

// Every load is unconditional (addresses clamped into the matrix and into
// column 0 of X), so the compiler's wait counts stay exact and the next
// quad's loads remain in flight while the current quad is multiplied.  A
// group past the last one (K / 32 not a multiple of 4) gets scale 0, which
// zeroes its weights; a padding column multiplies real activations of column
// 0 and its outputs are never stored.
//
// Activations: a quad covers 256 contiguous bytes (4 groups x 32 halves) of
// each column.  Load j brings columns 4j .. 4j+3, lane l taking the 16-byte
// block l % 16 of column 4j + l / 16, so each load instruction reads whole
// cache lines; `xoff[j]` is the lane's offset (in halves) of that block in
// the quad at k = 0.
//
// Codes and scales: lane l loads group 4q + (l & 3) of row (l >> 2) of each
// row tile, so each 16-lane quarter of a load reads 64 contiguous bytes of
// four rows (a lane per row, as the matrix op's operand layout has it,
// would touch sixteen rows per quarter and four times the cache accesses);
// mma_quad moves each value to its matrix-op lane.
template <int RT>
__device__ __forceinline__ void load_quad(Quad<RT> &o, const uint8_t *const (&wrow)[RT],
                                          const uint16_t *const (&srow)[RT],
                                          const uint16_t *X16, const uint32_t (&xoff)[4], int q,
                                          int kq, int wq, int gq, int C) {
    o.live = q * 4 + kq < C; // the group of this lane's matrix-op operands
    const int gw = q * 4 + wq;
    const int gc = gw < C ? gw : C - 1;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        o.w[t] = ntload16(wrow[t] + (size_t)gc * 16);
        o.s[t] = ntload2(srow[t] + gc);
    }
    const int gx = q * 4 + gq;
    const uint32_t xg = (uint32_t)(gx < C ? gx : C - 1) * 32u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o.x[j] = gload16(X16 + xoff[j] + xg);
}

// Column stride of the per-wave activation tile in LDS, in 16-byte blocks:
// 16 blocks of data + 1 of padding, so the 16 lanes of a row reading the
// same block of 16 different columns hit 16 different bank quads.
constexpr int kXStride = 17;

// The quad's activations go through the wave's own LDS tile `xs` (column c
// at xs[c * kXStride], its 256 bytes in k order): the lane writes its four
// loaded blocks, then reads the four blocks of group kq of its column `rc`.
// Only this wave touches `xs`, and a wave's LDS operations execute in
// order, so no workgroup barrier is needed; the wave barriers keep the
// compiler from moving the reads above the writes or the next quad's writes
// above these reads.
// `perm` is the byte address of the loading lane of this lane's operands
// (row i16, group kq: lane 4 * i16 + kq) for ds_bpermute.
template <int RT>
__device__ __forceinline__ void mma_quad(const Quad<RT> &o, float4_t (&acc)[RT], uint32_t bias,
                                         uint4 *xs, int lane, int rc, int kq, int perm) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        xs[(4 * j + (lane >> 4)) * kXStride + (lane & 15)] = o.x[j];
    __builtin_amdgcn_wave_barrier();
    half8_t bop[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
        bop[p] = __builtin_bit_cast(half8_t, permute_block(xs[rc * kXStride + kq * 4 + p]));
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const uint32_t sb = (uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)o.s[t]);
        const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)(o.live ? sb : 0u));
        const half2_t s2 = {sh, sh};
        const uint32_t wd[4] = {(uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)o.w[t].x),
                                (uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)o.w[t].y),
                                (uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)o.w[t].z),
                                (uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)o.w[t].w)};
#pragma unroll
        for (int p = 0; p < 4; ++p)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant_word(wd[p], s2, bias),
                                                            bop[p], acc[t], 0, 0, 0);
    }
}

// Epilogues.  Store: Y = W X.  Acc: Y += W X (each output is written by one
// lane: no race).  SiluPair: W holds `npair` gate rows then `npair` up rows;
// the first RT/2 row tiles of a wave are gate rows and the rest the up rows
// of the same units, and the kernel writes M[b][u] = binary16(silu(g) * up)
// (silu(g) = g / (1 + exp(-g)), in fp32) instead of the fp32 products.
enum class GEpi { Store, Acc, SiluPair };

template <int RT, int NW, GEpi E>
__global__ void __launch_bounds__(64 * NW)
gemm_mfma_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
                 const uint16_t *__restrict__ X16, float *__restrict__ Y, int64_t N, int K,
                 int B, uint16_t *__restrict__ M, int64_t npair) {
    static_assert(E != GEpi::SiluPair || RT % 2 == 0, "gate and up tiles come in pairs");
    __shared__ float4_t red[NW][RT][64];
    __shared__ uint4 xs_all[NW][16 * kXStride];
    const uint32_t bias = vgpr_const(0x64006400u);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i16 = lane & 15;
    const int kq = lane >> 4;
    const int C = K >> 5;
    const int nquads = (C + 3) >> 2;
    const size_t row_bytes = (size_t)K >> 1;
    // first row (Store, Acc) or first unit (SiluPair) of this workgroup
    const int64_t row0 = (int64_t)blockIdx.x * (E == GEpi::SiluPair ? 8 * RT : 16 * RT);

    const bool bvalid = i16 < B;
    const int rc = bvalid ? i16 : 0;
    const int gq = (lane >> 2) & 3;
    const int wq = lane & 3;
    const int perm = (i16 * 4 + kq) * 4;
    uint32_t xoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = 4 * j + (lane >> 4);
        xoff[j] = (uint32_t)(c < B ? c : 0) * (uint32_t)K + (uint32_t)(lane & 3) * 8u;
    }
    uint4 *xs = xs_all[wave];

    const uint8_t *wrow[RT];
    const uint16_t *srow[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        int64_t row;
        if constexpr (E == GEpi::SiluPair) {
            const int th = t % (RT / 2);
            row = row0 + th * 16 + (lane >> 2);
            row = row < npair ? row : npair - 1;
            if (t >= RT / 2)
                row += npair;
        } else {
            row = row0 + t * 16 + (lane >> 2);
            row = row < N ? row : N - 1;
        }
        wrow[t] = W + (size_t)row * row_bytes;
        srow[t] = S + (size_t)row * C;
    }

    float4_t acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
        acc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // Two register buffers: the next quad's loads are in flight while the
    // current one is unpacked and multiplied.  Inside the loop both
    // prefetches are unconditional, so the compiler's wait before each
    // multiply covers only the quad it needs.
    Quad<RT> qa, qb;
    int q = wave;
    if (q < nquads) {
        load_quad<RT>(qa, wrow, srow, X16, xoff, q, kq, wq, gq, C);
        while (q + 2 * NW < nquads) {
            load_quad<RT>(qb, wrow, srow, X16, xoff, q + NW, kq, wq, gq, C);
            __builtin_amdgcn_sched_barrier(0); // issue before waiting for qa
            mma_quad<RT>(qa, acc, bias, xs, lane, rc, kq, perm);
            load_quad<RT>(qa, wrow, srow, X16, xoff, q + 2 * NW, kq, wq, gq, C);
            __builtin_amdgcn_sched_barrier(0);
            mma_quad<RT>(qb, acc, bias, xs, lane, rc, kq, perm);
            q += 2 * NW;
        }
        if (q + NW < nquads) {
            load_quad<RT>(qb, wrow, srow, X16, xoff, q + NW, kq, wq, gq, C);
            __builtin_amdgcn_sched_barrier(0);
            mma_quad<RT>(qa, acc, bias, xs, lane, rc, kq, perm);
            mma_quad<RT>(qb, acc, bias, xs, lane, rc, kq, perm);
        } else {
            mma_quad<RT>(qa, acc, bias, xs, lane, rc, kq, perm);
        }
    }

    if constexpr (NW > 1) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
            red[wave][t][lane] = acc[t];
        __syncthreads();
        if (wave != 0)
            return;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            float4_t v = red[0][t][lane];
            for (int w2 = 1; w2 < NW; ++w2)
                v += red[w2][t][lane];
            acc[t] = v;
        }
    }
    // D layout: lane holds rows 4*(lane/16) + 0..3 of column lane % 16.
    if (!bvalid)
        return;
    if constexpr (E == GEpi::SiluPair) {
#pragma unroll
        for (int t = 0; t < RT / 2; ++t) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t unit = row0 + t * 16 + 4 * kq + e;
                if (unit < npair) {
                    const float g = acc[t][e], up = acc[t + RT / 2][e];
                    const float silu = g / (1.0f + expf(-g));
                    M[(size_t)i16 * npair + unit] =
                        __builtin_bit_cast(uint16_t, (_Float16)(silu * up));
                }
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = row0 + t * 16 + 4 * kq + e;
                if (row < N) {
                    if constexpr (E == GEpi::Acc)
                        Y[(size_t)i16 * N + row] += acc[t][e];
                    else
                        Y[(size_t)i16 * N + row] = acc[t][e];
                }
            }
        }
    }
}

using GemmFn = void (*)(const uint8_t *, const uint16_t *, const uint16_t *, float *, int64_t,
                        int, int, uint16_t *, int64_t);

template <GEpi E>
GemmFn pick_gemm(int RT, int NW) {
#define Q4_PICK(rt, nw)                                                          \
    if (RT == rt && NW == nw)                                                    \
        return gemm_mfma_kernel<rt, nw, E>;
    if constexpr (E == GEpi::SiluPair) {
        Q4_PICK(2, 4) Q4_PICK(4, 4) Q4_PICK(8, 4)
    } else {
        Q4_PICK(1, 4) Q4_PICK(2, 4) Q4_PICK(4, 4) Q4_PICK(8, 4)
        Q4_PICK(1, 8) Q4_PICK(2, 8) Q4_PICK(4, 8)
        Q4_PICK(1, 16) Q4_PICK(2, 16)
    }
#undef Q4_PICK
    return nullptr;
}

// Row tiles per wave for a product of N rows and B columns, from a sweep
// over the 8B product shapes (6144, 4096, 28672 x 4096 and 4096 x 14336;
// B = 2, 4, 8, 16).  Every row tile a wave holds reuses the activation
// registers, so wider batches want more row tiles per wave, as long as
// about 3/4 of the CUs still get a workgroup; since the activations are
// loaded as whole lines and the codes four rows per quarter-wave, eight
// tiles no longer pay at B = 16 (28672 x 4096: 28.9 us against 28.0 with
// four).  The row tiles do not change
// any output's summation order; the k split (waves per workgroup) does, so
// it stays fixed at kGemmWaves: a column's result is then independent of B
// and of the other columns.
constexpr int kGemmWaves = 4;

int pick_row_tiles(int64_t N, int32_t B) {
    const int64_t tiles = (N + 15) / 16;
    const int cus = device_cus();
    const int rt_cap = B <= 2 ? 2 : 4;
    int RT = 1;
    while (RT * 2 <= rt_cap && tiles / (RT * 2) >= (int64_t)cus * 3 / 4)
        RT *= 2;
    return RT;
}

} // namespace

q4_status launch_gemm_mfma_cfg(const uint8_t *packed, const uint16_t *scales,
                               const uint16_t *X16, float *Y, int64_t N, int64_t K,
                               int32_t B, int RT, int NW, hipStream_t stream, bool accumulate) {
    GemmFn fn = accumulate ? pick_gemm<GEpi::Acc>(RT, NW) : pick_gemm<GEpi::Store>(RT, NW);
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED, "gemm: no kernel for row_tiles=%d waves=%d", RT, NW);
    const int64_t blocks = (N + 16 * RT - 1) / (16 * RT);
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * NW), 0, stream, packed, scales,
                       X16, Y, N, (int)K, B, nullptr, (int64_t)0);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

q4_status launch_gemm_mfma(const uint8_t *packed, const uint16_t *scales, const uint16_t *X16,
                           float *Y, int64_t N, int64_t K, int32_t B, hipStream_t stream,
                           bool accumulate) {
    if (gemv_batch_fits(B, K)) {
        EpiArgs ea{};
        ea.y = Y;
        return launch_gemv_batch(packed, scales, X16, N, K, B,
                                 accumulate ? Epi::Residual : Epi::Store, ea, stream);
    }
    return launch_gemm_mfma_cfg(packed, scales, X16, Y, N, K, B, pick_row_tiles(N, B),
                                kGemmWaves, stream, accumulate);
}

q4_status launch_gemm_silu_pair(const uint8_t *packed, const uint16_t *scales,
                                const uint16_t *X16, uint16_t *M, int64_t npair, int64_t K,
                                int32_t B, hipStream_t stream) {
    if (gemv_batch_fits(B, K)) {
        EpiArgs ea{};
        ea.out16 = M;
        ea.pair_off = npair;
        return launch_gemv_batch(packed, scales, X16, 2 * npair, K, B, Epi::SiluPair, ea,
                                 stream);
    }
    const int RT = std::max(2, pick_row_tiles(2 * npair, B));
    GemmFn fn = pick_gemm<GEpi::SiluPair>(RT, kGemmWaves);
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED, "gemm: no paired kernel for row_tiles=%d", RT);
    const int64_t blocks = (npair + 8 * RT - 1) / (8 * RT);
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * kGemmWaves), 0, stream, packed,
                       scales, X16, nullptr, 2 * npair, (int)K, B, M, npair);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace q4

extern "C" q4_status q4_gemm_smallbatch(const uint8_t *packed, const uint16_t *scales,
                                        const uint16_t *X_f16, float *Y, int64_t N,
                                        int64_t K, int32_t B, hipStream_t stream) {
    Q4_CHECK(q4::check_matrix(packed, scales, N, K, "q4_gemm_smallbatch"));
    if (!X_f16 || !Y)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_gemm_smallbatch: null X or Y");
    if (B < 1 || B > Q4_MAX_BATCH)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_gemm_smallbatch: B=%d outside [1, %d]", B,
                        Q4_MAX_BATCH);
    if (!q4::aligned(X_f16, 16) || !q4::aligned(Y, 4))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_gemm_smallbatch: X must be 16-byte and Y 4-byte aligned");
    if (B == 1) {
        q4::EpiArgs ea{};
        ea.y = Y;
        return q4::launch_gemv(packed, scales, X_f16, q4::Pro::F16, N, K, q4::Epi::Store, ea,
                              stream);
    }
    return q4::launch_gemm_mfma(packed, scales, X_f16, Y, N, K, B, stream, false);
}

extern "C" q4_status q4_gemm_tuned(const uint8_t *packed, const uint16_t *scales,
                                   const uint16_t *X_f16, float *Y, int64_t N, int64_t K,
                                   int32_t B, int32_t row_tiles, int32_t waves,
                                   hipStream_t stream) {
    Q4_CHECK(q4::check_matrix(packed, scales, N, K, "q4_gemm_tuned"));
    if (!X_f16 || !Y)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_gemm_tuned: null X or Y");
    if (B < 1 || B > Q4_MAX_BATCH)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_gemm_tuned: B=%d outside [1, %d]", B,
                        Q4_MAX_BATCH);
    if (!q4::aligned(X_f16, 16) || !q4::aligned(Y, 4))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_gemm_tuned: X must be 16-byte and Y 4-byte aligned");
    return q4::launch_gemm_mfma_cfg(packed, scales, X_f16, Y, N, K, B, row_tiles, waves,
                                    stream, false);
}

extern "C" q4_status q4_gemm_valu(const uint8_t *packed, const uint16_t *scales,
                                  const uint16_t *X_f16, float *Y, int64_t N, int64_t K,
                                  int32_t B, hipStream_t stream) {
    Q4_CHECK(q4::check_matrix(packed, scales, N, K, "q4_gemm_valu"));
    if (!X_f16 || !Y)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_gemm_valu: null X or Y");
    if (!(B == 2 || B == 3 || B == 4 || B == 8))
        return q4::fail(Q4_ERR_UNSUPPORTED, "q4_gemm_valu: B=%d not in {2, 3, 4, 8}", B);
    if (!q4::aligned(X_f16, 16) || !q4::aligned(Y, 4))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_gemm_valu: X must be 16-byte and Y 4-byte aligned");
    q4::EpiArgs ea{};
    ea.y = Y;
    return q4::launch_gemv_batch(packed, scales, X_f16, N, K, B, q4::Epi::Store, ea, stream);
}
