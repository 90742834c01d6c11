// Small-batch INT4 product Y[b] = W X[b] (2 <= B <= 16) on gfx950 matrix
// cores.
//
// Operation: PIPO: Pipelined Offloading for Efficient Inference on Consumer
// Devices, "Method", bullets "Computation optimization" and "Automatic
// configuration" -- the 4-bit kernel serves batches below 16; a batch of B
// activation vectors (e.g. a speculative-verify batch) reuses every unpacked
// weight B times.  Up to three columns (whose binary16 copies fit 64 KB of
// LDS) the dot2 kernel of q4_gemv_batch.hip is faster; beyond that its dot
// products take over the VALU, so the multiply-adds go to
// v_mfma_f32_16x16x32_f16 here and the VALU only unpacks.
//
// Arithmetic, per group g of 32 k and output (b, n): the matrix op forms
// t = sum_{k in g} (code - 8) * x_b[k] from exact binary16 operands (the
// codes enter as the small integers -8..7, never multiplied by the scale in
// binary16), and the group scale is applied to t in fp32:
// acc += float(s_g) * t.  So any finite binary16 scale, subnormal ones
// included, is applied exactly as the batch-1 product applies it.
//
// One MFMA covers one group: 16 batch columns (the A operand, B padded with
// column 0's data, never stored) x 32 k x 16 weight rows (the B operand).
// Lane l supplies column / row l % 16 and the 8-value k block l / 16, which
// is word l / 16 of the group (8 codes); the D tile leaves row l % 16 of
// the weights and batch columns 4 (l / 16) .. +3 in lane l, so every lane
// needs one scale per group.  The k order inside a word is the unpack order
// (k0,k4,k1,k5,k2,k6,k3,k7); the activation block is permuted to match.
#include <algorithm>
#include <map>
#include <mutex>

#include "q4_internal.h"
#include "q4_verify.h"

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

// 8 codes of one 32-bit word -> the 8 exact binary16 values code - 8 in
// unpack order.  (v & 0x000F000F) | 0x64006400 is the pair (1024 + c0,
// 1024 + c4); subtracting 1032 is exact.  `bias` (0x64006400) lives in a
// VGPR so each pair is one v_and_or_b32.
__device__ __forceinline__ half8_t codes_word(uint32_t v, uint32_t bias) {
    const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
    half2_t p0 = as_h2((v & 0x000F000Fu) | bias) - off;
    half2_t p1 = as_h2(((v >> 4) & 0x000F000Fu) | bias) - off;
    half2_t p2 = as_h2(((v >> 8) & 0x000F000Fu) | bias) - off;
    half2_t p3 = as_h2(((v >> 12) & 0x000F000Fu) | bias) - off;
    uint4 u = {as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)};
    return __builtin_bit_cast(half8_t, u);
}

__device__ __forceinline__ uint4 ntload16(const void *p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(1))) u32x4 global_t;
    const u32x4 v = __builtin_nontemporal_load((global_t *)p);
    return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ uint2 gload8(const void *p) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef const __attribute__((address_space(1))) u32x2 global_t;
    const u32x2 v = *(global_t *)(p);
    return uint2{v.x, v.y};
}

// Operands of one group quad as this lane loaded them.
//   w[t]: a 16-byte group of codes of row tile t: group 4q + (l & 3) of
//         row l >> 2, so each 16-lane quarter of a load reads 64 contiguous
//         bytes of four rows; mma_quad transposes them through LDS.
//   s[t]: the scales of this lane's own row (l % 16) of tile t for the four
//         groups of the quad.  SC8: one 8-byte load, s[t][0] = groups 0|1,
//         s[t][1] = groups 2|3 (binary16 pairs).  Otherwise one 2-byte load
//         per group, zero-extended into s[t][p].
//   x[j]: four 16-byte blocks of activations, rearranged through LDS.
template <int RT, bool SC8>
struct Quad {
    uint4 w[RT];
    uint32_t s[RT][SC8 ? 2 : 4];
    uint4 x[4];
};

// Every load is unconditional (addresses clamped into the matrix and into
// column 0 of X), so the compiler's wait counts stay exact and the next
// quad's loads remain in flight while the current quad is multiplied.  A
// group past the last one (K / 32 not a multiple of 4, only without SC8)
// gets scale 0 at its use; a padding column multiplies real activations of
// column 0 and its outputs are never stored.
//
// Activations: a quad covers 256 contiguous bytes (4 groups x 32 halves) of
// each column.  Load j brings columns 4j .. 4j+3, lane l taking the 16-byte
// block l % 16 of column 4j + l / 16, so each load instruction reads whole
// cache lines; `xoff[j]` is the lane's offset (in halves) of that block in
// the quad at k = 0.
template <int RT, bool SC8>
__device__ __forceinline__ void load_quad(Quad<RT, SC8> &o, const uint8_t *const (&wrow)[RT],
                                          const uint16_t *const (&srow)[RT],
                                          const uint16_t *X16, const uint32_t (&xoff)[4], int q,
                                          int wq, int gq, int C) {
    const int gw = q * 4 + wq;
    const int gc = gw < C ? gw : C - 1;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        o.w[t] = ntload16(wrow[t] + (size_t)gc * 16);
        if constexpr (SC8) {
            const uint2 v = gload8(srow[t] + (size_t)q * 4);
            o.s[t][0] = v.x;
            o.s[t][1] = v.y;
        } else {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int g = q * 4 + p;
                o.s[t][p] = gload(srow[t] + (g < C ? g : C - 1));
            }
        }
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
// Row stride of the per-wave code tile, in 32-bit words: 16 of data + 2 of
// padding, so the 32 lanes of a half-wave reading word kq of group p of
// rows 0..15 touch 32 different banks.
constexpr int kCStride = 18;

// Binary16 bits -> fp32.
__device__ __forceinline__ float h2f(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// The quad's activations go through the wave's own LDS tile `xs` (column c
// at xs[c * kXStride], its 256 bytes in k order) and its codes through the
// wave's code tile `cs` (row r of tile t at cs[(t * 16 + r) * kCStride],
// word w of group g at +4g + w): each lane writes what it loaded, then
// reads what its matrix-op lane needs -- for MFMA p (group p of the quad)
// block 4p + kq of its column and word kq of group p of its row.  Only this
// wave touches its tiles, and a wave's LDS operations execute in order, so
// no workgroup barrier is needed; the wave barriers keep the compiler from
// moving the reads above the writes or the next quad's writes above these
// reads.
template <int RT, bool SC8>
__device__ __forceinline__ void mma_quad(const Quad<RT, SC8> &o, float4_t (&acc)[RT],
                                         uint32_t bias, uint4 *xs, uint32_t *cs, int lane,
                                         int rc, int i16, int kq, int q, int C) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        xs[(4 * j + (lane >> 4)) * kXStride + (lane & 15)] = o.x[j];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        uint2 *dst = reinterpret_cast<uint2 *>(cs + (t * 16 + (lane >> 2)) * kCStride +
                                               (lane & 3) * 4);
        dst[0] = uint2{o.w[t].x, o.w[t].y};
        dst[1] = uint2{o.w[t].z, o.w[t].w};
    }
    __builtin_amdgcn_wave_barrier();
    half8_t aop[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
        aop[p] = __builtin_bit_cast(half8_t, permute_block(xs[rc * kXStride + p * 4 + kq]));
    uint32_t wd[RT][4];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int p = 0; p < 4; ++p)
            wd[t][p] = cs[(t * 16 + i16) * kCStride + p * 4 + kq];
    __builtin_amdgcn_wave_barrier();
    const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float sp;
            if constexpr (SC8)
                sp = h2f(p & 1 ? o.s[t][p >> 1] >> 16 : o.s[t][p >> 1] & 0xFFFFu);
            else
                sp = q * 4 + p < C ? h2f(o.s[t][p]) : 0.0f;
            const float4_t d =
                __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[p], codes_word(wd[t][p], bias),
                                                       zero, 0, 0, 0);
            acc[t][0] = fmaf(sp, d[0], acc[t][0]);
            acc[t][1] = fmaf(sp, d[1], acc[t][1]);
            acc[t][2] = fmaf(sp, d[2], acc[t][2]);
            acc[t][3] = fmaf(sp, d[3], acc[t][3]);
        }
    }
}

// A quad after its trip through the wave's LDS tiles: the four raw
// activation blocks and the code words the matrix-op lanes need, with the
// quad's scales.
template <int RT, bool SC8>
struct Ops {
    uint4 a[4];
    uint32_t wd[RT][4];
    uint32_t s[RT][SC8 ? 2 : 4];
};

// Writes a loaded quad to the wave's tiles and reads back its operands.
// The reads' results are first used by compute_quad, one pipeline step
// later, so their LDS latency overlaps the previous quad's matrix ops.
template <int RT, bool SC8>
__device__ __forceinline__ void stage_quad(const Quad<RT, SC8> &o, Ops<RT, SC8> &op, uint4 *xs,
                                           uint32_t *cs, int lane, int rc, int i16, int kq) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        xs[(4 * j + (lane >> 4)) * kXStride + (lane & 15)] = o.x[j];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        uint2 *dst = reinterpret_cast<uint2 *>(cs + (t * 16 + (lane >> 2)) * kCStride +
                                               (lane & 3) * 4);
        dst[0] = uint2{o.w[t].x, o.w[t].y};
        dst[1] = uint2{o.w[t].z, o.w[t].w};
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int p = 0; p < 4; ++p)
        op.a[p] = xs[rc * kXStride + p * 4 + kq];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int p = 0; p < 4; ++p)
            op.wd[t][p] = cs[(t * 16 + i16) * kCStride + p * 4 + kq];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int p = 0; p < (SC8 ? 2 : 4); ++p)
            op.s[t][p] = o.s[t][p];
    __builtin_amdgcn_wave_barrier();
}

template <int RT, bool SC8>
__device__ __forceinline__ void compute_quad(const Ops<RT, SC8> &op, float4_t (&acc)[RT],
                                             uint32_t bias, int q, int C) {
    half8_t aop[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
        aop[p] = __builtin_bit_cast(half8_t, permute_block(op.a[p]));
    const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float sp;
            if constexpr (SC8)
                sp = h2f(p & 1 ? op.s[t][p >> 1] >> 16 : op.s[t][p >> 1] & 0xFFFFu);
            else
                sp = q * 4 + p < C ? h2f(op.s[t][p]) : 0.0f;
            const float4_t d =
                __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[p], codes_word(op.wd[t][p], bias),
                                                       zero, 0, 0, 0);
            acc[t][0] = fmaf(sp, d[0], acc[t][0]);
            acc[t][1] = fmaf(sp, d[1], acc[t][1]);
            acc[t][2] = fmaf(sp, d[2], acc[t][2]);
            acc[t][3] = fmaf(sp, d[3], acc[t][3]);
        }
    }
}

// Epilogues.  Store: Y = W X.  Acc: Y += W X (each output is written by one
// lane: no race).  SiluPair: W holds `npair` gate rows then `npair` up rows;
// the first RT/2 row tiles of a wave are gate rows and the rest the up rows
// of the same units, and the kernel writes M[b][u] = binary16(silu(g) * up)
// (silu(g) = g / (1 + exp(-g)), in fp32) instead of the fp32 products.
// Rope: the QKV product whose epilogue stores the attention inputs (see
// launch_gemm_qkv_rope); its units are the row pairs (j, j + hd / 2) of a
// head, unit u = head * hd / 2 + j.
enum class GEpi { Store, Acc, SiluPair, Rope };

// Row of tile t, row-in-tile rr, for the workgroup starting at row0 (Store,
// Acc) or unit row0 (SiluPair, Rope), clamped into the matrix.
template <int RT, GEpi E>
__device__ __forceinline__ int64_t tile_row(int64_t row0, int t, int rr, int64_t N,
                                            int64_t npair, int hd = 0) {
    int64_t row;
    if constexpr (E == GEpi::SiluPair) {
        row = row0 + (t % (RT / 2)) * 16 + rr;
        row = row < npair ? row : npair - 1;
        if (t >= RT / 2)
            row += npair;
    } else if constexpr (E == GEpi::Rope) {
        int64_t unit = row0 + (t % (RT / 2)) * 16 + rr;
        unit = unit < npair ? unit : npair - 1;
        const int half = hd >> 1;
        row = (unit / half) * hd + unit % half + (t >= RT / 2 ? half : 0);
    } else {
        row = row0 + t * 16 + rr;
        row = row < N ? row : N - 1;
    }
    return row;
}

template <int RT, int NW, GEpi E, bool SC8>
__global__ void __launch_bounds__(64 * NW)
gemm_mfma_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
                 const uint16_t *__restrict__ X16, float *__restrict__ Y, int64_t N, int K,
                 int B, uint16_t *__restrict__ M, int64_t npair, GRope rp) {
    static_assert(E != GEpi::SiluPair || RT % 2 == 0, "gate and up tiles come in pairs");
    static_assert(E != GEpi::Rope || RT == 2, "a rotation pair is one tile and its partner");
    // Per wave: the activation tile (16 x kXStride blocks) and the code tile
    // (RT * 16 x kCStride words); after the loop the same memory holds the
    // k-split partial sums.
    constexpr int kWaveWords = 16 * kXStride * 4 + RT * 16 * kCStride;
    constexpr int kTileWords = NW * kWaveWords;
    constexpr int kRedWords = NW * RT * 64 * 4;
    __shared__ uint4 lds_raw[((kTileWords > kRedWords ? kTileWords : kRedWords) + 3) / 4];
    const uint32_t bias = vgpr_const(0x64006400u);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i16 = lane & 15;
    const int kq = lane >> 4;
    const int C = K >> 5;
    const int nquads = (C + 3) >> 2;
    const size_t row_bytes = (size_t)K >> 1;
    // first row (Store, Acc) or first unit (SiluPair, Rope) of this workgroup
    const int64_t row0 =
        (int64_t)blockIdx.x * (E == GEpi::SiluPair || E == GEpi::Rope ? 8 * RT : 16 * RT);
    const int pos0 = E == GEpi::Rope ? *rp.pos_dev : 0;

    const int rc = i16 < B ? i16 : 0; // column whose activations this lane supplies
    const int gq = (lane >> 2) & 3;
    const int wq = lane & 3;
    uint32_t xoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = 4 * j + (lane >> 4);
        xoff[j] = (uint32_t)(c < B ? c : 0) * (uint32_t)K + (uint32_t)(lane & 3) * 8u;
    }
    uint32_t *wave_lds = reinterpret_cast<uint32_t *>(lds_raw) + wave * kWaveWords;
    uint4 *xs = reinterpret_cast<uint4 *>(wave_lds);
    uint32_t *cs = wave_lds + 16 * kXStride * 4;

    const uint8_t *wrow[RT];
    const uint16_t *srow[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        wrow[t] = W + (size_t)tile_row<RT, E>(row0, t, lane >> 2, N, npair, rp.hd) * row_bytes;
        srow[t] = S + (size_t)tile_row<RT, E>(row0, t, i16, N, npair, rp.hd) * C;
    }

    float4_t acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
        acc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // One row tile per wave (the 4096-row products: one workgroup per CU,
    // one wave per SIMD, nothing else to hide a wave's latencies): a
    // three-step pipeline per quad -- global loads into a register quad (two
    // buffers), the LDS transpose into operand registers (two buffers), the
    // matrix ops.  Step j loads quad j + 2, stages quad j + 1 and multiplies
    // quad j, so each quad's loads have one step to land and its LDS reads
    // overlap the previous quad's matrix ops (B = 16: 4096 x 4096 6.8 us
    // against 7.2, 4096 x 14336 17.2 against 18.5; with more row tiles the
    // extra registers cost more occupancy than the overlap gains).  The same
    // operations in the same order per quad as the loop below: the bits do
    // not change.
    if constexpr (RT == 1) {
        Quad<RT, SC8> q0b, q1b;
        Ops<RT, SC8> o0, o1;
        if (wave < nquads) {
            const int nqw = (nquads - 1 - wave) / NW + 1;
            auto quad = [&](int j) { return wave + NW * j; };
            int j = 0;
            load_quad<RT, SC8>(q0b, wrow, srow, X16, xoff, quad(0), wq, gq, C);
            __builtin_amdgcn_sched_barrier(0);
            load_quad<RT, SC8>(q1b, wrow, srow, X16, xoff, quad(nqw > 1 ? 1 : 0), wq, gq, C);
            __builtin_amdgcn_sched_barrier(0);
            stage_quad<RT, SC8>(q0b, o0, xs, cs, lane, rc, i16, kq);
            while (j + 3 < nqw) {
                load_quad<RT, SC8>(q0b, wrow, srow, X16, xoff, quad(j + 2), wq, gq, C);
                __builtin_amdgcn_sched_barrier(0);
                stage_quad<RT, SC8>(q1b, o1, xs, cs, lane, rc, i16, kq);
                compute_quad<RT, SC8>(o0, acc, bias, quad(j), C);
                load_quad<RT, SC8>(q1b, wrow, srow, X16, xoff, quad(j + 3), wq, gq, C);
                __builtin_amdgcn_sched_barrier(0);
                stage_quad<RT, SC8>(q0b, o0, xs, cs, lane, rc, i16, kq);
                compute_quad<RT, SC8>(o1, acc, bias, quad(j + 1), C);
                j += 2;
            }
            if (j + 2 < nqw) {
                load_quad<RT, SC8>(q0b, wrow, srow, X16, xoff, quad(j + 2), wq, gq, C);
                __builtin_amdgcn_sched_barrier(0);
                stage_quad<RT, SC8>(q1b, o1, xs, cs, lane, rc, i16, kq);
                compute_quad<RT, SC8>(o0, acc, bias, quad(j), C);
                stage_quad<RT, SC8>(q0b, o0, xs, cs, lane, rc, i16, kq);
                compute_quad<RT, SC8>(o1, acc, bias, quad(j + 1), C);
                compute_quad<RT, SC8>(o0, acc, bias, quad(j + 2), C);
            } else if (j + 1 < nqw) {
                stage_quad<RT, SC8>(q1b, o1, xs, cs, lane, rc, i16, kq);
                compute_quad<RT, SC8>(o0, acc, bias, quad(j), C);
                compute_quad<RT, SC8>(o1, acc, bias, quad(j + 1), C);
            } else {
                compute_quad<RT, SC8>(o0, acc, bias, quad(j), C);
            }
        }
    } else {
        // Two register buffers: the next quad's loads are in flight while the
        // current one is unpacked and multiplied.  Inside the loop both
        // prefetches are unconditional, so the compiler's wait before each
        // multiply covers only the quad it needs.
        Quad<RT, SC8> qa, qb;
        int q = wave;
        if (q < nquads) {
            load_quad<RT, SC8>(qa, wrow, srow, X16, xoff, q, wq, gq, C);
            while (q + 2 * NW < nquads) {
                load_quad<RT, SC8>(qb, wrow, srow, X16, xoff, q + NW, wq, gq, C);
                __builtin_amdgcn_sched_barrier(0); // issue before waiting for qa
                mma_quad<RT, SC8>(qa, acc, bias, xs, cs, lane, rc, i16, kq, q, C);
                load_quad<RT, SC8>(qa, wrow, srow, X16, xoff, q + 2 * NW, wq, gq, C);
                __builtin_amdgcn_sched_barrier(0);
                mma_quad<RT, SC8>(qb, acc, bias, xs, cs, lane, rc, i16, kq, q + NW, C);
                q += 2 * NW;
            }
            if (q + NW < nquads) {
                load_quad<RT, SC8>(qb, wrow, srow, X16, xoff, q + NW, wq, gq, C);
                __builtin_amdgcn_sched_barrier(0);
                mma_quad<RT, SC8>(qa, acc, bias, xs, cs, lane, rc, i16, kq, q, C);
                mma_quad<RT, SC8>(qb, acc, bias, xs, cs, lane, rc, i16, kq, q + NW, C);
            } else {
                mma_quad<RT, SC8>(qa, acc, bias, xs, cs, lane, rc, i16, kq, q, C);
            }
        }
    }

    // Rope: the rotation table entries of the lane's unit at the positions
    // of its four columns, loaded before the k-split merge
    float2 rcs[4];
    if constexpr (E == GEpi::Rope) {
        const int half = rp.hd >> 1;
        int64_t unit = row0 + i16;
        unit = unit < npair ? unit : npair - 1;
        const int d = (int)(unit % half);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int b = 4 * kq + e < B ? 4 * kq + e : B - 1;
            rcs[e] = rp.rope[(size_t)(pos0 + b) * half + d];
        }
    }

    if constexpr (NW > 1) {
        float4_t *red = reinterpret_cast<float4_t *>(lds_raw); // [NW][RT][64]
        __syncthreads(); // every wave is done with its tiles
#pragma unroll
        for (int t = 0; t < RT; ++t)
            red[(wave * RT + t) * 64 + lane] = acc[t];
        __syncthreads();
        if (wave != 0)
            return;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            float4_t v = red[t * 64 + lane];
            for (int w2 = 1; w2 < NW; ++w2)
                v += red[(w2 * RT + t) * 64 + lane];
            acc[t] = v;
        }
    }
    // D layout: lane holds weight row i16 of each tile for batch columns
    // 4 * kq + 0..3.
    if constexpr (E == GEpi::Rope) {
        // the unrotated rows to Y; then the rotate-half rotation of the pair
        // (a, b) in fp32 from the table entry (cos, sin): query heads to
        // qrot, key heads rounded to binary16 into the key cache, value heads
        // rounded into the value cache, at row *pos_dev + column
        const int half = rp.hd >> 1;
        const int64_t unit = row0 + i16;
        const int head = (int)(unit / half), d = (int)(unit % half);
        const size_t ra = (size_t)head * rp.hd + d;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int b = 4 * kq + e;
            if (unit < npair && b < B) {
                const float a = acc[0][e], bb = acc[1][e];
                Y[(size_t)b * N + ra] = a;
                Y[(size_t)b * N + ra + half] = bb;
                const float2 cs = rcs[e];
                const float r0 = a * cs.x - bb * cs.y, r1 = a * cs.y + bb * cs.x;
                if (head < rp.nq) {
                    float *q = rp.qrot + (size_t)b * rp.nq * rp.hd + ra;
                    q[0] = r0;
                    q[half] = r1;
                } else if (head < rp.nq + rp.nkv) {
                    uint16_t *k = rp.kc +
                                  ((size_t)(head - rp.nq) * rp.max_ctx + pos0 + b) * rp.hd + d;
                    k[0] = __builtin_bit_cast(uint16_t, (_Float16)r0);
                    k[half] = __builtin_bit_cast(uint16_t, (_Float16)r1);
                } else {
                    uint16_t *v =
                        rp.vc +
                        ((size_t)(head - rp.nq - rp.nkv) * rp.max_ctx + pos0 + b) * rp.hd + d;
                    v[0] = __builtin_bit_cast(uint16_t, (_Float16)a);
                    v[half] = __builtin_bit_cast(uint16_t, (_Float16)bb);
                }
            }
        }
    } else if constexpr (E == GEpi::SiluPair) {
#pragma unroll
        for (int t = 0; t < RT / 2; ++t) {
            const int64_t unit = row0 + t * 16 + i16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int b = 4 * kq + e;
                if (unit < npair && b < B) {
                    const float g = acc[t][e], up = acc[t + RT / 2][e];
                    const float silu = g / (1.0f + expf(-g));
                    M[(size_t)b * npair + unit] =
                        __builtin_bit_cast(uint16_t, (_Float16)(silu * up));
                }
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int64_t row = row0 + t * 16 + i16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int b = 4 * kq + e;
                if (row < N && b < B) {
                    if constexpr (E == GEpi::Acc)
                        Y[(size_t)b * N + row] += acc[t][e];
                    else
                        Y[(size_t)b * N + row] = acc[t][e];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Activation-resident launch: one workgroup per compute unit holds the whole
// activation X[B][K] in LDS and walks a contiguous, balanced range of row
// tiles; used where every compute unit gets four or more tiles (the 28672-row
// gate+up product: 7 tiles each on 256 units).
//
// Staging: direct-to-LDS loads (no registers), each reading 1 KB of one
// column into a column-major area (column stride 1 mod 8 blocks of 16
// bytes), then one in-place pass that puts every 8-half block into the
// matrix op's k order.  A wave then reads group g of its column l % 16,
// block l / 16, as one 16-byte LDS read without bank conflicts.
//
// Waves: 4 NS per workgroup -- four k quarters (wave w takes quads w, w + 4,
// ... exactly as gemm_mfma_kernel does, and the quarters' partial sums are
// added in quarter order) times NS sets taking alternate tiles.  Every quad
// is multiplied with the same operations in the same order as there, so
// both kernels give the same bits.  What differs is the data movement: the
// activation is read from the caches once per compute unit instead of once
// per wave, quad and row block, it needs no per-quad rearranging, and a
// wave's registers carry only codes and scales, so xres_ring quads of them
// are in flight.  Paired rows (SiluPair) use tiles of 8 gate rows and the 8
// up rows of the same units, so their tiles divide as evenly as 8-unit
// steps allow (14336 units: 1792 tiles).
// Measured on the 8B gate+up shape (28672 x 4096, µs, against the row-tile
// launch on the same box): B = 4 23.1 / 24.6, B = 8 21.6 / 24.6, B = 16
// 23.0 / 25.9.  With one or two tiles per unit (QKV, O) one workgroup per
// unit has too little to hide its staging (O at B = 16: 11 µs against 6.7),
// so those keep the row-tile launch.
//
// LDS: [0, xa) the activation; then one code tile per wave; then the
// partial sums of every tile but the sets' last ones, per k quarter (the
// last tiles' stay in registers and go through the activation area at the
// end).
constexpr int kXresWaves = 4; // the k split, as in gemm_mfma_kernel
constexpr int kCTileBytes = 16 * kCStride * 4;
// Blocks per staged activation column: the column's 4 C blocks plus 1..8
// of padding, so that consecutive columns start 16 bytes further along the
// LDS banks (stride = 1 mod 8 blocks) and the 16 columns one matrix-op read
// touches fall into different banks.
__host__ __device__ constexpr int xres_col_blocks(int C) {
    return C * 4 + ((1 - C * 4) % 8 + 8) % 8;
}
constexpr int kPartBytes = 64 * 16;
// NS wave sets take tiles set, set + NS, ...; quads in flight per wave
// (registers: two sets may hold 256 VGPRs a wave, four 128; six quads in
// flight with four sets measured slower than four).
template <int NS>
constexpr int xres_ring() {
    return NS <= 2 ? 8 : 4;
}
// Four sets (16 waves, four per SIMD) measured ahead of two on the gate+up
// shape (B = 4: 23.7 against 25.4 µs, B = 8: 22.4 against 23.2).
constexpr int kXresSetsUsed = 4;

// Codes and scales of one quad for one lane, as gemm_mfma_kernel loads them
// for one row tile (lane l: group 4q + l % 4 of tile row l / 4; the scales
// of tile row l % 16).
template <bool SC8>
struct WSlot {
    uint4 w;
    uint32_t s[SC8 ? 2 : 4];
};

// Matrix row of tile row rr (0..15) of tile t, clamped into the matrix.
// SiluPair: rows 0..7 gate rows of units 8t .. 8t+7, rows 8..15 their up
// rows (npair further on).
template <GEpi E>
__device__ __forceinline__ int64_t xres_row(int64_t t, int rr, int64_t N, int64_t npair) {
    if constexpr (E == GEpi::SiluPair) {
        int64_t unit = t * 8 + (rr & 7);
        unit = unit < npair ? unit : npair - 1;
        return rr >= 8 ? unit + npair : unit;
    } else {
        const int64_t row = t * 16 + rr;
        return row < N ? row : N - 1;
    }
}

// Plain loads for the codes: the two 64-byte halves of a 128-byte line of a
// row belong to neighbouring quads, read by two k quarters of the same
// workgroup; with non-temporal loads the line was often gone from L2 when
// the second half was read (1.16 x the weight bytes fetched from HBM on the
// gate+up shape, and 3-6% slower).
template <bool SC8>
__device__ __forceinline__ void xres_load(WSlot<SC8> &o, const uint8_t *wrow,
                                          const uint16_t *srow, int q, int wq, int C) {
    const int gw = q * 4 + wq;
    o.w = gload16(wrow + (size_t)(gw < C ? gw : C - 1) * 16);
    if constexpr (SC8) {
        const uint2 v = gload8(srow + (size_t)q * 4);
        o.s[0] = v.x;
        o.s[1] = v.y;
    } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int g = q * 4 + p;
            o.s[p] = gload(srow + (g < C ? g : C - 1));
        }
    }
}

// A quad's operands after staging: the raw activation blocks, the code
// words of the matrix-op lanes and the group scales already widened to fp32
// (the exact conversion compute_quad applies; done here, it consumes the
// loaded scale registers in the step that waits for them, so a ring slot's
// registers are free to be refilled and the compiler has no loaded value to
// carry around the loop).
struct XOps {
    uint4 a[4];
    uint32_t wd[4];
    float sf[4];
};

// Binary16 bits (low half) -> fp32, as an instruction the compiler cannot
// fold into the multiply-adds (v_fma_mix_f32 would keep the loaded scale
// registers live up to the matrix ops); the same exact conversion.
__device__ __forceinline__ float h2f_now(uint32_t bits) {
    float r;
    asm volatile("v_cvt_f32_f16 %0, %1" : "=v"(r) : "v"(bits));
    return r;
}

// Codes of a loaded quad through the wave's code tile into the matrix-op
// lanes (as stage_quad does), activation blocks straight from the staged
// activation.
// xl = rc * xres_col_blocks(C) + kq: the lane's block within group 0 of
// its column; the group offset 4 g is wave-uniform.
template <bool SC8>
__device__ __forceinline__ void xres_stage(const WSlot<SC8> &o, XOps &op, const uint4 *xs,
                                           uint32_t *cs, int lane, int xl, int i16, int kq,
                                           int q, int C, int B) {
    uint2 *dst = reinterpret_cast<uint2 *>(cs + (lane >> 2) * kCStride + (lane & 3) * 4);
    dst[0] = uint2{o.w.x, o.w.y};
    dst[1] = uint2{o.w.z, o.w.w};
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int g = q * 4 + p;
        op.a[p] = xs[(g < C ? g : C - 1) * 4 + xl];
    }
#pragma unroll
    for (int p = 0; p < 4; ++p)
        op.wd[p] = cs[i16 * kCStride + p * 4 + kq];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        if constexpr (SC8)
            op.sf[p] = h2f_now(p & 1 ? o.s[p >> 1] >> 16 : o.s[p >> 1]);
        else
            op.sf[p] = q * 4 + p < C ? h2f_now(o.s[p]) : 0.0f;
    }
    __builtin_amdgcn_wave_barrier();
}

// compute_quad for one row tile with the scales staged in fp32 and the
// activation blocks already in unpack order: the same operations in the
// same order.
__device__ __forceinline__ void xres_compute(const XOps &op, float4_t &acc, uint32_t bias) {
    half8_t aop[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
        aop[p] = __builtin_bit_cast(half8_t, op.a[p]);
    // the four matrix ops first (independent, so they overlap), then the
    // scales in group order
    const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    float4_t d[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
        d[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[p], codes_word(op.wd[p], bias), zero,
                                                     0, 0, 0);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        acc[0] = fmaf(op.sf[p], d[p][0], acc[0]);
        acc[1] = fmaf(op.sf[p], d[p][1], acc[1]);
        acc[2] = fmaf(op.sf[p], d[p][2], acc[2]);
        acc[3] = fmaf(op.sf[p], d[p][3], acc[3]);
    }
}

template <GEpi E, bool SC8, int NS>
__global__ void __launch_bounds__(64 * kXresWaves * NS)
gemm_xres_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
                 const uint16_t *__restrict__ X16, float *__restrict__ Y, int64_t N, int K,
                 int B, uint16_t *__restrict__ M, int64_t npair, int64_t ntiles, int xa) {
    constexpr int kXresSets = NS;
    constexpr int kXresThreads = 64 * kXresWaves * NS;
    constexpr int kXresRing = xres_ring<NS>();
    static_assert(kXresRing % 2 == 0, "the staged operands alternate between two buffers");
    extern __shared__ uint4 xres_lds[];
    uint8_t *lds8 = reinterpret_cast<uint8_t *>(xres_lds);
    const uint4 *xs = xres_lds;
    const uint32_t bias = vgpr_const(0x64006400u);
    const int lane = threadIdx.x & 63;
    // wave wid: k quarter `wave`, tile set `set` (tiles set, set + 2, ...)
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave = wid % kXresWaves;
    const int set = wid / kXresWaves;
    const int i16 = lane & 15;
    const int kq = lane >> 4;
    const int wq = lane & 3;
    const int C = K >> 5;
    const int SB = xres_col_blocks(C);
    const int xl = (i16 < B ? i16 : 0) * SB + kq;
    const int nquads = (C + 3) >> 2;
    const size_t row_bytes = (size_t)K >> 1;
    uint32_t *cs = reinterpret_cast<uint32_t *>(lds8 + xa + wid * kCTileBytes);
    float4_t *red =
        reinterpret_cast<float4_t *>(lds8 + xa + kXresWaves * kXresSets * kCTileBytes);

    const int64_t t0 = (int64_t)blockIdx.x * ntiles / gridDim.x;
    const int ntl = (int)((int64_t)(blockIdx.x + 1) * ntiles / gridDim.x - t0);
    const int nts = set < ntl ? (ntl - set + kXresSets - 1) / kXresSets : 0; // this set's tiles
    const int nqw = wave < nquads ? (nquads - 1 - wave) / kXresWaves + 1 : 0;
    const int nitems = nqw * nts;

    // Stage the activation column by column: each direct-to-LDS load reads
    // 64 consecutive 16-byte blocks (1 KB) of one column into consecutive
    // LDS blocks; lanes past the column's end are masked off.
    const int ncb = C * 4;              // blocks per column
    const int nic = (ncb + 63) >> 6;    // loads per column
    {
        typedef const void __attribute__((address_space(1))) *gptr_t;
        typedef void __attribute__((address_space(3))) *lptr_t;
        for (int k = wid; k < B * nic; k += kXresWaves * kXresSets) {
            const int b = k / nic, j = k - b * nic;
            const int blk = j * 64 + lane;
            if (blk < ncb)
                __builtin_amdgcn_global_load_lds(
                    (gptr_t)(X16 + (size_t)b * K + (size_t)blk * 8),
                    (lptr_t)(lds8 + ((size_t)b * SB + j * 64) * 16), 16, 0, 0);
        }
    }

    // Load stream (item li: the set's tile lt, quad index lj of this wave),
    // clamped to the wave's last item; every slot refill is unconditional.
    int lt = 0, lj = 0, li = 0;
    const int64_t tset = t0 + (set < ntl ? set : ntl - 1);
    const uint8_t *wrow = W + (size_t)xres_row<E>(tset, lane >> 2, N, npair) * row_bytes;
    const uint16_t *srow = S + (size_t)xres_row<E>(tset, i16, N, npair) * C;
    auto load_next = [&](WSlot<SC8> &slot) {
        const int q = wave + kXresWaves * lj; // a wave without quads reloads the last
        xres_load<SC8>(slot, wrow, srow, q < nquads ? q : nquads - 1, wq, C);
        if (li + 1 < nitems) {
            ++li;
            if (++lj == nqw) {
                lj = 0;
                ++lt;
                const int64_t t = tset + (int64_t)kXresSets * lt;
                wrow = W + (size_t)xres_row<E>(t, lane >> 2, N, npair) * row_bytes;
                srow = S + (size_t)xres_row<E>(t, i16, N, npair) * C;
            }
        }
    };

    WSlot<SC8> ring[kXresRing];
#pragma unroll
    for (int d = 0; d < kXresRing; ++d) {
        load_next(ring[d]);
        __builtin_amdgcn_sched_barrier(0);
    }
    // vmcnt(0) (gfx9 encoding, other counters unconstrained): this wave's
    // activation blocks have landed (and its first quads with them)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    // Every block into the matrix op's k order, once, in place.
    for (int b = 0; b < B; ++b)
        for (int blk = threadIdx.x; blk < ncb; blk += kXresThreads)
            xres_lds[(size_t)b * SB + blk] = permute_block(xres_lds[(size_t)b * SB + blk]);
    __syncthreads();

    const float4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    float4_t acc[1] = {zero4};
    // stage side: quad index sj of the next item; compute side: the set's
    // tile ct, quad index cj
    int sj = 0, ct = 0, cj = 0;
    // Staging runs every step, past the wave's last item too (it then
    // stages a copy of the last item, never multiplied): with it under a
    // condition the compiler could no longer count the LDS reads in flight
    // and waited for all of them before every quad's matrix ops.
    XOps ops[2];
    if (nitems > 0) {
        xres_stage<SC8>(ring[0], ops[0], xs, cs, lane, xl, i16, kq, wave, C, B);
        sj = nqw > 1 ? 1 : 0;
    }
    load_next(ring[0]);
    for (int base = 0; base < nitems; base += kXresRing) {
#pragma unroll
        for (int d = 0; d < kXresRing; ++d) {
            const int i = base + d;
            xres_stage<SC8>(ring[(d + 1) % kXresRing], ops[(d + 1) & 1], xs, cs, lane, xl, i16,
                            kq, wave + kXresWaves * sj, C, B);
            if (i + 1 < nitems && ++sj == nqw)
                sj = 0;
            // the slot's old registers are consumed before its refill is
            // issued, so the refill reuses them (otherwise the compiler
            // renames them and copies them back at the loop's end, where it
            // must wait for every load in flight)
            __builtin_amdgcn_sched_barrier(0);
            load_next(ring[(d + 1) % kXresRing]);
            __builtin_amdgcn_sched_barrier(0);
            if (i < nitems) {
                xres_compute(ops[d & 1], acc[0], bias);
                if (++cj == nqw) {
                    cj = 0;
                    if (ct < nts - 1) { // not the set's last tile
                        red[((set + kXresSets * ct) * kXresWaves + wave) * 64 + lane] = acc[0];
                        acc[0] = zero4;
                    }
                    ++ct;
                }
            }
        }
    }
    if (nqw == 0) {
        for (int j = 0; j + 1 < nts; ++j)
            red[((set + kXresSets * j) * kXresWaves + wave) * 64 + lane] = zero4;
    }
    __syncthreads(); // every wave is done with the activation and its code tile
    // The sets' last tiles are the workgroup's last NS (tl >= ntl - NS);
    // their partial sums go through the start of the activation area.
    float4_t *last = reinterpret_cast<float4_t *>(lds8);
    last[wid * 64 + lane] = acc[0];
    __syncthreads();

    // Tile tl's sum over the k quarters, in quarter order, as
    // gemm_mfma_kernel adds them; wave wid finishes the tiles wid, wid + 4 NS, ...
    auto part = [&](int tl, int w2, int l) -> float4_t {
        return tl >= ntl - NS ? last[((tl % kXresSets) * kXresWaves + w2) * 64 + l]
                              : red[(tl * kXresWaves + w2) * 64 + l];
    };
    for (int tl = wid; tl < ntl; tl += kXresWaves * kXresSets) {
        const int64_t t = t0 + tl;
        float4_t v = part(tl, 0, lane);
#pragma unroll
        for (int w2 = 1; w2 < kXresWaves; ++w2)
            v += part(tl, w2, lane);
        if constexpr (E == GEpi::SiluPair) {
            float4_t u = part(tl, 0, lane + 8 < 64 ? lane + 8 : lane);
#pragma unroll
            for (int w2 = 1; w2 < kXresWaves; ++w2)
                u += part(tl, w2, lane + 8 < 64 ? lane + 8 : lane);
            const int64_t unit = t * 8 + i16;
            if (i16 < 8 && unit < npair) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int b = 4 * kq + e;
                    if (b < B) {
                        const float g = v[e], up = u[e];
                        const float silu = g / (1.0f + expf(-g));
                        M[(size_t)b * npair + unit] =
                            __builtin_bit_cast(uint16_t, (_Float16)(silu * up));
                    }
                }
            }
        } else {
            const int64_t row = t * 16 + i16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int b = 4 * kq + e;
                if (row < N && b < B) {
                    if constexpr (E == GEpi::Acc)
                        Y[(size_t)b * N + row] += v[e];
                    else
                        Y[(size_t)b * N + row] = v[e];
                }
            }
        }
    }
}

using GemmFn = void (*)(const uint8_t *, const uint16_t *, const uint16_t *, float *, int64_t,
                        int, int, uint16_t *, int64_t, GRope);

using GemmXresFn = void (*)(const uint8_t *, const uint16_t *, const uint16_t *, float *,
                            int64_t, int, int, uint16_t *, int64_t, int64_t, int);

template <GEpi E, bool SC8>
GemmFn pick_gemm_sc(int RT, int NW) {
#define Q4_PICK(rt, nw)                                                          \
    if (RT == rt && NW == nw)                                                    \
        return gemm_mfma_kernel<rt, nw, E, SC8>;
    if constexpr (E == GEpi::SiluPair) {
        Q4_PICK(2, 4) Q4_PICK(4, 4) Q4_PICK(8, 4)
    } else if constexpr (E == GEpi::Rope) {
        Q4_PICK(2, 4) Q4_PICK(2, 8)
    } else {
        Q4_PICK(1, 4) Q4_PICK(2, 4) Q4_PICK(4, 4) Q4_PICK(8, 4)
        Q4_PICK(1, 8) Q4_PICK(2, 8) Q4_PICK(4, 8)
        Q4_PICK(1, 16) Q4_PICK(2, 16)
    }
#undef Q4_PICK
    return nullptr;
}

// The scales of a row quad are read with one 8-byte load when every row's
// scale array starts 8-byte aligned (K / 32 a multiple of 4 and an aligned
// base), else one 2-byte load per group.
template <GEpi E>
GemmFn pick_gemm(int RT, int NW, int64_t K, const uint16_t *scales) {
    const bool sc8 = (K / 32) % 4 == 0 && aligned(scales, 8);
    return sc8 ? pick_gemm_sc<E, true>(RT, NW) : pick_gemm_sc<E, false>(RT, NW);
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
// it depends on the shape only (kGemmWaves, or pick_waves below): a
// column's result is then independent of B and of the other columns.
constexpr int kGemmWaves = 4;

// Products of at most one row tile per compute unit (the 4096-row O and
// down products on 256 units) split k eight ways instead: more waves share
// each unit's few rows (µs, eight / four waves: O 4096 x 4096 at B = 4
// 5.98 / 6.83, B = 8 6.09 / 6.63, B = 16 6.61 / 6.73; down 4096 x 14336
// 13.7 / 17.4, 14.4 / 16.7, 16.9 / 17.2; QKV 6144 rows and wider products
// gain nothing).  Decided by the shape alone, so every column's result
// stays independent of B.
int pick_waves(int64_t N) {
    return (N + 15) / 16 <= device_cus() ? 8 : kGemmWaves;
}

int pick_row_tiles(int64_t N, int32_t B) {
    const int64_t tiles = (N + 15) / 16;
    const int cus = device_cus();
    const int rt_cap = B <= 2 ? 2 : 4;
    int RT = 1;
    while (RT * 2 <= rt_cap && tiles / (RT * 2) >= (int64_t)cus * 3 / 4)
        RT *= 2;
    return RT;
}


// Activation-resident launch shape: one workgroup per compute unit (at most
// one per tile), each holding the activation, the code tiles and the partial
// sums of all its tiles but the last.  grid == 0: it does not fit in the
// LDS one workgroup may take, and the row-tile launch above is used (same
// bits).
struct XresCfg {
    int grid = 0;
    int xa = 0;
    int sets = 0;
    size_t lds = 0;
    int64_t ntiles = 0;
};

template <GEpi E, bool SC8, int NS>
GemmXresFn xres_fn() {
    return gemm_xres_kernel<E, SC8, NS>;
}

// The largest LDS allocation one workgroup may opt into on the current
// device, with every activation-resident kernel opted in (once per device).
size_t xres_lds_limit() {
    static std::mutex mu;
    static std::map<int, size_t> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(dev);
    if (it != cache.end())
        return it->second;
    int max_lds = 0, optin = 0;
    if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
        hipSuccess)
        max_lds = 0;
    if (hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev) !=
        hipSuccess)
        optin = 0;
    size_t lim = (size_t)std::max(max_lds, optin);
    for (GemmXresFn fn :
         {xres_fn<GEpi::Store, true, kXresSetsUsed>(), xres_fn<GEpi::Store, false, kXresSetsUsed>(),
          xres_fn<GEpi::Acc, true, kXresSetsUsed>(), xres_fn<GEpi::Acc, false, kXresSetsUsed>(),
          xres_fn<GEpi::SiluPair, true, kXresSetsUsed>(),
          xres_fn<GEpi::SiluPair, false, kXresSetsUsed>()})
        if (hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lim) != hipSuccess)
            lim = std::min<size_t>(lim, 65536);
    cache[dev] = lim;
    return lim;
}

// rows: N (Store, Acc) or the unit count npair (SiluPair, 8 units a tile).
XresCfg xres_config(int64_t rows, int64_t K, int32_t B, bool paired) {
    XresCfg c;
    const int64_t C = K / 32;
    const int64_t xa = ((int64_t)B * xres_col_blocks((int)C) * 16 + 1023) / 1024 * 1024;
    c.ntiles = paired ? (rows + 7) / 8 : (rows + 15) / 16;
    const int64_t grid = std::min<int64_t>(device_cus(), c.ntiles);
    const int64_t maxt = (c.ntiles + grid - 1) / grid;
    if (maxt < kXresSetsUsed)
        return c; // a tile or two per compute unit: the row-tile launch is faster
    const int sets = kXresSetsUsed;
    const size_t lds = (size_t)xa + kXresWaves * sets * kCTileBytes +
                       (size_t)std::max<int64_t>(maxt - sets, 0) * kXresWaves * kPartBytes;
    if (grid < 1 || lds > xres_lds_limit())
        return c;
    c.grid = (int)grid;
    c.xa = (int)xa;
    c.sets = sets;
    c.lds = lds;
    return c;
}

template <GEpi E>
GemmXresFn pick_xres(int64_t K, const uint16_t *scales) {
    const bool sc8 = (K / 32) % 4 == 0 && aligned(scales, 8);
    return sc8 ? xres_fn<E, true, kXresSetsUsed>() : xres_fn<E, false, kXresSetsUsed>();
}

q4_status launch_xres(GemmXresFn fn, const XresCfg &c, const uint8_t *packed,
                      const uint16_t *scales, const uint16_t *X16, float *Y, int64_t N,
                      int64_t K, int32_t B, uint16_t *M, int64_t npair, hipStream_t stream) {
    hipLaunchKernelGGL(fn, dim3((unsigned)c.grid), dim3(64 * kXresWaves * c.sets), c.lds, stream,
                       packed,
                       scales, X16, Y, N, (int)K, B, M, npair, c.ntiles, c.xa);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace

q4_status launch_gemm_mfma_cfg(const uint8_t *packed, const uint16_t *scales,
                               const uint16_t *X16, float *Y, int64_t N, int64_t K,
                               int32_t B, int RT, int NW, hipStream_t stream, bool accumulate) {
    GemmFn fn = accumulate ? pick_gemm<GEpi::Acc>(RT, NW, K, scales)
                             : pick_gemm<GEpi::Store>(RT, NW, K, scales);
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED, "gemm: no kernel for row_tiles=%d waves=%d", RT, NW);
    const int64_t blocks = (N + 16 * RT - 1) / (16 * RT);
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * NW), 0, stream, packed, scales,
                       X16, Y, N, (int)K, B, nullptr, (int64_t)0, GRope{});
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
    const XresCfg c = xres_config(N, K, B, false);
    if (c.grid > 0)
        return launch_xres(accumulate ? pick_xres<GEpi::Acc>(K, scales)
                                      : pick_xres<GEpi::Store>(K, scales),
                           c, packed, scales, X16, Y, N, K, B, nullptr, 0, stream);
    return launch_gemm_mfma_cfg(packed, scales, X16, Y, N, K, B, pick_row_tiles(N, B),
                                pick_waves(N), stream, accumulate);
}

// Three columns take the activation-resident launch where it applies: the
// vector-ALU kernel's paired form needs 171 registers there (two waves per
// SIMD), and the 8B verify step at three columns took 1.82 ms with it
// against 1.72 ms with the matrix cores.
bool silu_pair_on_valu(int64_t npair, int64_t K, int32_t B) {
    return gemv_batch_fits(B, K) && !(B == 3 && xres_config(npair, K, B, true).grid > 0);
}

q4_status launch_gemm_silu_pair(const uint8_t *packed, const uint16_t *scales,
                                const uint16_t *X16, uint16_t *M, int64_t npair, int64_t K,
                                int32_t B, hipStream_t stream) {
    if (silu_pair_on_valu(npair, K, B)) {
        EpiArgs ea{};
        ea.out16 = M;
        ea.pair_off = npair;
        return launch_gemv_batch(packed, scales, X16, 2 * npair, K, B, Epi::SiluPair, ea,
                                 stream);
    }
    const XresCfg c = xres_config(npair, K, B, true);
    if (c.grid > 0)
        return launch_xres(pick_xres<GEpi::SiluPair>(K, scales), c, packed, scales, X16,
                           nullptr, 2 * npair, K, B, M, npair, stream);
    const int RT = std::max(2, pick_row_tiles(2 * npair, B));
    GemmFn fn = pick_gemm<GEpi::SiluPair>(RT, kGemmWaves, K, scales);
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED, "gemm: no paired kernel for row_tiles=%d", RT);
    const int64_t blocks = (npair + 8 * RT - 1) / (8 * RT);
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * kGemmWaves), 0, stream, packed,
                       scales, X16, nullptr, 2 * npair, (int)K, B, M, npair, GRope{});
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

q4_status launch_gemm_qkv_rope(const uint8_t *packed, const uint16_t *scales,
                               const uint16_t *X16, float *Y, int64_t N, int64_t K, int32_t B,
                               const GRope &rp, hipStream_t stream, bool *stored) {
    *stored = false;
    // the vector-ALU and activation-resident launches keep their plain
    // epilogue; the caller appends the rows after them
    if (gemv_batch_fits(B, K) || xres_config(N, K, B, false).grid > 0)
        return launch_gemm_mfma(packed, scales, X16, Y, N, K, B, stream);
    if (rp.hd < 32 || rp.hd % 32 || N != (int64_t)(rp.nq + 2 * rp.nkv) * rp.hd)
        return fail(Q4_ERR_INVALID_ARG, "gemm: rotary rows need N == (H + 2 Hkv) * hd");
    const int NW = pick_waves(N);
    GemmFn fn = pick_gemm<GEpi::Rope>(2, NW, K, scales);
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED, "gemm: no rotary kernel for waves=%d", NW);
    const int64_t npair = N / 2;
    const int64_t blocks = (npair + 15) / 16;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * NW), 0, stream, packed, scales,
                       X16, Y, N, (int)K, B, nullptr, npair, rp);
    Q4_HIP(hipGetLastError());
    *stored = true;
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
