// INT4 matrix-vector products with one row per wave instruction.
//
// Operation: PIPO: Pipelined Offloading for Efficient Inference on Consumer
// Devices, "Method", bullet "Computation optimization" -- the vector is
// multiplied directly by the 4-bit weights; no dequantized matrix is ever
// written.  Unpack and per-chunk arithmetic are those of q4_gemv.hip.
//
// Work decomposition (our own for CDNA4).  Every wave works alone after the
// workgroup has staged the activation: no k split, no workgroup barrier in
// the loop.  A wave takes R rows at a time; lane l reads the 16-byte chunks
// (groups of 32 codes) l, l + 64, ... of each row, so one load instruction
// covers 1 KB of one row -- a linear sweep, which the HBM streams faster
// than several shorter runs of different rows.  A row total is a 64-lane
// DPP/permlane sum.
//   gemv_row_kernel   K <= 4096 (at most two chunks per lane): all chunks of
//                     a group in flight at once, the lane's activation
//                     chunks copied from LDS into registers once;
//   gemv_rowp_kernel  wider rows: a group's chunks in phases of PH chunks
//                     per lane (the wave's registers hold one phase), the
//                     activation read from LDS chunk by chunk;
//   gemv_row_batch_kernel  2..4 (8) binary16 columns staged in LDS; up to
//                     K = 4096 and three columns every column's activation
//                     chunks of the lane held in registers as above, wider
//                     rows or batches in phases read from LDS.
// The workgroup stages the activation, or its RMSNorm, once with linear
// loads, with the staging code of the other product kernel (the same bits).
//
// Summation order of one output: per lane, its chunks in increasing order
// (each chunk: exact binary16 products summed by v_dot2_f32_f16, then the
// group scale in fp32), then the fixed 64-lane sum.  All three kernels keep
// exactly this order, whatever R, PH or the grid: a product's bits do not
// depend on its launch shape, and each column of a 2..4-column product
// equals the batch-1 product of that column bitwise.
#include <algorithm>

#include "q4_gemv_core.h"
#include "q4_lanes.h"
#include "q4_verify.h"

namespace q4 {
namespace {

constexpr int kRowWaves = 4;
constexpr int kRowThreads = 64 * kRowWaves;
static_assert(kRowThreads == kThreads, "the staging code assumes the product's workgroup");

// Sum over the 64 lanes with identical bits in every lane: every step adds
// a value and its partner's in the same order on both sides (quad xor
// pairs, half-row and row mirrors, then the row and half-wave swaps), so a
// row total can be stored from any lane -- the batch kernel stores column b
// of row r from another lane than the batch-1 kernels do.
__device__ __forceinline__ float wave_total(float x) {
    x = row16_sum(x);
    const lanes::Rows16 r(x);
    x = lanes::fa(r.a) + lanes::fa(r.b);
    const lanes::Halves32 h(x);
    return lanes::fa(h.a) + lanes::fa(h.b);
}

// Chunks first, first + 1, ... of this lane: index lane + 64 j, clamped into
// the row (loads stay in bounds); `valid` marks the real ones (a clamped
// chunk gets scale 0, so it adds exactly nothing).
template <int NC>
struct RowChunks {
    int c[NC];
    bool valid[NC];
};

template <int NC>
__device__ __forceinline__ RowChunks<NC> row_chunks(int lane, int C, int first = 0) {
    RowChunks<NC> g;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = lane + 64 * (first + j);
        g.valid[j] = c < C;
        g.c[j] = c < C ? c : C - 1;
    }
    return g;
}

// Output units per group of R rows: SiluPair pairs gate row u with up row
// u + pair_off, QkvRope row j of a head with row j + hd / 2 (the two halves
// the rotation mixes), so R rows hold R / 2 units.
template <Epi E, int R>
constexpr int units_per_group() {
    return E == Epi::SiluPair || E == Epi::QkvRope ? R / 2 : R;
}

// Matrix row of row slot r of group g (units past the end repeat the last).
template <Epi E, int R>
__device__ __forceinline__ int64_t group_row(int64_t g, int r, int64_t n_units,
                                             const EpiArgs &ea) {
    constexpr int UP = units_per_group<E, R>();
    int64_t unit = g * UP + r % UP;
    unit = unit < n_units ? unit : n_units - 1;
    if constexpr (E == Epi::SiluPair) {
        return unit + (r / UP) * ea.pair_off;
    } else if constexpr (E == Epi::QkvRope) {
        const int half = ea.hd >> 1;
        const int u = (int)unit;
        return (int64_t)(u / half) * ea.hd + u % half + (r / UP) * half;
    } else {
        return unit;
    }
}

// Loads of the chunks `ch` of the R rows of group g.  Always all NC of
// them (a phase past the row's end loads its clamped last chunk): with
// loads under a condition the compiler can no longer count the ones in
// flight and waits for all before the first product (the 4096 x 14336
// product of a decoder layer took 11.3 us that way against 8.5).
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

// Residual epilogue: the old value of the row that this lane stores in
// group g (lane r stores row r); 0 for the other epilogues.
template <int R, Epi E>
__device__ __forceinline__ float residual_of(const EpiArgs &ea, int64_t g, int lane,
                                             int64_t n_units) {
    if constexpr (E == Epi::Residual)
        return gload(ea.y + group_row<E, R>(g, lane < R ? lane : 0, n_units, ea));
    else
        return 0.0f;
}

// QkvRope: the rotation table entry (cos, sin) of the unit that this lane
// stores in group g (lane i stores unit i) at position pos; read with the
// group's weights, so the store does not wait for it.  (0, 0) otherwise.
template <int R, Epi E>
__device__ __forceinline__ float2 rope_of(const EpiArgs &ea, int64_t g, int lane,
                                          int64_t n_units, int pos) {
    if constexpr (E == Epi::QkvRope) {
        constexpr int UP = units_per_group<E, R>();
        int64_t unit = g * UP + (lane < UP ? lane : 0);
        unit = unit < n_units ? unit : n_units - 1;
        const int half = ea.hd >> 1;
        return ea.rope[(size_t)pos * half + (int)unit % half];
    } else {
        return make_float2(0.0f, 0.0f);
    }
}

// Writes the row totals of group g (every lane holds them) through
// epilogue E: lane r stores row r, SiluPair and QkvRope lane i unit i.
template <int R, Epi E>
__device__ __forceinline__ void group_store(const float (&tot)[R], int64_t g, int lane,
                                            float hcur, int64_t N, int64_t n_units,
                                            const EpiArgs &ea, float2 cs = {}, int pos = 0) {
    constexpr int UP = units_per_group<E, R>();
    if constexpr (E == Epi::QkvRope) {
        // The unrotated rows to y as every QKV product stores them; then
        // the rotate-half rotation of the pair (a, b) at angle pos * base^(-2d/hd)
        // for query and key heads, in fp32 from the table entry (cos, sin):
        // query heads to qrot, key heads rounded to binary16 into the key
        // cache; value heads rounded into the value cache.
        const int half = ea.hd >> 1;
#pragma unroll
        for (int i = 0; i < UP; ++i) {
            const int64_t unit = g * UP + i;
            if (lane == i && unit < n_units) {
                const int u = (int)unit;
                const int head = u / half, d = u % half;
                const float a = tot[i], b = tot[i + UP];
                const size_t ra = (size_t)head * ea.hd + d;
                ea.y[ra] = a;
                ea.y[ra + half] = b;
                const float r0 = a * cs.x - b * cs.y, r1 = a * cs.y + b * cs.x;
                if (head < ea.n_q_heads) {
                    ea.qrot[ra] = r0;
                    ea.qrot[ra + half] = r1;
                } else if (head < ea.n_q_heads + ea.n_kv_heads) {
                    uint16_t *k = ea.kc +
                                  ((size_t)(head - ea.n_q_heads) * ea.max_ctx + pos) * ea.hd + d;
                    k[0] = f32_to_f16(r0);
                    k[half] = f32_to_f16(r1);
                } else {
                    uint16_t *v =
                        ea.vc +
                        ((size_t)(head - ea.n_q_heads - ea.n_kv_heads) * ea.max_ctx + pos) *
                            ea.hd +
                        d;
                    v[0] = f32_to_f16(a);
                    v[half] = f32_to_f16(b);
                }
            }
        }
    } else if constexpr (E == Epi::SiluPair) {
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
}

// NC (<= 2) chunks per lane, R rows per group, epilogue E, prologue P.
// Grid: waves take groups wave, wave + total waves, ...  The first group's
// loads go out between the activation loads and the staging arithmetic;
// every later group's after the previous group's stores (issued before
// them they cost registers and time).
template <int NC, int R, Epi E, Pro P>
__global__ void __launch_bounds__(kRowThreads)
gemv_row_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
                const void *__restrict__ xin, int64_t N, int K, int64_t n_units, EpiArgs ea) {
    static_assert((E != Epi::SiluPair && E != Epi::QkvRope) || R % 2 == 0,
                  "paired rows come in pairs");
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
    const int pos = E == Epi::QkvRope ? *ea.pos_dev : 0;
    const uint32_t bias = vgpr_const(0x64006400u);
    const RowChunks<NC> ch = row_chunks<NC>(lane, C);

    XStage st;
    stage_issue<P, false>(xin, K, st);
    uint4 w[R][NC];
    uint16_t s[R][NC];
    const int64_t g0 = g < ngroups ? g : ngroups - 1;
    group_loads<NC, R, E>(W, S, C, n_units, ea, g0, ch, w, s);
    float hv = residual_of<R, E>(ea, g0, lane, n_units);
    float2 cs = rope_of<R, E>(ea, g0, lane, n_units, pos);
    stage_finish<P, false>(xin, xs, K, ea, wsum, st);
    __syncthreads();
    if (g >= ngroups)
        return; // no barrier below: a wave without rows simply leaves
    uint4 xq[NC][4];
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
        for (int p = 0; p < 4; ++p)
            xq[j][p] = xs[p * C + ch.c[j]];

    while (true) {
        float tot[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            tot[r] = 0.0f;
#pragma unroll
            for (int j = 0; j < NC; ++j)
                tot[r] = chunk_acc(w[r][j], xq[j], ch.valid[j] ? f16_to_f32(s[r][j]) : 0.0f,
                                   tot[r], bias);
        }
        // every row's lane sum first, then the R wave sums, so that their
        // DPP chains can interleave
#pragma unroll
        for (int r = 0; r < R; ++r)
            tot[r] = wave_total(tot[r]);
        group_store<R, E>(tot, g, lane, hv, N, n_units, ea, cs, pos);
        g += nwaves;
        if (g >= ngroups)
            break;
        group_loads<NC, R, E>(W, S, C, n_units, ea, g, ch, w, s);
        hv = residual_of<R, E>(ea, g, lane, n_units);
        cs = rope_of<R, E>(ea, g, lane, n_units, pos);
    }
}

// Wide rows: the wave walks each group of R rows in phases of PH chunks per
// lane (load the phase, multiply it; its registers hold one phase), the
// activation read from LDS chunk by chunk.  The first phase of the first
// group is loaded before the staging arithmetic, as above.
template <int PH, int R, Epi E, Pro P>
__global__ void __launch_bounds__(kRowThreads)
gemv_rowp_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
                 const void *__restrict__ xin, int64_t N, int K, int64_t n_units, EpiArgs ea) {
    static_assert((E != Epi::SiluPair && E != Epi::QkvRope) || R % 2 == 0,
                  "paired rows come in pairs");
    constexpr int UP = units_per_group<E, R>();
    extern __shared__ uint4 xs[];
    __shared__ float wsum[kWaves];
    const int lane = threadIdx.x & 63;
    const int64_t wave =
        __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kRowWaves + (threadIdx.x >> 6)));
    const int64_t nwaves = (int64_t)gridDim.x * kRowWaves;
    const int C = K >> 5;
    const int pos = E == Epi::QkvRope ? *ea.pos_dev : 0;
    const int nc = (C + 63) / 64;       // chunks per lane
    const int nph = (nc + PH - 1) / PH; // phases per group
    const int64_t ngroups = (n_units + UP - 1) / UP;
    const uint32_t bias = vgpr_const(0x64006400u);
    int64_t g = wave;

    XStage st;
    stage_issue<P, false>(xin, K, st);
    uint4 w[R][PH];
    uint16_t s[R][PH];
    RowChunks<PH> ch = row_chunks<PH>(lane, C);
    const int64_t g0 = g < ngroups ? g : ngroups - 1;
    group_loads<PH, R, E>(W, S, C, n_units, ea, g0, ch, w, s);
    float hv = residual_of<R, E>(ea, g0, lane, n_units);
    float2 cs = rope_of<R, E>(ea, g0, lane, n_units, pos);
    stage_finish<P, false>(xin, xs, K, ea, wsum, st);
    __syncthreads();
    if (g >= ngroups)
        return; // no barrier below: a wave without rows simply leaves

    while (true) {
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = 0.0f;
        for (int ph = 0; ph < nph; ++ph) {
            const int live = min(PH, nc - ph * PH);
            if (ph > 0) {
                ch = row_chunks<PH>(lane, C, ph * PH);
                group_loads<PH, R, E>(W, S, C, n_units, ea, g, ch, w, s);
            }
#pragma unroll
            for (int i = 0; i < PH; ++i) {
                if (i < live) {
                    uint4 xj[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        xj[p] = xs[p * C + ch.c[i]];
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[r] = chunk_acc(w[r][i], xj, ch.valid[i] ? f16_to_f32(s[r][i]) : 0.0f,
                                           acc[r], bias);
                }
            }
        }
        float tot[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            tot[r] = wave_total(acc[r]);
        group_store<R, E>(tot, g, lane, hv, N, n_units, ea, cs, pos);
        g += nwaves;
        if (g >= ngroups)
            break;
        ch = row_chunks<PH>(lane, C);
        group_loads<PH, R, E>(W, S, C, n_units, ea, g, ch, w, s);
        hv = residual_of<R, E>(ea, g, lane, n_units);
        cs = rope_of<R, E>(ea, g, lane, n_units, pos);
    }
}

// Residual epilogue of the batch kernel: the old value of the output that
// this lane stores in group g (lane r * B + b stores row r of column b).
template <int R, int B, Epi E>
__device__ __forceinline__ float batch_residual_of(const EpiArgs &ea, int64_t N, int64_t g,
                                                   int lane, int64_t n_units) {
    if constexpr (E == Epi::Residual) {
        const int l = lane < R * B ? lane : 0;
        return gload(ea.y + (size_t)(l % B) * N + group_row<E, R>(g, l / B, n_units, ea));
    } else {
        return 0.0f;
    }
}

// RMSNorm prologue of the batch kernel for B fp32 columns h[B][K], K <=
// 4096, four waves: per column exactly the single-token prologue's
// operations in its order (thread t sums the squares of its blocks t,
// t + 256 in that order, then the wave sums and the four wave totals in
// wave order), so every column stages the bits its token alone would.
// Loads: issued by rmsnorm_issue before the weights; blocks past the
// column's end wrap around (no load behind a per-lane branch).
constexpr int kNormBlocks = 2; // blocks of 8 values per thread and column (K <= 4096)

template <int B>
struct NormStage {
    uint4 v[B][kNormBlocks][2];
};

template <int B>
__device__ __forceinline__ void rmsnorm_issue(const float *h, int K, NormStage<B> &st) {
    const int nb8 = K >> 3;
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int j = 0; j < kNormBlocks; ++j) {
            const int i = threadIdx.x + j * kThreads;
            const float *p = h + (size_t)b * K + 8 * (size_t)(i < nb8 ? i : i % nb8);
            st.v[b][j][0] = gload16(p);
            st.v[b][j][1] = gload16(p + 4);
        }
}

template <int B>
__device__ __forceinline__ void rmsnorm_finish(uint4 *xs, int K, const EpiArgs &ea,
                                               float (*wsum)[kWaves], const NormStage<B> &st) {
    const int C = K >> 5;
    const int nb8 = K >> 3;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < kNormBlocks; ++j) {
            if (threadIdx.x + j * kThreads < nb8) {
                float f[8];
                unpack_f32x8(st.v[b][j][0], st.v[b][j][1], f);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    ss = fmaf(f[i], f[i], ss);
            }
        }
        ss = wave_sum(ss);
        if ((threadIdx.x & 63) == 0)
            wsum[b][threadIdx.x >> 6] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float tot = wsum[b][0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            tot += wsum[b][w];
        const float r = 1.0f / sqrtf(tot / (float)K + eps_of(ea));
#pragma unroll
        for (int j = 0; j < kNormBlocks; ++j) {
            const int i = threadIdx.x + j * kThreads;
            if (i < nb8) {
                float f[8];
                unpack_f32x8(st.v[b][j][0], st.v[b][j][1], f);
                uint32_t p[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    p[q] = (uint32_t)f32_to_f16(f[2 * q] * r) |
                           ((uint32_t)f32_to_f16(f[2 * q + 1] * r) << 16);
                xs[(size_t)b * 4 * C + (i & 3) * C + (i >> 2)] =
                    permute8(uint4{p[0], p[1], p[2], p[3]});
            }
        }
    }
}

// B columns staged in LDS (pair order, [B][4][C]): binary16 columns
// X16[B][K] (P = F16), or the RMSNorm of fp32 columns h[B][K] (P =
// RmsNorm, with XR and four waves; ea.eps).  Per column the batch-1
// kernels' arithmetic and order, the chunks in phases of PH per lane.  XR
// (PH = all chunks of a lane, K <= 4096): the lane's activation chunks of
// every column copied from LDS into registers once, as the batch-1 kernel
// does, and each row unpacked once per chunk for all columns; otherwise
// every chunk's column pairs are read from LDS.  WV waves per workgroup:
// more where the staged columns leave room for few workgroups per compute
// unit.  Store / Residual: ea.y = Y f32 [B][N]; SiluPair: ea.out16 = M
// binary16 [B][pair_off].
template <int PH, int R, int B, Epi E, int WV, bool XR, Pro P>
__global__ void __launch_bounds__(64 * WV)
gemv_row_batch_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
                      const void *__restrict__ xin, int64_t N, int K, int64_t n_units,
                      EpiArgs ea) {
    static_assert(E != Epi::SiluPair || R % 2 == 0, "paired rows come in pairs");
    static_assert(!XR || PH <= 2, "register-held activations: at most two chunks per lane");
    static_assert(P == Pro::F16 || (XR && WV == kWaves), "the norm prologue: XR, four waves");
    constexpr int UP = units_per_group<E, R>();
    extern __shared__ uint4 xs[];
    const uint16_t *X16 = static_cast<const uint16_t *>(xin);
    const int lane = threadIdx.x & 63;
    const int64_t wave =
        __builtin_amdgcn_readfirstlane((int)(blockIdx.x * WV + (threadIdx.x >> 6)));
    const int64_t nwaves = (int64_t)gridDim.x * WV;
    const int C = K >> 5;
    const int nb = K >> 3; // 8-value blocks per column
    const int nc = (C + 63) / 64;
    const int nph = XR ? 1 : (nc + PH - 1) / PH;
    const int64_t ngroups = (n_units + UP - 1) / UP;
    // The columns' first SB blocks per thread are loaded before the weights,
    // as the batch-1 kernels stage theirs: a wave's loads complete in issue
    // order, so staging loads issued after the weights would wait for them.
    // Indices past the end wrap around (no load behind a per-lane branch);
    // blocks beyond SB per thread are staged after the weights by a loop.
    constexpr int kT = 64 * WV;
    constexpr int SB = P == Pro::RmsNorm ? 1 : XR ? (B * 512 + kT - 1) / kT : 8;
    const int nblk = B * nb;
    uint4 sv[SB];
    NormStage<P == Pro::RmsNorm ? B : 1> nst;
    if constexpr (P == Pro::RmsNorm) {
        rmsnorm_issue<B>(static_cast<const float *>(xin), K, nst);
    } else {
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int i = threadIdx.x + j * kT;
            sv[j] = gload16(X16 + 8 * (size_t)(i < nblk ? i : i % nblk));
        }
    }
    uint4 w[R][PH];
    uint16_t s[R][PH];
    RowChunks<PH> ch = row_chunks<PH>(lane, C);
    int64_t g = wave;
    const int64_t g0 = g < ngroups ? g : ngroups - 1;
    group_loads<PH, R, E>(W, S, C, n_units, ea, g0, ch, w, s);
    float hv = batch_residual_of<R, B, E>(ea, N, g0, lane, n_units);
    if constexpr (P == Pro::RmsNorm) {
        __shared__ float wsum[B][kWaves];
        rmsnorm_finish<B>(xs, K, ea, wsum, nst);
    } else {
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int i = threadIdx.x + j * kT;
            if (i < nblk) {
                const int b = i / nb, k8 = i - b * nb;
                xs[(size_t)b * 4 * C + (k8 & 3) * C + (k8 >> 2)] = permute8(sv[j]);
            }
        }
    }
    if constexpr (!XR) { // XR: SB covers every block of K <= 4096
        for (int i = threadIdx.x + SB * kT; i < nblk; i += kT) {
            const int b = i / nb, k8 = i - b * nb;
            xs[(size_t)b * 4 * C + (k8 & 3) * C + (k8 >> 2)] =
                permute8(gload16(X16 + 8 * (size_t)i));
        }
    }
    __syncthreads();
    if (g >= ngroups)
        return;
    const uint32_t bias = vgpr_const(0x64006400u);
    const half2_t off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2_t off_hi = {(_Float16)1152.0f, (_Float16)1152.0f};
    uint4 xr[XR ? B : 1][XR ? PH : 1][4];
    if constexpr (XR) {
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int j = 0; j < PH; ++j)
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    xr[b][j][p] = xs[(size_t)b * 4 * C + p * C + ch.c[j]];
    }
    while (true) {
        float acc[R][B];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b)
                acc[r][b] = 0.0f;
        for (int ph = 0; ph < nph; ++ph) {
            const int live = XR ? PH : min(PH, nc - ph * PH);
            if (!XR && ph > 0) {
                ch = row_chunks<PH>(lane, C, ph * PH);
                group_loads<PH, R, E>(W, S, C, n_units, ea, g, ch, w, s);
            }
#pragma unroll
            for (int j = 0; j < PH; ++j) {
                if (j >= live)
                    continue;
                if constexpr (XR) {
                    // one row at a time: its chunk unpacked once, then
                    // multiplied with every column's registers
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        half2_t q[16];
                        const uint4 wv = w[r][j];
                        const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t v = wd[i], u = v >> 8;
                            q[4 * i + 0] = as_h2((v & 0x000F000Fu) | bias) - off_lo;
                            q[4 * i + 1] = as_h2((v & 0x00F000F0u) | bias) - off_hi;
                            q[4 * i + 2] = as_h2((u & 0x000F000Fu) | bias) - off_lo;
                            q[4 * i + 3] = as_h2((u & 0x00F000F0u) | bias) - off_hi;
                        }
                        const float sc = ch.valid[j] ? f16_to_f32(s[r][j]) : 0.0f;
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            float tlo = 0.0f, thi = 0.0f;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                tlo = __builtin_amdgcn_fdot2(q[4 * i + 0], as_h2(xr[b][j][i].x),
                                                             tlo, false);
                                thi = __builtin_amdgcn_fdot2(q[4 * i + 1], as_h2(xr[b][j][i].y),
                                                             thi, false);
                                tlo = __builtin_amdgcn_fdot2(q[4 * i + 2], as_h2(xr[b][j][i].z),
                                                             tlo, false);
                                thi = __builtin_amdgcn_fdot2(q[4 * i + 3], as_h2(xr[b][j][i].w),
                                                             thi, false);
                            }
                            acc[r][b] = fmaf(sc, fmaf(thi, 0.0625f, tlo), acc[r][b]);
                        }
                    }
                } else {
                    half2_t q[R][16];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint4 wv = w[r][j];
                        const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
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
                                tlo = __builtin_amdgcn_fdot2(q[r][4 * i + 0], as_h2(xq[i].x),
                                                             tlo, false);
                                thi = __builtin_amdgcn_fdot2(q[r][4 * i + 1], as_h2(xq[i].y),
                                                             thi, false);
                                tlo = __builtin_amdgcn_fdot2(q[r][4 * i + 2], as_h2(xq[i].z),
                                                             tlo, false);
                                thi = __builtin_amdgcn_fdot2(q[r][4 * i + 3], as_h2(xq[i].w),
                                                             thi, false);
                            }
                            acc[r][b] = fmaf(sc, fmaf(thi, 0.0625f, tlo), acc[r][b]);
                        }
                    }
                }
            }
        }
        const int64_t gn = g + nwaves;
        float hvn = 0.0f;
        if (gn < ngroups) {
            if constexpr (!XR)
                ch = row_chunks<PH>(lane, C);
            group_loads<PH, R, E>(W, S, C, n_units, ea, gn, ch, w, s);
            hvn = batch_residual_of<R, B, E>(ea, N, gn, lane, n_units);
        }
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
                            *y = hv + acc[r][b];
                        else
                            *y = acc[r][b];
                    }
                }
        }
        if (gn >= ngroups)
            break;
        hv = hvn;
        g = gn;
    }
}

using RowFn = void (*)(const uint8_t *, const uint16_t *, const void *, int64_t, int, int64_t,
                       EpiArgs);
using RowBatchFn = void (*)(const uint8_t *, const uint16_t *, const void *, int64_t, int,
                            int64_t, EpiArgs);

template <Epi E, Pro P>
RowFn pick_row(int NC, int R) {
#define Q4_PICK(nc, r)                                                                   \
    if (NC == nc && R == r)                                                              \
        return gemv_row_kernel<nc, r, E, P>;
    Q4_PICK(1, 2) Q4_PICK(1, 4) Q4_PICK(2, 2) Q4_PICK(2, 4)
#undef Q4_PICK
    return nullptr;
}

// Phased kernels: the launch shapes row_config picks, and for Store every
// shape the measurement entry offers.  Paired rows (SiluPair) keep the
// pipelined kernel of q4_gemv.hip for K > 4096, so none is built for them.
template <Epi E, Pro P>
RowFn pick_rowp(int PH, int R) {
#define Q4_PICK(ph, r)                                                                   \
    if (PH == ph && R == r)                                                              \
        return gemv_rowp_kernel<ph, r, E, P>;
    if constexpr (E == Epi::Store) {
        Q4_PICK(1, 1) Q4_PICK(2, 1) Q4_PICK(4, 1) Q4_PICK(7, 1)
        Q4_PICK(1, 2) Q4_PICK(2, 2) Q4_PICK(4, 2) Q4_PICK(7, 2)
        Q4_PICK(2, 4) Q4_PICK(4, 4)
    } else if constexpr (E == Epi::QkvRope) {
        Q4_PICK(1, 2) Q4_PICK(4, 2) Q4_PICK(7, 2)
    } else if constexpr (E != Epi::SiluPair) {
        Q4_PICK(1, 2) Q4_PICK(4, 1) Q4_PICK(7, 1)
    }
#undef Q4_PICK
    return nullptr;
}

// PH == 0: the all-chunks kernel with NC chunks per lane.
template <Epi E, Pro P>
RowFn pick_shape(int NC, int PH, int R) {
    return PH == 0 ? pick_row<E, P>(NC, R) : pick_rowp<E, P>(PH, R);
}

RowFn pick_any(Epi e, Pro p, int NC, int PH, int R) {
    if (p == Pro::RmsNorm) {
        switch (e) {
        case Epi::QkvGather: return pick_shape<Epi::QkvGather, Pro::RmsNorm>(NC, PH, R);
        case Epi::SiluPair: return pick_shape<Epi::SiluPair, Pro::RmsNorm>(NC, PH, R);
        case Epi::QkvRope: return pick_shape<Epi::QkvRope, Pro::RmsNorm>(NC, PH, R);
        default: return nullptr;
        }
    }
    switch (e) {
    case Epi::Store: return pick_shape<Epi::Store, Pro::F16>(NC, PH, R);
    case Epi::Residual: return pick_shape<Epi::Residual, Pro::F16>(NC, PH, R);
    case Epi::QkvGather: return pick_shape<Epi::QkvGather, Pro::F16>(NC, PH, R);
    case Epi::SiluPair: return pick_shape<Epi::SiluPair, Pro::F16>(NC, PH, R);
    case Epi::QkvRope: return nullptr; // always behind the RMSNorm prologue
    }
    return nullptr;
}

// Launch shape of the 2..8-column product (PH chunks per phase, R rows per
// group, WV waves per workgroup, XR register-held activations), from
// graph-replayed launches over weight copies larger than the last-level
// cache (us at two columns, 8B shapes):
//   K <= 4096: two rows per group; at two and three columns the activation
//     in registers (4096 x 4096: 4.8 against 5.3 from LDS, 6144 x 4096 6.2
//     against 6.5); four rows per group hold too many registers (28672 x
//     4096: 20.4 against 18.7 at two rows);
//   K >= 12288 (two columns fill 56 KB of LDS, two workgroups per compute
//     unit): one row in phases of seven with eight waves per workgroup
//     (4096 x 14336: 12.3-12.7 against 18.5 with four waves and 13.0 with
//     two rows per group).
struct BatchCfg {
    int PH, R, WV;
    bool XR;
};

BatchCfg batch_config(int64_t K, int B) {
    const int nc = (int)((K / 32 + 63) / 64);
    if (nc <= 2)
        return BatchCfg{nc, 2, 4, B <= 3};
    if (nc >= 7)
        return BatchCfg{7, 1, 8, false};
    return BatchCfg{4, 2, 4, false};
}

// RMSNorm prologue (P = RmsNorm): the register-held shapes of the products
// that follow a norm in the verify step (QKV: Store; gate+up: SiluPair).
template <Epi E>
RowBatchFn pick_row_batch_norm(const BatchCfg &c, int B) {
#define Q4_PICK(ph, b)                                                                   \
    if (c.PH == ph && c.R == 2 && B == b && c.WV == kWaves && c.XR)                      \
        return gemv_row_batch_kernel<ph, 2, b, E, kWaves, true, Pro::RmsNorm>;
    if constexpr (E == Epi::Store || E == Epi::SiluPair) {
        Q4_PICK(1, 2) Q4_PICK(1, 3) Q4_PICK(2, 2) Q4_PICK(2, 3)
    }
#undef Q4_PICK
    return nullptr;
}

template <Epi E>
RowBatchFn pick_row_batch(const BatchCfg &c, int B) {
#define Q4_PICK(ph, r, b, wv, xr)                                                        \
    if (c.PH == ph && c.R == r && B == b && c.WV == wv && c.XR == xr)                    \
        return gemv_row_batch_kernel<ph, r, b, E, wv, xr, Pro::F16>;
    // two chunks or fewer per lane, two or three columns: registers
    Q4_PICK(1, 2, 2, 4, true) Q4_PICK(1, 2, 3, 4, true)
    Q4_PICK(2, 2, 2, 4, true) Q4_PICK(2, 2, 3, 4, true)
    // four columns (eight for Store) at K <= 4096, and K = 8192
    Q4_PICK(1, 2, 4, 4, false) Q4_PICK(2, 2, 4, 4, false)
    Q4_PICK(4, 2, 2, 4, false) Q4_PICK(4, 2, 3, 4, false) Q4_PICK(4, 2, 4, 4, false)
    if constexpr (E == Epi::Store) {
        Q4_PICK(1, 2, 8, 4, false) Q4_PICK(2, 2, 8, 4, false) Q4_PICK(4, 2, 8, 4, false)
    }
    // seven or more chunks per lane (two columns fit the stage up to K = 16384)
    if constexpr (E != Epi::SiluPair) {
        Q4_PICK(7, 1, 2, 8, false)
    }
#undef Q4_PICK
    return nullptr;
}


// Launch shape of the batch-1 product by its shape (NC chunks per lane; PH
// 0 for the all-chunks kernel, else chunks per phase; R rows per group;
// grid workgroups, 0 for the default), from back-to-back timings of each
// shape (a graph of launches over weight copies larger than the last-level
// cache):
//   K <= 4096: all chunks in flight, four rows per group for tall products
//     (28672 x 4096: 13.1 us against 13.7 with two), two otherwise (4096 x
//     4096: 4.1 against 4.4);
//   K >= 12288 (seven or more chunks per lane): one row in phases of seven
//     (4096 x 14336: 8.5 us against 9.4 in phases of four and 9.6 with the
//     kernel of q4_gemv.hip), 512 workgroups from K = 24576 (8192 x 28672:
//     26.0 against 29.0 with one group per wave);
//   otherwise (K = 8192 in the models): up to 8192 rows two rows in phases
//     of one (8192 x 8192: 9.7 against 10.3), else one row in phases of four
//     (10240 x 8192: 10.7 against 12.0).
struct RowCfg {
    int NC, PH, R, grid;
};

RowCfg row_config(int64_t rows, int64_t K) {
    const int nc = (int)((K / 32 + 63) / 64);
    if (nc <= 2)
        return RowCfg{nc, 0, rows >= 16384 ? 4 : 2, 0};
    if (nc >= 7)
        return RowCfg{nc, 7, 1, K >= 24576 ? 512 : 0};
    if (rows <= 8192)
        return RowCfg{nc, 1, 2, 0};
    return RowCfg{nc, 4, 1, 0};
}

// Workgroups: one group of rows per wave, at most `grid` (default four per
// compute unit: 10240 x 8192 took 11.7 us at 1024 workgroups against 12.6
// at 1280).
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
    } else if (epi == Epi::QkvRope) {
        if (ea.hd < 2 || ea.hd % 2 || N % ea.hd ||
            N != (int64_t)(ea.n_q_heads + 2 * ea.n_kv_heads) * ea.hd)
            return fail(Q4_ERR_INVALID_ARG, "%s: rotary rows need N == (H + 2 Hkv) * hd", what);
        *n_units = N / 2;
    } else {
        *n_units = N;
    }
    return Q4_OK;
}

q4_status launch_row_fn(RowFn fn, const uint8_t *packed, const uint16_t *scales,
                        const void *xin, int64_t N, int64_t K, Epi epi, const EpiArgs &ea, int R,
                        int grid, hipStream_t stream) {
    int64_t n_units = 0;
    Q4_CHECK(row_units(epi, N, ea, &n_units, "gemv rows"));
    const int UP = epi == Epi::SiluPair || epi == Epi::QkvRope ? R / 2 : R;
    const int64_t blocks = row_grid((n_units + UP - 1) / UP, grid);
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kRowThreads), (size_t)K * 2, stream,
                       packed, scales, xin, N, (int)K, n_units, ea);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace

// Every product with K <= 4096 runs the row kernels, and every wider one
// but the paired gate+up rows, whose software-pipelined loop in q4_gemv.hip
// stays faster there (57344 x 8192: 44.6 us against 45.5 for the best
// phased shape).
bool use_row_kernels(Epi e, int64_t K) { return K <= 4096 || e != Epi::SiluPair; }

q4_status launch_gemv_row(const uint8_t *packed, const uint16_t *scales, const void *xin,
                          Pro pro, int64_t N, int64_t K, Epi epi, const EpiArgs &ea,
                          hipStream_t stream) {
    RowCfg c = row_config(N, K);
    if (epi == Epi::QkvRope && c.R == 1)
        c.R = 2; // the rotation's row pairs share a group
    const RowFn fn = pick_any(epi, pro, c.NC, c.PH, c.R);
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED, "gemv rows: no kernel for K=%lld", (long long)K);
    return launch_row_fn(fn, packed, scales, xin, N, K, epi, ea, c.R, c.grid, stream);
}

namespace {

q4_status launch_row_batch_fn(RowBatchFn fn, const BatchCfg &c, const uint8_t *packed,
                              const uint16_t *scales, const void *xin, int64_t N, int64_t K,
                              int32_t B, Epi epi, const EpiArgs &ea, hipStream_t stream) {
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED, "gemv rows batch: no kernel for B=%d K=%lld", B,
                    (long long)K);
    int64_t n_units = 0;
    Q4_CHECK(row_units(epi, N, ea, &n_units, "gemv rows batch"));
    const int UP = epi == Epi::SiluPair ? c.R / 2 : c.R;
    const int64_t ngroups = (n_units + UP - 1) / UP;
    // one group per wave, at most sixteen waves per compute unit
    const int64_t blocks = std::max<int64_t>(
        1, std::min<int64_t>((ngroups + c.WV - 1) / c.WV, 16 / c.WV * (int64_t)device_cus()));
    const size_t lds = (size_t)B * 4 * (size_t)(K / 32) * 16;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * c.WV), lds, stream, packed, scales,
                       xin, N, (int)K, n_units, ea);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace

q4_status launch_gemv_row_batch(const uint8_t *packed, const uint16_t *scales,
                                const uint16_t *X16, int64_t N, int64_t K, int32_t B, Epi epi,
                                const EpiArgs &ea, hipStream_t stream) {
    const BatchCfg c = batch_config(K, B);
    const RowBatchFn fn = epi == Epi::SiluPair  ? pick_row_batch<Epi::SiluPair>(c, B)
                          : epi == Epi::Residual ? pick_row_batch<Epi::Residual>(c, B)
                          : epi == Epi::Store    ? pick_row_batch<Epi::Store>(c, B)
                                                 : nullptr;
    return launch_row_batch_fn(fn, c, packed, scales, X16, N, K, B, epi, ea, stream);
}

bool batch_norm_fits(int64_t K, int32_t B) {
    return gemv_batch_fits(B, K) && batch_config(K, B).XR;
}

q4_status launch_batch_norm_product(const uint8_t *packed, const uint16_t *scales,
                                    const float *H, int64_t N, int64_t K, int32_t B, Epi epi,
                                    const EpiArgs &ea, hipStream_t stream) {
    if (!batch_norm_fits(K, B))
        return fail(Q4_ERR_UNSUPPORTED, "batch norm product: B=%d K=%lld", B, (long long)K);
    const BatchCfg c = batch_config(K, B);
    const RowBatchFn fn = epi == Epi::SiluPair ? pick_row_batch_norm<Epi::SiluPair>(c, B)
                          : epi == Epi::Store  ? pick_row_batch_norm<Epi::Store>(c, B)
                                               : nullptr;
    return launch_row_batch_fn(fn, c, packed, scales, H, N, K, B, epi, ea, stream);
}

} // namespace q4

namespace {

q4_status check_tuned(const uint8_t *packed, const uint16_t *scales, const uint16_t *x_f16,
                      const float *y, int64_t N, int64_t K, int32_t workgroups,
                      const char *what) {
    Q4_CHECK(q4::check_matrix(packed, scales, N, K, what));
    if (!x_f16 || !y)
        return q4::fail(Q4_ERR_INVALID_ARG, "%s: null x or y", what);
    if (!q4::aligned(x_f16, 16) || !q4::aligned(y, 4))
        return q4::fail(Q4_ERR_INVALID_ARG, "%s: x must be 16-byte and y 4-byte aligned", what);
    if (workgroups < 0)
        return q4::fail(Q4_ERR_INVALID_ARG, "%s: workgroups must be >= 0", what);
    return Q4_OK;
}

} // namespace

extern "C" q4_status q4_gemv_rows_tuned(const uint8_t *packed, const uint16_t *scales,
                                        const uint16_t *x_f16, float *y, int64_t N, int64_t K,
                                        int32_t rows_per_wave, int32_t workgroups,
                                        hipStream_t stream) {
    Q4_CHECK(check_tuned(packed, scales, x_f16, y, N, K, workgroups, "q4_gemv_rows_tuned"));
    if (!(rows_per_wave == 2 || rows_per_wave == 4))
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_gemv_rows_tuned: rows_per_wave must be 2 or 4");
    if (K > 4096)
        return q4::fail(Q4_ERR_UNSUPPORTED, "q4_gemv_rows_tuned: K=%lld above 4096",
                        (long long)K);
    q4::EpiArgs ea{};
    ea.y = y;
    const int nc = (int)((K / 32 + 63) / 64);
    const q4::RowFn fn = q4::pick_row<q4::Epi::Store, q4::Pro::F16>(nc, rows_per_wave);
    return q4::launch_row_fn(fn, packed, scales, x_f16, N, K, q4::Epi::Store, ea, rows_per_wave,
                             workgroups, stream);
}

extern "C" q4_status q4_gemv_rowp_tuned(const uint8_t *packed, const uint16_t *scales,
                                        const uint16_t *x_f16, float *y, int64_t N, int64_t K,
                                        int32_t rows_per_wave, int32_t chunks_per_phase,
                                        int32_t workgroups, hipStream_t stream) {
    Q4_CHECK(check_tuned(packed, scales, x_f16, y, N, K, workgroups, "q4_gemv_rowp_tuned"));
    const q4::RowFn fn =
        q4::pick_rowp<q4::Epi::Store, q4::Pro::F16>(chunks_per_phase, rows_per_wave);
    if (!fn)
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_gemv_rowp_tuned: rows_per_wave 1 or 2 with chunks_per_phase 1, 2, 4 "
                        "or 7, or 4 with 2 or 4");
    q4::EpiArgs ea{};
    ea.y = y;
    return q4::launch_row_fn(fn, packed, scales, x_f16, N, K, q4::Epi::Store, ea, rows_per_wave,
                             workgroups, stream);
}
