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

#include "q4_gemv_core.h"

namespace q4 {
namespace {

// R rows per 16-lane row, KS waves per row's k range, U chunks of each row
// loaded per lane before use, NT non-temporal weight loads.
template <int R, int KS, int U, bool NT, Epi E, Pro P>
__global__ void __launch_bounds__(kThreads)
gemv_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
            const void *__restrict__ xin, int64_t N, int K, int64_t n_units, EpiArgs ea) {
    extern __shared__ uint4 xs[];
    __shared__ float red[kWaves][kSlots][R];
    __shared__ float wsum[kWaves];
    const uint32_t bias = vgpr_const(0x64006400u);
    const uint8_t *wp[R];
    const uint16_t *sp[R];
    uint4 w[U][R];
    uint16_t s[U][R];
    // Activation loads first, then the first weight loads, then the rest of
    // the prologue while the weights are in flight.  (Waiting for the
    // activation before issuing any weight load measured slower on every
    // decode shape.)
    // The paired gate+up rows after an RMSNorm stage behind their first
    // weight batch (measured faster, see stage_issue); every other variant
    // issues that batch unconditionally and stages as soon as the activation
    // has landed.
    constexpr bool kEarly = !(E == Epi::SiluPair && P == Pro::RmsNorm);
    XStage st;
    float hv[R];
    stage_issue<P, false, kEarly>(xin, K, st);
    if constexpr (E == Epi::Residual)
        load_residual<R, KS, E>(ea, N, blockIdx.x, hv);
    prefetch_block<R, KS, U, NT, E, !kEarly>(W, S, N, K, n_units, ea, blockIdx.x, w, s, wp, sp);
    stage_finish<P, false>(xin, xs, K, ea, wsum, st);
    __syncthreads();
    run_units<R, KS, U, NT, E>(W, S, N, K, n_units, ea, blockIdx.x, gridDim.x, xs, red, w, s,
                               wp, sp, bias, hv);
}

// The same product with the software-pipelined loop: two register buffers
// of U chunks x R rows, the next batch always in flight (q4_gemv_core.h).
// Requires K % (512 * KS * U) == 0 and grid <= row blocks.
template <int R, int KS, int U, bool NT, Epi E, Pro P>
__global__ void __launch_bounds__(kThreads)
gemv_pipe_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ S,
                 const void *__restrict__ xin, int64_t N, int K, int64_t n_units, EpiArgs ea) {
    extern __shared__ uint4 xs[];
    __shared__ float red[kWaves][kSlots][R];
    __shared__ float wsum[kWaves];
    const uint32_t bias = vgpr_const(0x64006400u);
    uint4 wA[U][R], wB[U][R];
    uint32_t sA[U][R], sB[U][R];
    XStage st;
    stage_issue<P, false>(xin, K, st);
    prefetch_pipe<R, KS, U, NT, E>(W, S, N, K, n_units, ea, blockIdx.x, gridDim.x, wA, sA, wB,
                                   sB);
    stage_finish<P, false>(xin, xs, K, ea, wsum, st);
    __syncthreads();
    run_units_pipe<R, KS, U, NT, E>(W, S, N, K, n_units, ea, blockIdx.x, gridDim.x, xs, red, wA,
                                    sA, wB, sB, bias);
}

// ---------------------------------------------------------------- launch
using KernelFn = void (*)(const uint8_t *, const uint16_t *, const void *, int64_t, int,
                          int64_t, EpiArgs);

// Launch shape of one product kernel: U chunks of each row in flight per
// lane (2, 4 or 8); pipe selects the software-pipelined loop (two buffers of
// two chunks, non-temporal loads only) instead of the single-buffer loop.
struct Cfg {
    int R, KS, U;
    bool NT;
    bool pipe;
};

template <Epi E, Pro P, int R, int KS>
KernelFn pick_ut(const Cfg &c) {
    if (c.pipe)
        return c.U == 2 && c.NT ? gemv_pipe_kernel<R, KS, 2, true, E, P> : nullptr;
    if (c.U == 2)
        return c.NT ? gemv_kernel<R, KS, 2, true, E, P> : gemv_kernel<R, KS, 2, false, E, P>;
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
    case Epi::QkvRope: return nullptr; // row kernels only
    }
    return nullptr;
}

// Resident workgroups per launch of kernel `fn` with `lds` bytes of LDS on
// the current device, cached in a fixed table (no heap allocation, so the
// launch path allocates nothing); a full table just recomputes.
int resident_blocks(KernelFn fn, size_t lds) {
    struct Entry {
        KernelFn fn;
        size_t lds;
        int dev;
        int total;
    };
    constexpr int kEntries = 512;
    static std::mutex mu;
    static Entry cache[kEntries];
    static int used = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lk(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].fn == fn && cache[i].lds == lds && cache[i].dev == dev)
            return cache[i].total;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kThreads, lds) != hipSuccess ||
        nb < 1)
        nb = 1;
    const int total = nb * device_cus();
    if (used < kEntries)
        cache[used++] = Entry{fn, lds, dev, total};
    return total;
}

// Launch shape of this kernel by product shape.  The library runs it only
// for paired rows (SiluPair) with K > 4096 and their 2..4-column products;
// every other product runs the row-per-wave kernels of q4_gemv_row.hip,
// which were faster there.  The shapes below, from back-to-back launch
// timings of every shape on the decode matrices with their real prologues
// and epilogues (non-temporal loads won or tied everywhere), remain what
// the measurement entry q4_gemv_tuned compares against:
//   * K = 4096: one row per 16-lane row with a 2-way k split (see below);
//     the paired gate+up rows also prefer a 2-way split (28672 x 4096:
//     14.5-14.8 vs 15.0-15.5 us);
//   * K = 8192 with 8192..12288 rows prefers one row per 16-lane row
//     (10240 x 8192: 12.2 vs 14.5 us; 8192 x 8192 with 8 chunks in flight:
//     11.0 vs 12.6 us);
//   * K = 14336: one row, 4-way split (4096 x 14336: 10.0 vs 10.25 us);
//   * K = 28672 prefers a 2-way split (27.4 vs 28.2 us);
//   * otherwise two rows per 16-lane row with a 4-way k split (best or
//     within 3% on the largest products, 57344 x 8192).
// The epilogue variant (paired rows) needs two rows per slot.
Cfg choose_config(Epi e, Pro p, int64_t N, int64_t K) {
    const int64_t C = K / 32;
    Cfg c{2, 4, 4, true, false};
    // The paired gate+up rows at K >= 8192 (57344 x 8192) stream faster with
    // the pipelined loop and a 2-way split (44.1-44.5 vs 46.6-47.5 us); the
    // other decode shapes gain nothing from it (their time goes to the
    // launch's start and tail, not to the steady stream).
    if (e == Epi::SiluPair && K >= 8192 && C % 64 == 0)
        return Cfg{2, 2, 2, true, true};
    if (K < 8192) {
        if (e == Epi::SiluPair) {
            c.KS = 2;
        } else {
            // one row per 16-lane row, 2-way split: with the activation
            // staged as soon as it lands, 4096 x 4096 takes 4.63 us against
            // 4.9 with a 4-way split, 6144 x 4096 5.37 against 6.7
            c.R = 1;
            c.KS = 2;
        }
    } else if (e != Epi::SiluPair && K < 12288 && N <= 12288) {
        c.R = 1;
        if (N > 8192) {
            c.KS = 2;
        } else {
            c.KS = 4;
            c.U = 8;
        }
    } else if (K >= 16384) {
        c.KS = 2;
    } else if (e != Epi::SiluPair && K >= 12288) {
        c.R = 1;
    }
    while (c.KS > 1 && C < 16 * c.KS)
        c.KS /= 2;
    // Narrow rows without a k split exist only with two rows per slot for the
    // decode epilogues.
    if (c.KS == 1 && c.R == 1 && e != Epi::Store)
        c.R = 2;
    // After a binary16 activation the first batch is issued unconditionally,
    // so no more chunks in flight than a lane has per row (K = 4096 with a
    // 4-way split leaves two per lane); the RMSNorm prologue skips the extra
    // loads and keeps the measured defaults (QKV 6.9 us with eight vs 7.1-7.5
    // with two).
    const int64_t nl = (C + 16 * c.KS - 1) / (16 * c.KS);
    while (c.U > 2 && c.U / 2 >= nl)
        c.U /= 2;
    return c;
}

} // namespace

void gemv_shape(Epi e, int64_t N, int64_t K, int *R, int *KS) {
    const Cfg c = choose_config(e, Pro::F16, N, K);
    *R = c.R;
    *KS = c.KS;
}

q4_status launch_gemv_cfg(const uint8_t *packed, const uint16_t *scales, const void *xin,
                          Pro pro, int64_t N, int64_t K, Epi epi, const EpiArgs &ea, int R,
                          int KS, int U, bool NT, bool pipe, hipStream_t stream) {
    Cfg cfg{R, KS, U, NT, pipe};
    KernelFn fn = pick_kernel(epi, pro, cfg);
    if (!fn)
        return fail(Q4_ERR_UNSUPPORTED,
                    "gemv: no kernel for rows_per_slot=%d k_split=%d chunks=%d", R, KS, U);
    if (pipe && (K / 32) % (32 * KS) != 0)
        return fail(Q4_ERR_UNSUPPORTED,
                    "gemv: the pipelined loop needs K %% (1024 * k_split) == 0 (K=%lld)",
                    (long long)K);
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
    if (use_row_kernels(epi, K))
        return launch_gemv_row(packed, scales, xin, pro, N, K, epi, ea, stream);
    const Cfg c = choose_config(epi, pro, epi == Epi::SiluPair ? 2 * ea.pair_off : N, K);
    return launch_gemv_cfg(packed, scales, xin, pro, N, K, epi, ea, c.R, c.KS, c.U, c.NT, c.pipe,
                           stream);
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
        !(chunks_in_flight == 2 || chunks_in_flight == 4 || chunks_in_flight == 8))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_gemv_tuned: rows_per_slot and k_split must be 1, 2 or 4, "
                        "chunks_in_flight 2, 4 or 8");
    q4::EpiArgs ea{};
    ea.y = y;
    // chunks_in_flight == 2 selects the software-pipelined loop
    return q4::launch_gemv_cfg(packed, scales, x_f16, q4::Pro::F16, N, K, q4::Epi::Store, ea,
                               rows_per_slot, k_split, chunks_in_flight, nontemporal != 0,
                               chunks_in_flight == 2, stream);
}
