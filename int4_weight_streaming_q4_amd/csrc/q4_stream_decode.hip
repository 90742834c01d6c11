// Streaming persistent decode step: one launch runs all layers of a token,
// with the weight stream decoupled from the layer's data dependencies.
//
// The per-token layer loop without per-kernel scheduling (PipeLLM: Faster
// Local LLM Inference Than llama.cpp via System-Level Optimizations,
// "Layer 1: CUDA Graph Compilation"), with the weights fed ahead of the
// computation that needs them (the same page, "Layer 2: Asynchronous Weight
// Prefetching"; PIPO: Pipelined Offloading for Efficient Inference on
// Consumer Devices, "Method", "Pipeline design") -- here from HBM into the
// on-chip LDS of every CU instead of from host memory into HBM.
//
// One workgroup per CU, 16 waves:
//   * 4 producer waves walk this workgroup's share of every product of every
//     layer in schedule order and copy the packed codes and scales straight
//     from HBM into an LDS ring with direct-to-LDS loads (no registers).  A
//     ring slot holds one 64-chunk segment of one row (1 KB of codes, 128 B
//     of scales).  Producers wait only for ring space, never for
//     activations or grid barriers, so HBM keeps streaming while the
//     consumers wait for the previous product to finish everywhere.
//   * 12 consumer waves stage each product's activation into LDS (binary16,
//     permuted to the unpack order; RMSNorm of the fp32 residual for QKV and
//     gate+up), then take units (two rows, or one gate/up row pair) round
//     robin, multiply the ring's chunks by the staged activation with the
//     same dequant-free arithmetic as the product kernel, reduce each row
//     over the wave and run the product's epilogue.  Between products the
//     consumers of all workgroups meet at a grid barrier (per-workgroup
//     arrival words polled by workgroup 0, one release word).
//
// Synchronisation inside a workgroup uses LDS counters: producer p publishes
// how many of its slots have landed (after waiting for its own loads), each
// consumer wave how many of its units it has finished (which frees their
// slots).  The producer touches these counters with inline-asm LDS accesses
// so the compiler does not drain the whole load queue before each one (it
// cannot tell that they do not alias the ring).  Every wait is bounded; past
// the bound it raises the error flag and all waves leave their loops.
#include <algorithm>
#include <map>
#include <mutex>

#include "q4_gemv_core.h"
#include "q4_persistent.h"

namespace q4 {
namespace {

constexpr int kSWaves = 16;
constexpr int kSThreads = 64 * kSWaves;
constexpr int kProd = 4;                  // producer waves 0..3
constexpr int kCons = kSWaves - kProd;    // consumer waves 4..15
constexpr int kConsThreads = 64 * kCons;
constexpr int kSeg = 64;                  // chunks per ring slot
constexpr int kSlotBytes = kSeg * 16 + kSeg * 2;
constexpr int kCtlBytes = 2048;
constexpr uint32_t kSSpin = 1u << 22;    // LDS polls (each with a short sleep)
constexpr uint32_t kGSpin = 1u << 20;    // global-memory polls

// LDS control words (uint32 offsets).
constexpr int kLanded = 0;     // [kProd] slots landed per producer
constexpr int kCBar = 32;      // consumer barrier arrivals
constexpr int kGo = 33;        // last grid epoch released to the consumers
constexpr int kAbort = 34;     // set when this workgroup gave up waiting
constexpr int kPartial = 64;   // [kCons] RMSNorm partial sums
constexpr int kGeo = 128;      // the Geo struct below
constexpr int kConsumed = 256; // [nslots] ring slot generations consumed

// s_waitcnt immediate (gfx9 encoding) for "at most N vector-memory
// operations outstanding", leaving the other counters unconstrained.
constexpr int waitcnt_vm(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)p;
}

// Producer-side LDS counter access, invisible to the compiler's wait
// insertion (see the header comment).
// Counters are wave-uniform: reads are broadcast from lane 0 so the
// control flow that depends on them stays scalar.
__device__ __forceinline__ uint32_t p_lds_read(const uint32_t *p) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(v)
                 : "v"(lds_addr(p))
                 : "memory");
    return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ void p_lds_write(uint32_t *p, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(lds_addr(p)), "v"(v)
                 : "memory");
}

__device__ __forceinline__ uint32_t c_load(const uint32_t *p) {
    return __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
}

__device__ __forceinline__ bool gerr(const uint32_t *bar) {
    return __builtin_amdgcn_readfirstlane(
               __hip_atomic_load(bar + kBarErr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0u;
}

__device__ __forceinline__ void raise_err(uint32_t *bar) {
    __hip_atomic_store(bar + kBarErr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Shapes of the four products and this workgroup's share of them.
struct Geo {
    int64_t N[4];
    int K[4], C[4], S[4];     // K, chunks per row, ring slots per row
    int64_t u0[4];            // first unit of this workgroup
    int nu[4];                // units of this workgroup
    int slot_pre[5];          // slots before product k within a layer
    int unit_pre[5];          // units before product k within a layer
};

__device__ __forceinline__ void make_geo(const PersistArgs &a, Geo &g) {
    // written by one thread into LDS; everyone reads it after a barrier
    const int64_t nqkv = (int64_t)(a.H + 2 * a.Hkv) * a.hd;
    g.N[0] = nqkv;
    g.N[1] = a.d;
    g.N[2] = 2 * (int64_t)a.dff;
    g.N[3] = a.d;
    g.K[0] = a.d;
    g.K[1] = a.H * a.hd;
    g.K[2] = a.d;
    g.K[3] = a.dff;
    const int64_t G = gridDim.x, b = blockIdx.x;
    g.slot_pre[0] = 0;
    g.unit_pre[0] = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        g.C[k] = g.K[k] >> 5;
        g.S[k] = (g.C[k] + kSeg - 1) / kSeg;
        const int64_t units = k == 2 ? (int64_t)a.dff : (g.N[k] + 1) / 2;
        g.u0[k] = units * b / G;
        g.nu[k] = (int)(units * (b + 1) / G - g.u0[k]);
        g.slot_pre[k + 1] = g.slot_pre[k] + g.nu[k] * 2 * g.S[k];
        g.unit_pre[k + 1] = g.unit_pre[k] + g.nu[k];
    }
}

// Matrix row of row r (0 or 1) of unit u in product k; N[k] or more when the
// unit has no such row.
__device__ __forceinline__ int64_t unit_row(const Geo &g, const PersistArgs &a, int k, int64_t u,
                                            int r) {
    if (k == 2)
        return r == 0 ? u : (int64_t)a.dff + u;
    return 2 * u + r;
}

// ------------------------------------------------------------ producer
// Slot order within a product: units in groups of kCons (one per consumer
// wave), and inside a group segment-major, then row, then unit, so that the
// consumer waves walk their units in step and the slots they need at any
// moment are adjacent in the stream.
template <int kDepth> // slots in flight per producer wave
__device__ __forceinline__ void producer(const PersistArgs &a,
                                         const DevLayer *__restrict__ layers, const Geo &gs_lds,
                                         uint32_t *ctl, char *ring, uint32_t nslots, int pw,
                                         int p0, int p1) {
    // A register copy of the shapes, taken before the first direct-to-LDS
    // load: ordinary LDS reads after that point would make the compiler wait
    // for every outstanding load first.
    const Geo g = gs_lds;
    const int lane = threadIdx.x & 63;
    uint32_t *landed = ctl + kLanded + pw;
    const uint32_t *consumed = ctl + kConsumed;
    uint32_t issued = 0;
    uint32_t gs = 0, pos = 0, gen = 0; // slot, its ring position and pass
    bool abort = false;
    for (int l = p0 / 4; l <= (p1 - 1) / 4 && !abort; ++l) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (abort)
                break;
            if (l * 4 + k < p0 || l * 4 + k >= p1)
                continue;
            // scalar loads (read-only table): they do not share the vector
            // memory counter with the ring loads
            const uint8_t *W = layers[l].packed[k];
            const uint16_t *Sc = layers[l].scales[k];
            const int C = g.C[k], S = g.S[k], nu = g.nu[k];
            for (int j0 = 0; j0 < nu && !abort; j0 += kCons) {
                const int nj = min(kCons, nu - j0);
                for (int sg = 0; sg < S && !abort; ++sg) {
                    for (int r = 0; r < 2 && !abort; ++r) {
                        // slots gs .. gs + nj - 1; this wave's are those
                        // congruent to pw modulo kProd
                        const int w0 = (int)((uint32_t)(pw - (int)gs) & (kProd - 1));
                        uint32_t my_pos = pos + (uint32_t)w0, my_gen = gen;
                        if (my_pos >= nslots) {
                            my_pos -= nslots;
                            ++my_gen;
                        }
                        for (int w = w0; w < nj; w += kProd) {
                            // The ring position's previous slot must have been
                            // read (its consumer stored generation my_gen).
                            if (my_gen > 0 && p_lds_read(consumed + my_pos) < my_gen) {
                                // Landed counts must be current before waiting
                                // on consumers that may wait on them.
                                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                                if (lane == 0)
                                    p_lds_write(landed, issued);
                                uint32_t n = 0;
                                while (p_lds_read(consumed + my_pos) < my_gen) {
                                    __builtin_amdgcn_s_sleep(1);
                                    if ((++n & 255u) == 0u &&
                                        (gerr(a.bar) || p_lds_read(ctl + kAbort) != 0u)) {
                                        abort = true;
                                        break;
                                    }
                                    if (n > kSSpin) {
                                        raise_err(a.bar);
                                        abort = true;
                                        break;
                                    }
                                }
                                if (abort)
                                    break;
                            }
                            const int64_t row = unit_row(g, a, k, g.u0[k] + j0 + w, r);
                            char *slot = ring + (size_t)my_pos * kSlotBytes;
                            if (row < g.N[k]) {
                                const int c = sg * kSeg + lane;
                                if (c < C)
                                    __builtin_amdgcn_global_load_lds(
                                        (gptr_t)(W + ((size_t)row * C + c) * 16), (lptr_t)slot,
                                        16, 0, 2);
                                const int c2 = sg * kSeg + 2 * lane;
                                if (lane < kSeg / 2 && c2 < C)
                                    __builtin_amdgcn_global_load_lds(
                                        (gptr_t)(Sc + (size_t)row * C + c2),
                                        (lptr_t)(slot + kSeg * 16), 4, 0, 2);
                            }
                            ++issued;
                            // At most 2 * kDepth loads (kDepth slots) in
                            // flight; every older slot of this wave landed.
                            __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kDepth));
                            if (issued > (uint32_t)kDepth && lane == 0)
                                p_lds_write(landed, issued - kDepth);
                            my_pos += kProd;
                            if (my_pos >= nslots) {
                                my_pos -= nslots;
                                ++my_gen;
                            }
                        }
                        // advance the shared slot counter past the nj slots
                        gs += (uint32_t)nj;
                        pos += (uint32_t)nj;
                        while (pos >= nslots) {
                            pos -= nslots;
                            ++gen;
                        }
                    }
                }
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if (lane == 0)
        p_lds_write(landed, abort ? 0xFFFFFFFFu : issued);
}

// ------------------------------------------------------------ consumers
struct CState {
    uint32_t *ctl;
    uint32_t front = 0;  // slots below this one have landed
    uint32_t bars = 0;   // consumer barriers passed
    uint32_t nsync = 0;  // grid barriers passed
    uint32_t parity = 0;
    bool abort = false;
};

// Barrier of the consumer waves of this workgroup (LDS counter).
__device__ __forceinline__ void cons_barrier(CState &cs, uint32_t *bar) {
    const int lane = threadIdx.x & 63;
    ++cs.bars;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0)
        __hip_atomic_fetch_add(cs.ctl + kCBar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint32_t target = cs.bars * kCons;
    uint32_t n = 0;
    while (c_load(cs.ctl + kCBar) < target) {
        __builtin_amdgcn_s_sleep(1);
        if ((++n & 255u) == 0u && gerr(bar)) {
            cs.abort = true;
            break;
        }
        if (n > kSSpin) {
            raise_err(bar);
            cs.abort = true;
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Polls a barrier word in global memory.  Every poll of every waiting
// workgroup goes to the same memory channel, so the polls are spaced out
// (a tight loop from hundreds of workgroups slows all memory traffic).
__device__ __forceinline__ bool spin_global(const uint32_t *p, uint32_t want, uint32_t *bar) {
    uint32_t n = 0;
    while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want) {
        __builtin_amdgcn_s_sleep(4);
        if ((++n & 63u) == 0u && gerr(bar))
            return false;
        if (n > kGSpin) {
            raise_err(bar);
            return false;
        }
    }
    return true;
}

// Grid barrier between products, consumer waves only.  Activation stores
// and loads are agent-scope atomics (coherent without cache maintenance), so
// a wave only waits for its own stores to complete; then the consumer waves
// meet in the workgroup and the first one does the grid-level
// arrival/release.
__device__ __forceinline__ void grid_sync(CState &cs, const PersistArgs &a, int cw) {
    __builtin_amdgcn_s_waitcnt(0);
    cons_barrier(cs, a.bar);
    const uint32_t epoch = (cs.parity << 31) | ++cs.nsync;
    if (cw == 0 && !cs.abort) {
        uint32_t *flags = a.bar + kBarFlags;
        uint32_t *rel = flags + kMaxPersistentGrid;
        const int lane = threadIdx.x & 63;
        if (lane == 0)
            __hip_atomic_store(flags + blockIdx.x, epoch, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        bool ok = true;
        if (blockIdx.x == 0) {
            // Every lane loads all of its arrival words in one go (the loads
            // are independent, so they overlap), then the wave votes.
            uint32_t n = 0;
            for (;;) {
                bool mine = true;
#pragma unroll 4
                for (uint32_t i = lane; i < gridDim.x; i += 64)
                    mine = (__hip_atomic_load(flags + i, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) == epoch) && mine;
                if (__all(mine))
                    break;
                __builtin_amdgcn_s_sleep(2);
                if ((++n & 63u) == 0u && gerr(a.bar)) {
                    ok = false;
                    break;
                }
                if (n > kGSpin) {
                    raise_err(a.bar);
                    ok = false;
                    break;
                }
            }
            if (ok && lane == 0)
                __hip_atomic_store(rel, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (lane == 0) {
            ok = spin_global(rel, epoch, a.bar);
        }
        ok = __shfl(ok, 0);
        if (!ok) {
            cs.abort = true;
            if (lane == 0)
                __hip_atomic_store(cs.ctl + kAbort, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (lane == 0)
            __hip_atomic_store(cs.ctl + kGo, epoch, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    } else if (!cs.abort) {
        uint32_t n = 0;
        while (c_load(cs.ctl + kGo) != epoch) {
            __builtin_amdgcn_s_sleep(1);
            if ((++n & 255u) == 0u && gerr(a.bar)) {
                cs.abort = true;
                break;
            }
            if (n > kSSpin) {
                raise_err(a.bar);
                cs.abort = true;
                break;
            }
        }
    }
    if (c_load(cs.ctl + kAbort) != 0u)
        cs.abort = true;
}

// binary16 activation -> LDS (consumer threads only).
template <bool COH>
__device__ __forceinline__ void cons_stage_f16(const uint16_t *x16, uint4 *xs, int K, int tc) {
    const int C = K >> 5;
    for (int b = tc; b < (K >> 3); b += kConsThreads)
        xs[(b & 3) * C + (b >> 2)] = permute8(act_load16<COH>(x16 + 8 * (size_t)b));
}

// RMSNorm of the fp32 residual -> LDS (consumer threads only); every
// workgroup sums in the same order, so all stage identical bits.
template <bool COH>
__device__ __forceinline__ void cons_stage_rms(CState &cs, const PersistArgs &a, uint4 *xs,
                                               int K, int tc, int cw, uint16_t *norm_out) {
    constexpr int kKeep = 2;
    const int C = K >> 5;
    const int nb8 = K >> 3;
    float keep[kKeep][8];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < kKeep; ++j) {
        const int b = tc + j * kConsThreads;
        if (b < nb8) {
            load_f32x8<COH>(a.h + 8 * (size_t)b, keep[j]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ss = fmaf(keep[j][i], keep[j][i], ss);
        }
    }
    for (int b = tc + kKeep * kConsThreads; b < nb8; b += kConsThreads) {
        float f[8];
        load_f32x8<COH>(a.h + 8 * (size_t)b, f);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ss = fmaf(f[i], f[i], ss);
    }
    ss = wave_sum(ss);
    float *part = reinterpret_cast<float *>(cs.ctl + kPartial);
    if ((threadIdx.x & 63) == 0)
        part[cw] = ss;
    cons_barrier(cs, a.bar);
    float tot = part[0];
#pragma unroll
    for (int w = 1; w < kCons; ++w)
        tot += part[w];
    const float r = 1.0f / sqrtf(tot / (float)K + a.eps);
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
        const int b = tc + j * kConsThreads;
        if (b < nb8)
            emit(b, keep[j]);
    }
    for (int b = tc + kKeep * kConsThreads; b < nb8; b += kConsThreads) {
        float f[8];
        load_f32x8<COH>(a.h + 8 * (size_t)b, f);
        emit(b, f);
    }
}

// Waits until global slot `gs` has landed in the ring.  `front` caches a
// bound below which every slot is known to have landed (the smallest of the
// producers' counters, each turned into a global slot index), so most calls
// touch no LDS at all: polling waves share their SIMD's instruction issue
// with the producer.
__device__ __forceinline__ bool wait_slot(CState &cs, const PersistArgs &a, uint32_t gs) {
    if (gs < cs.front)
        return true;
    uint32_t n = 0;
    for (;;) {
        uint32_t f = 0xFFFFFFFFu;
        bool gave_up = false;
#pragma unroll
        for (int p = 0; p < kProd; ++p) {
            const uint32_t v = c_load(cs.ctl + kLanded + p);
            gave_up = gave_up || v == 0xFFFFFFFFu;
            f = min(f, v * kProd + p);
        }
        if (gave_up)
            return false; // a producer gave up
        cs.front = f;
        if (gs < f)
            return true;
        __builtin_amdgcn_s_sleep(2);
        if ((++n & 255u) == 0u && gerr(a.bar))
            return false;
        if (n > kSSpin) {
            raise_err(a.bar);
            return false;
        }
    }
}

// Marks global slot `gs` read: its ring position may take the next pass.
__device__ __forceinline__ void free_slot(uint32_t *ctl, uint32_t gs, uint32_t nslots) {
    const uint32_t pass = gs / nslots;
    __hip_atomic_store(ctl + kConsumed + (gs - pass * nslots), pass + 1, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <bool COH>
__device__ __forceinline__ void consumer(const PersistArgs &a, const Geo &g, uint32_t *ctl,
                                         uint4 *xs, const char *ring, uint32_t nslots, int cw,
                                         int p0, int p1) {
    const int lane = threadIdx.x & 63;
    const int tc = threadIdx.x - kProd * 64;
    const uint32_t bias = vgpr_const(0x64006400u);
    CState cs;
    cs.ctl = ctl;
    cs.parity = __hip_atomic_load(a.bar + kBarParity, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                1u;
    const int64_t v_off = (int64_t)(a.H + a.Hkv) * a.hd;
    const int group = a.H / a.Hkv;
    const uint32_t layer_slots = (uint32_t)g.slot_pre[4];
    // slot index of the first slot of phase p0 (slots count from 0 per launch)
    const uint32_t base = (uint32_t)(p0 / 4) * layer_slots + (uint32_t)g.slot_pre[p0 % 4];
    for (int l = p0 / 4; l <= (p1 - 1) / 4 && !cs.abort; ++l) {
        for (int k = 0; k < 4 && !cs.abort; ++k) {
            if (l * 4 + k < p0 || l * 4 + k >= p1)
                continue;
            const int K = g.K[k], C = g.C[k], S = g.S[k], nu = g.nu[k];
            if (k == 0)
                cons_stage_rms<COH>(cs, a, xs, K, tc, cw, nullptr);
            else if (k == 1)
                cons_stage_f16<COH>(a.oin, xs, K, tc);
            else if (k == 2)
                cons_stage_rms<COH>(cs, a, xs, K, tc, cw, a.norm_out);
            else
                cons_stage_f16<COH>(a.mlp, xs, K, tc);
            cons_barrier(cs, a.bar);
            const uint32_t pb = (uint32_t)l * layer_slots + (uint32_t)g.slot_pre[k] - base;
            // Unit j0 + cw of every group of kCons units (producer order).
            for (int j0 = 0; j0 + cw < nu && !cs.abort; j0 += kCons) {
                const int nj = min(kCons, nu - j0);
                const uint32_t gb = pb + (uint32_t)j0 * 2 * S;
                const int64_t u = g.u0[k] + j0 + cw;
                const int64_t row0 = unit_row(g, a, k, u, 0);
                const int64_t row1 = unit_row(g, a, k, u, 1);
                const bool v1 = row1 < g.N[k];
                float y0 = 0.0f, y1 = 0.0f;
                if (k == 1 || k == 3) {
                    if (lane == 0)
                        y0 = act_load_f32<COH>(a.h + row0);
                    if (lane == 1 && v1)
                        y1 = act_load_f32<COH>(a.h + row1);
                }
                float acc0 = 0.0f, acc1 = 0.0f;
                for (int sg = 0; sg < S; ++sg) {
                    const uint32_t s0 = gb + (uint32_t)(sg * 2 * nj + cw);
                    const uint32_t s1 = s0 + (uint32_t)nj;
                    if (!wait_slot(cs, a, s0) || !wait_slot(cs, a, s1)) {
                        cs.abort = true;
                        break;
                    }
                    const int c = sg * kSeg + lane;
                    if (c < C) {
                        uint4 xq[4];
#pragma unroll
                        for (int p = 0; p < 4; ++p)
                            xq[p] = xs[p * C + c];
                        const char *sl0 = ring + (size_t)(s0 % nslots) * kSlotBytes;
                        const uint4 w0 = reinterpret_cast<const uint4 *>(sl0)[lane];
                        const uint16_t sc0 =
                            reinterpret_cast<const uint16_t *>(sl0 + kSeg * 16)[lane];
                        acc0 = chunk_acc(w0, xq, f16_to_f32(sc0), acc0, bias);
                        if (v1) {
                            const char *sl1 = ring + (size_t)(s1 % nslots) * kSlotBytes;
                            const uint4 w1 = reinterpret_cast<const uint4 *>(sl1)[lane];
                            const uint16_t sc1 =
                                reinterpret_cast<const uint16_t *>(sl1 + kSeg * 16)[lane];
                            acc1 = chunk_acc(w1, xq, f16_to_f32(sc1), acc1, bias);
                        }
                    }
                    // Both slots' values are in registers (used above).
                    if (lane == 0) {
                        free_slot(ctl, s0, nslots);
                        free_slot(ctl, s1, nslots);
                    }
                }
                if (cs.abort)
                    break;
                const float t0 = wave_sum(acc0);
                const float t1 = wave_sum(acc1);
                if (k == 0) {
                    if (lane < 2 && (lane == 0 || v1)) {
                        const int64_t row = lane ? row1 : row0;
                        const float t = lane ? t1 : t0;
                        act_store_f32<COH>(a.qkv + row, t);
                        if (row >= v_off) {
                            const int64_t v = row - v_off;
                            const int64_t gq = v / a.hd, e = v % a.hd;
                            const uint16_t h16 = f32_to_f16(t);
                            for (int q = 0; q < group; ++q)
                                act_store_u16<COH>(a.oin + (gq * group + q) * a.hd + e, h16);
                        }
                    }
                } else if (k == 2) {
                    if (lane == 0) {
                        const float silu = t0 / (1.0f + expf(-t0));
                        act_store_u16<COH>(a.mlp + u, f32_to_f16(silu * t1));
                    }
                } else {
                    if (lane == 0)
                        act_store_f32<COH>(a.h + row0, y0 + t0);
                    if (lane == 1 && v1)
                        act_store_f32<COH>(a.h + row1, y1 + t1);
                }
            }
            const bool last = l * 4 + k + 1 == p1;
            if (!last && !cs.abort)
                grid_sync(cs, a, cw);
        }
    }
    if (cs.abort && lane == 0)
        __hip_atomic_store(ctl + kAbort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // the launch parity alternates only for launches that used grid barriers
    if (p1 - p0 > 1 && cw == 0 && blockIdx.x == 0 && lane == 0 && !cs.abort)
        __hip_atomic_store(a.bar + kBarParity, cs.parity ^ 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Phases [p0, p1) of the schedule (phase 4 l + k is product k of layer l).
// COH: several phases with grid barriers in between (coherent activation
// accesses); otherwise a single phase, published by the kernel boundary.
template <int kDepth, bool COH>
__global__ void __launch_bounds__(kSThreads)
decode_stream(PersistArgs a, const DevLayer *__restrict__ layers, int32_t xbytes,
              int32_t nslots, int32_t p0, int32_t p1) {
    extern __shared__ uint4 lds[];
    uint32_t *ctl = reinterpret_cast<uint32_t *>(lds);
    uint4 *xs = reinterpret_cast<uint4 *>(reinterpret_cast<char *>(lds) + kCtlBytes);
    char *ring = reinterpret_cast<char *>(lds) + kCtlBytes + xbytes;
    static_assert(kGeo * 4 + sizeof(Geo) <= kConsumed * 4, "control block");
    for (int i = threadIdx.x; i < kCtlBytes / 4; i += kSThreads)
        if (i < kGeo || i >= kConsumed)
            ctl[i] = 0u;
    Geo &g = *reinterpret_cast<Geo *>(ctl + kGeo);
    if (threadIdx.x == 0)
        make_geo(a, g);
    __syncthreads();
    // wave-uniform (scalar) role index: keeps the roles' control flow and
    // the weight-pointer loads scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (wave < kProd)
        producer<kDepth>(a, layers, g, ctl, ring, (uint32_t)nslots, wave, p0, p1);
    else
        consumer<COH>(a, g, ctl, xs, ring, (uint32_t)nslots, wave - kProd, p0, p1);
}

struct StreamCfg {
    int grid = 0;
    size_t lds = 0;
};

// In-flight depths: the deeper one when the ring has room for it.
constexpr int kDepthHi = 16, kDepthLo = 8;

StreamCfg stream_cfg() {
    static std::mutex mu;
    static std::map<int, StreamCfg> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(dev);
    if (it != cache.end())
        return it->second;
    StreamCfg c;
    // The largest LDS allocation one workgroup may opt into (160 KB per CU
    // on gfx950); fall back to the default per-block limit.
    int max_lds = 0, optin = 0;
    if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
        hipSuccess)
        max_lds = 0;
    if (hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev) !=
        hipSuccess)
        optin = 0;
    c.lds = (size_t)std::max(max_lds, optin);
    bool ok = c.lds > 0;
    for (const void *fn :
         {(const void *)decode_stream<kDepthHi, true>, (const void *)decode_stream<kDepthLo, true>,
          (const void *)decode_stream<kDepthHi, false>, (const void *)decode_stream<kDepthLo, false>})
        ok = ok && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)c.lds) == hipSuccess;
    int nb = 0;
    if (ok &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_stream<kDepthHi, true>, kSThreads,
                                                     c.lds) == hipSuccess &&
        nb >= 1)
        c.grid = device_cus();
    cache[dev] = c;
    return c;
}

size_t stream_xbytes(int32_t d, int32_t H, int32_t hd, int32_t dff) {
    return ((size_t)std::max({d, H * hd, dff}) * 2 + 15) & ~(size_t)15;
}

// Slots the ring needs beside those in flight: two per consumer wave.
constexpr int64_t kHeld = 2 * kCons;

} // namespace

q4_status stream_supported(int32_t d, int32_t H, int32_t hd, int32_t dff, int *nslots_out) {
    const int Ks[3] = {d, H * hd, dff};
    for (int K : Ks)
        if (K % 64 != 0)
            return fail(Q4_ERR_UNSUPPORTED, "streaming decode: K=%d is not a multiple of 64", K);
    const size_t xb = stream_xbytes(d, H, hd, dff);
    const StreamCfg c = stream_cfg();
    if (c.grid < 1 || c.grid > kMaxPersistentGrid)
        return fail(Q4_ERR_UNSUPPORTED, "streaming decode: no resident grid (LDS %zu)", c.lds);
    if (c.lds < kCtlBytes + xb)
        return fail(Q4_ERR_UNSUPPORTED, "streaming decode: activations exceed LDS");
    const int64_t nslots = std::min<int64_t>((int64_t)(c.lds - kCtlBytes - xb) / kSlotBytes,
                                             kCtlBytes / 4 - kConsumed);
    if (nslots < (int64_t)kProd * kDepthLo + kHeld)
        return fail(Q4_ERR_UNSUPPORTED, "streaming decode: ring of %lld slots too small",
                    (long long)nslots);
    if (nslots_out)
        *nslots_out = (int)nslots;
    return Q4_OK;
}

namespace {

q4_status launch_range(const PersistArgs &a, int32_t p0, int32_t p1, hipStream_t stream) {
    int nslots = 0;
    Q4_CHECK(stream_supported(a.d, a.H, a.hd, a.dff, &nslots));
    const size_t xb = stream_xbytes(a.d, a.H, a.hd, a.dff);
    const StreamCfg c = stream_cfg();
    const bool hi = nslots >= (int64_t)kProd * kDepthHi + kHeld;
    const bool coh = p1 - p0 > 1;
    auto fn = hi ? (coh ? decode_stream<kDepthHi, true> : decode_stream<kDepthHi, false>)
                 : (coh ? decode_stream<kDepthLo, true> : decode_stream<kDepthLo, false>);
    hipLaunchKernelGGL(fn, dim3((unsigned)c.grid), dim3(kSThreads), c.lds, stream, a, a.layers,
                       (int32_t)xb, (int32_t)nslots, p0, p1);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace

q4_status launch_stream(const PersistArgs &a, hipStream_t stream) {
    return launch_range(a, 0, 4 * a.n_layers, stream);
}

q4_status launch_stream_product(const PersistArgs &a, int32_t layer, int32_t which,
                                hipStream_t stream) {
    if (layer < 0 || layer >= a.n_layers || which < 0 || which > 3)
        return fail(Q4_ERR_INVALID_ARG, "streaming product: layer %d product %d", layer, which);
    return launch_range(a, 4 * layer + which, 4 * layer + which + 1, stream);
}

} // namespace q4
