// Persistent decode step: one kernel launch runs all layers of one token.
//
// The per-token layer loop (PipeLLM: Faster Local LLM Inference Than
// llama.cpp via System-Level Optimizations, "Layer 1: CUDA Graph
// Compilation" -- the decode loop replayed without per-kernel scheduling)
// becomes, on MI355X, a single resident grid that walks the four products of
// every layer (QKV, O, gate+up, down) with a grid-wide barrier between
// products.  Each product only needs the previous product's small output,
// while its weights are independent of it: every workgroup therefore issues
// the first weight loads of its next product BEFORE it waits at the barrier,
// so HBM keeps streaming across product boundaries instead of idling through
// a kernel drain, a launch and a prologue.
//
// The grid is sized to what fits on the device at once (occupancy x CUs);
// the barrier spins with a bounded count and, past it, raises an error flag
// and lets every wave run to the end (no wave can wait forever).  Workgroups
// exchange the activation vectors (residual, QKV output, attention output,
// gated MLP input) through agent-scope atomic stores and cached loads after
// a per-workgroup cache invalidation; the barrier publishes them with
// per-workgroup arrival words instead of one contended counter.
#include <algorithm>
#include <map>
#include <mutex>

#include "q4_gemv_core.h"
#include "q4_persistent.h"

namespace q4 {
namespace {

constexpr int PR = 2, PKS = 4, PU = 4;
constexpr bool PNT = true;
// ~1 s of polling before a barrier gives up.
constexpr uint32_t kSpinLimit = 1u << 20;

// Waits until *p == want.  Gives up (setting the error flag) after
// kSpinLimit polls, or at once when another wait already gave up.
__device__ __forceinline__ void spin_until(const uint32_t *p, uint32_t want, uint32_t *err) {
    uint32_t n = 0;
    while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want) {
        if ((++n & 63u) == 0u &&
            __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
            return;
        if (n > kSpinLimit) {
            __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
    }
}

// Grid barrier without contended atomics: every workgroup stores `epoch` to
// its own arrival word; workgroup 0's threads poll all arrival words, then
// store `epoch` to the release word that every workgroup polls.  Activation
// stores are agent-scope atomic stores, so each thread only has to wait for
// its own stores to complete before the arrival is published; on exit the
// workgroup invalidates its caches once so its ordinary loads see them.
__device__ __forceinline__ void flag_sync(uint32_t *bar, uint32_t epoch) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    uint32_t *err = bar + kBarErr;
    uint32_t *flags = bar + kBarFlags;
    uint32_t *rel = flags + kMaxPersistentGrid;
    if (threadIdx.x == 0)
        __hip_atomic_store(flags + blockIdx.x, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (blockIdx.x == 0) {
        for (uint32_t i = threadIdx.x; i < gridDim.x; i += blockDim.x)
            spin_until(flags + i, epoch, err);
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_store(rel, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (threadIdx.x == 0) {
        spin_until(rel, epoch, err);
    }
    // One wave invalidates this CU's and XCD's caches (agent-scope acquire)
    // before anyone reads the vectors other workgroups wrote.
    if (threadIdx.x < 64)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
}

struct Phase {
    const uint8_t *W;
    const uint16_t *S;
    int64_t N;
    int K;
    int64_t n_units;
};

__global__ void __launch_bounds__(kThreads) decode_persistent(PersistArgs a) {
    extern __shared__ uint4 xs[];
    __shared__ float red[kWaves][kSlots][PR];
    __shared__ float wsum[kWaves];
    const uint32_t bias = vgpr_const(0x64006400u);

    const int64_t nqkv = (int64_t)(a.H + 2 * a.Hkv) * a.hd;
    EpiArgs e_qkv{}, e_o{}, e_gu{}, e_down{};
    e_qkv.y = a.qkv;
    e_qkv.out16 = a.oin;
    e_qkv.v_off = (int64_t)(a.H + a.Hkv) * a.hd;
    e_qkv.hd = a.hd;
    e_qkv.group = a.H / a.Hkv;
    e_qkv.eps = a.eps;
    e_o.y = a.h;
    e_gu.out16 = a.mlp;
    e_gu.pair_off = a.dff;
    e_gu.eps = a.eps;
    e_gu.norm_out = a.norm_out;
    e_down.y = a.h;

    const uint8_t *wp[PR];
    const uint16_t *sp[PR];
    uint4 w[PU][PR];
    uint16_t s[PU][PR];
    float hvd[PR] = {}; // residual values: read late on this path
    const int64_t b0 = blockIdx.x, G = gridDim.x;
    // Barrier epochs of this launch: the parity bit alternates between
    // launches (workgroup 0 flips it at its end, after every workgroup has
    // read it), so no epoch of one launch equals one of the launch before.
    const uint32_t parity =
        __hip_atomic_load(a.bar + kBarParity, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1u;
    uint32_t nsync = 0;
    auto barrier = [&]() { flag_sync(a.bar, (parity << 31) | ++nsync); };

    auto ph_qkv = [&](const DevLayer &L) {
        return Phase{L.packed[0], L.scales[0], nqkv, a.d, (nqkv + PR - 1) / PR};
    };
    auto ph_o = [&](const DevLayer &L) {
        return Phase{L.packed[1], L.scales[1], a.d, a.H * a.hd, ((int64_t)a.d + PR - 1) / PR};
    };
    auto ph_gu = [&](const DevLayer &L) {
        return Phase{L.packed[2], L.scales[2], 2 * (int64_t)a.dff, a.d, (int64_t)a.dff};
    };
    auto ph_down = [&](const DevLayer &L) {
        return Phase{L.packed[3], L.scales[3], a.d, a.dff, ((int64_t)a.d + PR - 1) / PR};
    };

    {
        const Phase p = ph_qkv(a.layers[0]);
        prefetch_block<PR, PKS, PU, PNT, Epi::QkvGather>(p.W, p.S, p.N, p.K, p.n_units, e_qkv,
                                                         b0, w, s, wp, sp);
    }
    for (int l = 0; l < a.n_layers; ++l) {
        const DevLayer L = a.layers[l];
        {   // QKV; the first RMSNorm in the prologue
            const Phase p = ph_qkv(L);
            stage_activation<Pro::RmsNorm, true>(a.h, xs, p.K, e_qkv, wsum);
            __syncthreads();
            run_units<PR, PKS, PU, PNT, Epi::QkvGather, true>(p.W, p.S, p.N, p.K, p.n_units, e_qkv, b0,
                                                         G, xs, red, w, s, wp, sp, bias, hvd);
            const Phase q = ph_o(L);
            prefetch_block<PR, PKS, PU, PNT, Epi::Residual>(q.W, q.S, q.N, q.K, q.n_units, e_o,
                                                            b0, w, s, wp, sp);
            barrier();
        }
        {   // O, residual add
            const Phase p = ph_o(L);
            stage_activation<Pro::F16, true>(a.oin, xs, p.K, e_o, wsum);
            __syncthreads();
            run_units<PR, PKS, PU, PNT, Epi::Residual, true>(p.W, p.S, p.N, p.K, p.n_units, e_o, b0, G,
                                                        xs, red, w, s, wp, sp, bias, hvd);
            const Phase q = ph_gu(L);
            prefetch_block<PR, PKS, PU, PNT, Epi::SiluPair>(q.W, q.S, q.N, q.K, q.n_units, e_gu,
                                                            b0, w, s, wp, sp);
            barrier();
        }
        {   // gate+up; the second RMSNorm in the prologue, SiLU gate after
            const Phase p = ph_gu(L);
            stage_activation<Pro::RmsNorm, true>(a.h, xs, p.K, e_gu, wsum);
            __syncthreads();
            run_units<PR, PKS, PU, PNT, Epi::SiluPair, true>(p.W, p.S, p.N, p.K, p.n_units, e_gu, b0, G,
                                                        xs, red, w, s, wp, sp, bias, hvd);
            const Phase q = ph_down(L);
            prefetch_block<PR, PKS, PU, PNT, Epi::Residual>(q.W, q.S, q.N, q.K, q.n_units,
                                                            e_down, b0, w, s, wp, sp);
            barrier();
        }
        {   // down, residual add
            const Phase p = ph_down(L);
            stage_activation<Pro::F16, true>(a.mlp, xs, p.K, e_down, wsum);
            __syncthreads();
            run_units<PR, PKS, PU, PNT, Epi::Residual, true>(p.W, p.S, p.N, p.K, p.n_units, e_down, b0,
                                                        G, xs, red, w, s, wp, sp, bias, hvd);
            if (l + 1 < a.n_layers) {
                const Phase q = ph_qkv(a.layers[l + 1]);
                prefetch_block<PR, PKS, PU, PNT, Epi::QkvGather>(q.W, q.S, q.N, q.K, q.n_units,
                                                                 e_qkv, b0, w, s, wp, sp);
                barrier();
            }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0)
        __hip_atomic_store(a.bar + kBarParity, parity ^ 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

} // namespace

size_t persistent_lds_bytes(int32_t d, int32_t H, int32_t hd, int32_t dff) {
    return (size_t)std::max({d, H * hd, dff}) * 2;
}

int persistent_grid(size_t lds) {
    static std::mutex mu;
    static std::map<std::pair<int, size_t>, int> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lk(mu);
    auto key = std::make_pair(dev, lds);
    auto it = cache.find(key);
    if (it != cache.end())
        return it->second;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_persistent, kThreads, lds) !=
        hipSuccess)
        nb = 0;
    const int grid = nb * device_cus();
    cache[key] = grid;
    return grid;
}

q4_status launch_persistent(const PersistArgs &a, hipStream_t stream) {
    const size_t lds = persistent_lds_bytes(a.d, a.H, a.hd, a.dff);
    if (lds > 65536)
        return fail(Q4_ERR_UNSUPPORTED, "persistent decode: activation of %zu bytes exceeds LDS",
                    lds);
    const int grid = std::min(persistent_grid(lds), kMaxPersistentGrid);
    if (grid < 1)
        return fail(Q4_ERR_HIP, "persistent decode: no resident workgroup fits");
    hipLaunchKernelGGL(decode_persistent, dim3((unsigned)grid), dim3(kThreads), lds, stream, a);
    Q4_HIP(hipGetLastError());
    return Q4_OK;
}

} // namespace q4
