// Cross-lane reductions of a 64-lane wave as VALU operations (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {
namespace lanes {

// Cross-lane steps as VALU operations (DPP and gfx950's lane swaps) rather
// than LDS permutes: they sit on the critical path of every reduction.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1; // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E; // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// Values of the lanes 16 and 32 away, pairwise combined: every lane gets
// op(x[row r], x[row r ^ 1]) (16-lane rows) resp. op(x[lane], x[lane ^ 32]).
struct Rows16 {
    unsigned a, b;
    __device__ __forceinline__ Rows16(float x) {
        auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
        a = r[0];
        b = r[1];
    }
};
struct Halves32 {
    unsigned a, b;
    __device__ __forceinline__ Halves32(float x) {
        auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
        a = r[0];
        b = r[1];
    }
};
__device__ __forceinline__ float fa(unsigned u) { return __builtin_bit_cast(float, u); }

// Sum / max over all 64 lanes, result in every lane.
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<kQuadXor1>(x);
    x += dpp<kQuadXor2>(x);
    x += dpp<kRowRor4>(x);
    x += dpp<kRowRor8>(x);
    const Rows16 r(x);
    x = fa(r.a) + fa(r.b);
    const Halves32 h(x);
    return fa(h.a) + fa(h.b);
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<kQuadXor1>(x));
    x = fmaxf(x, dpp<kQuadXor2>(x));
    x = fmaxf(x, dpp<kRowRor4>(x));
    x = fmaxf(x, dpp<kRowRor8>(x));
    const Rows16 r(x);
    x = fmaxf(fa(r.a), fa(r.b));
    const Halves32 h(x);
    return fmaxf(fa(h.a), fa(h.b));
}


} // namespace lanes
} // namespace q4
