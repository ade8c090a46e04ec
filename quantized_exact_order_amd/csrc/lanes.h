// lanes.h -- xor lane exchanges within a wave64 by the cheapest instruction
// for each distance, for the row reductions and butterflies of the
// preparation and decode kernels.  The exchanged values are the same as
// those of __shfl_xor (a ds_bpermute through the LDS unit, with its address
// arithmetic); only the instruction differs.
#pragma once

#include <type_traits>

#include "device.h"

namespace sage {

// The value that lane l ^ M holds (M a power of two below 64):
//   M = 1, 2:      DPP quad permutation (v_mov_b32_dpp);
//   M = 4, 8, 16:  ds_swizzle_b32 in bitmask mode (within groups of 32 lanes:
//                  and-mask 0x1F, or-mask 0, xor-mask M), no LDS access;
//   M = 32:        v_permlane32_swap, which returns the upper half's values
//                  to the lower half and the lower half's to the upper one.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "xor distance");
    const int x = __float_as_int(v);
    int r;
    if constexpr (M == 1) {
        r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);          // quad_perm [1, 0, 3, 2]
    } else if constexpr (M == 2) {
        r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);          // quad_perm [2, 3, 0, 1]
    } else if constexpr (M == 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        r = (threadIdx.x & 32) ? (int)p[0] : (int)p[1];
    } else {
        r = __builtin_amdgcn_ds_swizzle(x, (M << 10) | 0x1F);
    }
    return __int_as_float(r);
}

// f(std::integral_constant<int, M>) for M = FROM, 2 FROM, ... below END.
template <int FROM, int END, typename F>
__device__ __forceinline__ void for_pow2(F &&f) {
    if constexpr (FROM < END) {
        f(std::integral_constant<int, FROM>{});
        for_pow2<2 * FROM, END>(f);
    }
}

// Maximum over the wave (any order gives the same value).
__device__ __forceinline__ float wave_max_x(float v) {
    for_pow2<1, 64>([&](auto m) { v = __builtin_fmaxf(v, xor_lane<decltype(m)::value>(v)); });
    return v;
}

}  // namespace sage
