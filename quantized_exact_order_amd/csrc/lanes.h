// lanes.h -- xor lane exchanges within a wave64 by the cheapest instruction
// for each distance, for the row reductions and butterflies of the
// preparation and decode kernels.  The exchanged values are the same as
// those of __shfl_xor (a ds_bpermute through the LDS unit, with its address
// arithmetic); only the instruction differs.
#pragma once

#include <type_traits>

#include "device.h"

namespace sage {

// The value that lane l ^ M holds (M a power of two below 64), all by VALU
// lane moves:
//   M = 1, 2:  DPP quad permutation (v_mov_b32_dpp quad_perm);
//   M = 4:     DPP row_half_mirror (l -> l ^ 7 within 8 lanes), then quad_perm
//              [3, 2, 1, 0] (l -> l ^ 3 within 4);
//   M = 8:     DPP row_ror:8 (a rotation by 8 within 16 lanes is l ^ 8);
//   M = 16:    v_permlane16_swap, M = 32: v_permlane32_swap; each returns the
//              partner rows' values to one half of the lanes in its first
//              result and to the other half in its second.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "xor distance");
    const int x = __float_as_int(v);
    int r;
    if constexpr (M == 1) {
        r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);          // quad_perm [1, 0, 3, 2]
    } else if constexpr (M == 2) {
        r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);          // quad_perm [2, 3, 0, 1]
    } else if constexpr (M == 4) {
        const int hm = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);  // row_half_mirror
        r = __builtin_amdgcn_mov_dpp(hm, 0x1B, 0xF, 0xF, false);          // quad_perm [3, 2, 1, 0]
    } else if constexpr (M == 8) {
        r = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);         // row_ror:8
    } else if constexpr (M == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        r = (threadIdx.x & 16) ? (int)p[0] : (int)p[1];
    } else {
        const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        r = (threadIdx.x & 32) ? (int)p[0] : (int)p[1];
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
