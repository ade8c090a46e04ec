// selftest.hip -- test hook for the number-format primitives of device.h.
//
// Applies one primitive of the preparation kernels to FP32 inputs given by
// their bit patterns, so that a test can compare the device rounding with an
// independent implementation over every pattern.  The primitives are the
// ones whose results are bit-exact outputs of the preparation (the page
// "Exact Numerical Contract", sections "Preparation", "Q And K
// Quantization" and "V And PV"), in the exact form those kernels use:
//   0  BF16 round to nearest even                          -> uint16
//   1  INT8 round to nearest even, saturate, NaN -> 0      -> int8
//   2  OCP E4M3 round to nearest even, saturate to 448     -> uint8
//   3  RMSNorm reciprocal  1.0f / sqrtf(x)                 -> float
//   4  quantization scale  x / 127.0f                      -> float
//   5  quantization multiplier  127.0f / x                 -> float
//   6  V scale  x / 2.25f                                  -> float
//   7  V multiplier  2.25f / x                             -> float
//   8  softmax exponential, the attention kernel's v_exp_f32 -> float
//      (not a bit-exact output: its accuracy is measured, not pinned)
//   9  OCP E4M3 as the V cast converts (pack4_e4m3_bounded) -> uint8
//      (equal to kind 2 for NaN and below 448 in magnitude)
//  10..15  the lane exchange of the row reductions and butterflies
//      (xor_lane<M>, M = 2^(kind - 10)): element i receives the input of
//      element i ^ M of its wave (a data move: the bits come through as
//      they are)                                       -> float bits
// The exchange kinds need whole waves: count a multiple of 64.

#include "device.h"
#include "lanes.h"

namespace sage {
namespace {

__global__ __launch_bounds__(256) void primitive_kernel(int kind, uint32_t first, uint32_t count, void *out) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= count) return;
    const float x = __uint_as_float(first + i);
    switch (kind) {
    case 0: static_cast<uint16_t *>(out)[i] = (uint16_t)(pack_bf16x2(x, 0.0f) & 0xffffu); break;
    case 1: static_cast<int8_t *>(out)[i] = (int8_t)to_i8(x); break;
    case 2: static_cast<uint8_t *>(out)[i] = (uint8_t)to_e4m3(x); break;
    case 3: static_cast<float *>(out)[i] = 1.0f / sqrtf(x); break;
    case 4: static_cast<float *>(out)[i] = x / 127.0f; break;
    case 5: static_cast<float *>(out)[i] = 127.0f / x; break;
    case 6: static_cast<float *>(out)[i] = x / 2.25f; break;
    case 7: static_cast<float *>(out)[i] = 2.25f / x; break;
    case 9: {
        const float v[4] = {x, 0.0f, 0.0f, 0.0f};
        static_cast<uint8_t *>(out)[i] = (uint8_t)(pack4_e4m3_bounded(v) & 0xffu);
        break;
    }
    case 10: static_cast<float *>(out)[i] = xor_lane<1>(x); break;
    case 11: static_cast<float *>(out)[i] = xor_lane<2>(x); break;
    case 12: static_cast<float *>(out)[i] = xor_lane<4>(x); break;
    case 13: static_cast<float *>(out)[i] = xor_lane<8>(x); break;
    case 14: static_cast<float *>(out)[i] = xor_lane<16>(x); break;
    case 15: static_cast<float *>(out)[i] = xor_lane<32>(x); break;
    default: static_cast<float *>(out)[i] = __builtin_amdgcn_exp2f(x); break;
    }
}

}  // namespace
}  // namespace sage

hipError_t sage_launch_primitive(int kind, uint32_t first, uint32_t count, void *out, hipStream_t s) {
    sage::primitive_kernel<<<dim3((count + 255u) / 256u), 256, 0, s>>>(kind, first, count, out);
    return hipGetLastError();
}
