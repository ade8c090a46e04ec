// device.h -- gfx950 device helpers shared by the preparation and attention
// kernels of this library: number-format conversions, lane exchanges and the
// parameter blocks the host passes to each kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Number formats.  All conversions that feed a bit-exact output round to
// nearest-even, as the contract page requires for BF16, INT8 (saturating) and
// E4M3 (saturating to the largest finite value).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// Two FP32 values -> packed BF16 pair (lo in bits 0-15), hardware RNE
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 v = {lo, hi};
    bf2 r = __builtin_convertvector(v, bf2);
    return __builtin_bit_cast(uint32_t, r);
}

// Value after rounding to BF16 (RNE), as FP32.
__device__ __forceinline__ float round_bf16(float x) { return bf16_lo(pack_bf16x2(x, 0.0f)); }

// FP32 -> INT8: round to nearest even, saturate to [-128, 127], NaN -> 0.
// v_cvt_i32_f32 itself maps NaN to 0 and saturates out-of-range values, and
// its input is already an integer here, so one med3 finishes the clamp.
__device__ __forceinline__ int32_t to_i8(float x) {
    const float r = rintf(x);                  // v_rndne_f32
    int32_t i;
    asm("v_cvt_i32_f32 %0, %1" : "=v"(i) : "v"(r));
    return min(max(i, -128), 127);
}

// FP32 -> OCP E4M3 byte, round to nearest even, saturating finite overflow to
// +-448 and NaN to 0x7F (sign kept).  Integer rounding on the FP32 encoding:
// normal results keep 3 of the 23 mantissa bits; values below 2^-6 are
// multiples of 2^-9 and are rounded with v_rndne_f32 after an exact 2^9 scale.
__device__ __forceinline__ uint32_t to_e4m3(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;
    if (a >= 0x43e00000u) return sign | 0x7eu;              // |x| >= 448
    if (a < 0x3c800000u) {                                    // |x| < 2^-6
        float q = rintf(__uint_as_float(a) * 512.0f);
        return sign | (uint32_t)q;
    }
    uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);            // RNE at bit 20
    uint32_t code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
    return sign | (code > 0x7eu ? 0x7eu : code);
}

// Four FP32 values -> four OCP E4M3 bytes (value i in byte i), equal to
// to_e4m3 of each for every value of magnitude below 448 and for NaN, which
// is all a caller may pass (the scaled V of the preparation is at most 2.25
// in magnitude).  The hardware conversion (v_cvt_pk_fp8_f32, round to nearest
// even) gives to_e4m3's byte for every such finite value; for a NaN it writes
// 0xFF whatever the sign, a byte no finite value below 448 produces, so a word
// holding one is redone with to_e4m3.
__device__ __forceinline__ uint32_t pack4_e4m3_bounded(const float (&x)[4]) {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
    if ((~r - 0x01010101u) & r & 0x80808080u)              // some byte is 0xFF
        r = to_e4m3(x[0]) | (to_e4m3(x[1]) << 8) | (to_e4m3(x[2]) << 16) | (to_e4m3(x[3]) << 24);
    return r;
}

// ---------------------------------------------------------------------------
// Lane exchanges (wave64).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = __builtin_fmaxf(v, shfl_xor_f(v, m));
    return v;
}

// ---------------------------------------------------------------------------
// Kernel parameter blocks.
// ---------------------------------------------------------------------------

struct View {
    const uint16_t *ptr;
    int64_t sb, sn, sh;
};

struct PrepParams {
    int B, N, Hq, Hkv, D, R, hadamard;
    float eps;
    View q, k, v;
    const uint16_t *w_q, *w_k;          // NULL = unit weights
    const uint16_t *cos_t, *sin_t;      // [N, R/2]
    int8_t *q8;
    float *q_scale;
    int8_t *k8;
    float *k_scale;
    float *k_mean;
    uint8_t *v8;
    float *v_scale;
    float *ws_ksum;                     // [B, Hkv, nk, D] per-tile K column sums
    float *ws_vmax;                     // [B, Hkv, nk, D] per-tile V column max |v|
    float *ws_vamax;                    // [B, Hkv, D] floored V channel maximum
    uint16_t *q_prep, *k_prep;          // optional BF16 [B, H, N, D] prepared Q / K
    int64_t q_rows, k_rows;
    int nq, nk;
};

struct AttnParams {
    int B, N, Hq, Hkv, grp, nq, nk;
    int64_t q_rows, k_rows;
    float c;                            // (1/sqrt(D)) * log2(e), FP32
    const int8_t *q8;
    const float *q_scale;
    const int8_t *k8;
    const float *k_scale;
    const uint8_t *v8;
    const float *v_scale;
    uint16_t *o;
    int64_t osb, osn, osh;
    // segmented (split-KV) schedule only: nseg runs of key tiles, and the
    // FP32 partials of each run (RO [B, Hq, nseg, N, D]; m and d [.., N, 2])
    int nseg;
    float *seg_ro;
    float *seg_md;
    // measurement only (NULL otherwise): per work-group, the shader-clock
    // counter and the constant-rate counter at the start and at the end of
    // its first wave, 4 x uint64 at stamps + 4 * (hardware block index)
    uint64_t *stamps;
};

// Clock stamps of one work-group (see AttnParams::stamps).
struct Stamp {
    uint64_t clk, wall;
};
__device__ __forceinline__ Stamp stamp_now(const uint64_t *stamps) {
    if (!stamps) return Stamp{0, 0};
    return Stamp{(uint64_t)clock64(), (uint64_t)wall_clock64()};
}
__device__ __forceinline__ void stamp_store(uint64_t *stamps, const Stamp &s0) {
    if (stamps && threadIdx.x == 0) {
        const Stamp s1{(uint64_t)clock64(), (uint64_t)wall_clock64()};
        uint64_t *dst = stamps + 4 * (int64_t)blockIdx.x;
        dst[0] = s0.clk; dst[1] = s0.wall; dst[2] = s1.clk; dst[3] = s1.wall;
    }
}

}  // namespace sage

// Host-side launchers (defined in prep.hip / attn.hip); return hipGetLastError().
hipError_t sage_launch_prep_stats(const sage::PrepParams &p, hipStream_t s);
hipError_t sage_launch_quant(const sage::PrepParams &p, hipStream_t s);
hipError_t sage_launch_attn(const sage::AttnParams &p, int D, hipStream_t s);
hipError_t sage_launch_attn_segmented(const sage::AttnParams &p, int D, hipStream_t s);

// In-tile key order of a v8 tile row: slot -> key (both 0..63).
__host__ __device__ __forceinline__ int sage_v8_slot_key(int slot) {
    // slot = 32*h + 16*c + r  <->  key = 32*c + 8*(r/4) + 4*h + r%4 : the key
    // that the INT8 QK accumulator register r of block c holds in lane half h.
    int h = slot >> 5, c = (slot >> 4) & 1, r = slot & 15;
    return 32 * c + 8 * (r >> 2) + 4 * h + (r & 3);
}
