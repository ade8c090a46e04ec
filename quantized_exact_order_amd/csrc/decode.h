// decode.h -- parameter blocks and launchers of the decode-time INT8 K cache
// (the NPU issue page on INT8 KV with per-head Hadamard rotation, part A).
#pragma once

#include "device.h"

namespace sage {

// V cache layout: BF16 blocks of 8 consecutive tokens per channel, element
// (t, d) of a (batch, KV head) at ((t / 8) * D + d) * 8 + t % 8, so that one
// 16-byte load gives a channel's 8 tokens (the B operand of the PV MFMA).
constexpr int kVBlock = 8;

// Appends n rows to the cache at positions [t0, t0 + n): K rotated by the
// normalized Walsh-Hadamard transform and quantized to INT8 with one FP32
// scale per (head, token); V copied as BF16 into its 8-token blocks, or
// rotated and quantized as K into INT8 8-token blocks.
struct KvAppendParams {
    int B, Hkv, D, n, t0, cap, nblk;    // nblk: 8-token blocks touched by [t0, t0 + n)
    View k, v;                          // [B, n, Hkv, D] BF16 views
    int8_t *k8;                         // [B, Hkv, cap, D]
    float *k_scale;                     // [B, Hkv, cap]
    uint16_t *vc;                       // [B, Hkv, cap / 8, D, 8], or NULL with INT8 V:
    int8_t *v8c;                        // [B, Hkv, cap / 8, D, 8] rotated INT8 V
    float *v_scale;                     // [B, Hkv, cap]
};

// Single-query attention of each query head over the first T cached tokens.
struct DecodeParams {
    int B, Hq, Hkv, grp, D, T, cap;
    int ns, nchunk;                     // 32-token steps per wave; chunks of 128 * ns tokens
    View q;                             // [B, 1, Hq, D] BF16 view (n = 0)
    const int8_t *k8;
    const float *k_scale;
    const uint16_t *vc;                 // BF16 V, or NULL with INT8 V:
    const int8_t *v8c;                  // rotated INT8 V (the output is rotated back)
    const float *v_scale;
    float *part;                        // [B, Hq, nchunk, kPartStride]: o partial, max, sum
    uint16_t *o;                        // [B, Hq, D] BF16
};

constexpr int kDecodeMaxGroup = 16;     // query heads per KV head (MFMA columns)
constexpr int kDecodeMaxSteps = 16;
// Chunk partial record: o[256], max, sum and two floats of padding, so that
// every record starts 16-byte aligned.
constexpr int kPartStride = 260;

// Steps per wave: about 512 work-groups over the whole cache (two per CU),
// between 1 and kDecodeMaxSteps.
inline int decode_steps(int B, int Hkv, int T) {
    const int64_t ns = (int64_t)B * Hkv * T / (128 * 512);
    return ns < 1 ? 1 : (ns > kDecodeMaxSteps ? kDecodeMaxSteps : (int)ns);
}
inline int64_t decode_nchunk(int B, int Hkv, int T) {
    const int64_t c = 128 * (int64_t)decode_steps(B, Hkv, T);
    return (T + c - 1) / c;
}
// Workspace: the chunk partials.
inline int64_t decode_ws_bytes(int B, int Hq, int Hkv, int T) {
    return (int64_t)B * Hq * decode_nchunk(B, Hkv, T) * kPartStride * 4;
}

// Size of the fixed per-GPU array that the allocation-free decode uses in
// place of the workspace: 16 MiB, 16,131 chunk records, e.g. the partials of
// B = 4 sequences of 32 query heads over 131,072 cached tokens (8.5 MB).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;

}  // namespace sage

hipError_t sage_launch_kv_append(const sage::KvAppendParams &p, hipStream_t s);
hipError_t sage_launch_decode(const sage::DecodeParams &p, hipStream_t s);
// Device address of the current GPU's fixed decode scratch array, looked up
// once per device (hipGetSymbolAddress) and kept.
hipError_t sage_decode_scratch(void **ptr);
