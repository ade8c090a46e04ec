// decode.h -- parameter blocks and launchers of the decode-time INT8 K cache
// (the NPU issue page on INT8 KV with per-head Hadamard rotation, part A).
#pragma once

#include "device.h"

namespace sage {

// Appends n rows to the cache at positions [t0, t0 + n): K rotated by the
// normalized Walsh-Hadamard transform and quantized to INT8 with one FP32
// scale per (head, token); V copied as BF16.
struct KvAppendParams {
    int B, Hkv, D, n, t0, cap;
    View k, v;                          // [B, n, Hkv, D] BF16 views
    int8_t *k8;                         // [B, Hkv, cap, D]
    float *k_scale;                     // [B, Hkv, cap]
    uint16_t *vc;                       // [B, Hkv, cap, D]
};

// Single-query attention of each query head over the first T cached tokens.
struct DecodeParams {
    int B, Hq, Hkv, grp, D, T, cap, nchunk;
    View q;                             // [B, 1, Hq, D] BF16 view (n = 0)
    const int8_t *k8;
    const float *k_scale;
    const uint16_t *vc;
    float *part;                        // [B, Hq, nchunk, kPartStride]: o partial, max, sum
    uint16_t *o;                        // [B, Hq, D] BF16
};

constexpr int kDecodeChunk = 256;       // cached tokens per work-group
// Chunk partial record: o[256], max, sum and two floats of padding, so that
// every record starts 16-byte aligned.
constexpr int kPartStride = 260;

}  // namespace sage

hipError_t sage_launch_kv_append(const sage::KvAppendParams &p, hipStream_t s);
hipError_t sage_launch_decode(const sage::DecodeParams &p, hipStream_t s);
