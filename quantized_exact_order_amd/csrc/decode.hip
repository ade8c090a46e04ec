// decode.hip -- decode-time INT8 K cache with per-head Hadamard rotation
// (the NPU issue page on INT8 KV with per-head Hadamard rotation, part A):
//   cache:  u = H k / sqrt(D) (normalized Walsh-Hadamard transform, FP32
//           butterflies span 1, 2, 4, ... in that order), amax = max(1e-7,
//           max|u|), k_scale = amax/127, k8 = rni_sat(u * (127/amax)); V BF16
//   query:  qr = H q / sqrt(D) (the same transform), so qr . u = q . k
//   decode: s_t = (qr . k8_t) * k_scale_t / sqrt(D), w = softmax(s),
//           o = sum_t w_t v_t, rounded to BF16.
// D = 256 (the page's head width; 1/sqrt(256) = 1/16 is exact).
//
// Decode reads the cache once: the work-group of (b, KV head, chunk of
// 128 ns tokens) serves all Hq/Hkv (<= 16) query heads of that KV head; its
// four waves take interleaved 32-token steps (so the work-group streams one
// contiguous range), each with an online softmax over its steps, and both
// contractions run on the matrix cores:
//   * scores: the rotated query of each head is expanded as
//     qr = s1 q1 + s2 q2 + s3 q3 + r with INT8 parts q_j, s_{j+1} = s_j / 128
//     and |r| <= s3 / 2 (below FP32 rounding of qr . k8), so that
//     qr . k8 = sum_j s_j (q_j . k8) with exact INT32 dot products
//     (v_mfma_i32_16x16x64_i8: 16 tokens x 16 heads, K rows read straight
//     from the cache as the A operand);
//   * PV: w = w_hi + w_lo (two BF16 parts, |w_lo| <= 2^-9 |w|, the rest below
//     2^-17 |w|) times BF16 V (v_mfma_f32_16x16x32_bf16, FP32 accumulation);
//     the cache keeps V in 8-token blocks per channel, so one 16-byte load is
//     a lane's B operand.
// The chunk's softmax partial (max, sum, o) goes to a workspace, and a second
// kernel combines the chunks in a fixed order.
// INT8 V (the same page: an INT8 V is rotated like K and needs the transform
// once more on the output): V rows are rotated and quantized as K rows, into
// 8-token blocks of bytes; the PV step folds each token's V scale into its
// weight and widens the bytes to BF16 exactly, and the combine applies the
// normalized transform (its own inverse) to the output before rounding.

#include "decode.h"
#include "lanes.h"

#include <mutex>

namespace sage {
namespace {

// Normalized 256-point Walsh-Hadamard transform of a row held as 4 values per
// lane (element 4 lane + i).  Stage span 1 and 2 inside the lane, spans 4..128
// across lanes 1..32 apart; each pair (a, b) -> (a + b, a - b) in FP32.
__device__ __forceinline__ void wht256(float u[4], int lane) {
    float a = u[0], b = u[1];
    u[0] = a + b; u[1] = a - b;
    a = u[2]; b = u[3];
    u[2] = a + b; u[3] = a - b;
    a = u[0]; b = u[2];
    u[0] = a + b; u[2] = a - b;
    a = u[1]; b = u[3];
    u[1] = a + b; u[3] = a - b;
    for_pow2<1, 64>([&](auto m) {
        constexpr int lm = decltype(m)::value;
        const bool upper = (lane & lm) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float other = xor_lane<lm>(u[i]);
            u[i] = upper ? (other - u[i]) : (u[i] + other);
        }
    });
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = u[i] * 0.0625f;
}

__device__ __forceinline__ void load4(const uint16_t *row, int lane, float x[4]) {
    const uint2 r = *reinterpret_cast<const uint2 *>(row + 4 * lane);
    x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x);
    x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Rotates and quantizes one BF16 row of 256 (one wave): returns the INT8
// values of channels 4 lane .. 4 lane + 3 packed in a word, and the row's
// amax = max(1e-7, max|u|) (the scale is amax / 127).
__device__ __forceinline__ uint32_t rot_quant_row(const uint16_t *row, int lane, float &amax) {
    float u[4];
    load4(row, lane, u);
    wht256(u, lane);
    float m = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(u[0]), __builtin_fabsf(u[1])),
                              __builtin_fmaxf(__builtin_fabsf(u[2]), __builtin_fabsf(u[3])));
    m = wave_max_x(m);
    amax = (m > 1e-7f) ? m : 1e-7f;
    const float mul = 127.0f / amax;
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= (uint32_t)(to_i8(u[i] * mul) & 0xff) << (8 * i);
    return w;
}

// Row t (cache position) of head h of a new K or V view; one wave.
__device__ __forceinline__ const uint16_t *new_row(const View &x, int t0, int b, int h, int t) {
    return x.ptr + (int64_t)b * x.sb + (int64_t)(t - t0) * x.sn + (int64_t)h * x.sh;
}

// Rotates, quantizes and stores K row t (cache position) of head h; one wave.
__device__ __forceinline__ void append_k_row(const KvAppendParams &p, int b, int h, int t, int lane) {
    const int64_t c = ((int64_t)b * p.Hkv + h) * p.cap + t;          // cache row
    float amax;
    const uint32_t w = rot_quant_row(new_row(p.k, p.t0, b, h, t), lane, amax);
    reinterpret_cast<uint32_t *>(p.k8 + c * 256)[lane] = w;
    if (lane == 0) p.k_scale[c] = amax / 127.0f;
}

// INT8 V: the new rows of 8-token block blk, rotated and quantized as K rows,
// into the block's bytes: lane owns channels 4 lane .. 4 lane + 3, 8 bytes
// (tokens) each, 32 contiguous bytes.
__device__ __forceinline__ void append_v8_block(const KvAppendParams &p, int b, int h, int blk, int ta, int te,
                                                int lane) {
    const int tb = kVBlock * blk;
    uint4 *dst = reinterpret_cast<uint4 *>(
        p.v8c + ((((int64_t)b * p.Hkv + h) * (p.cap / kVBlock) + blk) * 256 + 4 * lane) * kVBlock);
    uint4 w0 = make_uint4(0, 0, 0, 0), w1 = make_uint4(0, 0, 0, 0);
    if (te - ta < kVBlock) {
        w0 = dst[0];
        w1 = dst[1];
    }
    // channel i: tokens 0..3 in wd[i][0], 4..7 in wd[i][1], token e in byte e % 4
    uint32_t wd[4][2] = {{w0.x, w0.y}, {w0.z, w0.w}, {w1.x, w1.y}, {w1.z, w1.w}};
    for (int t = ta; t < te; ++t) {
        float amax;
        const uint32_t q = rot_quant_row(new_row(p.v, p.t0, b, h, t), lane, amax);
        const int e = t - tb, sh = 8 * (e & 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t byte = ((q >> (8 * i)) & 0xffu) << sh, keep = ~(0xffu << sh);
            if (e < 4) wd[i][0] = (wd[i][0] & keep) | byte;
            else wd[i][1] = (wd[i][1] & keep) | byte;
        }
        if (lane == 0) p.v_scale[((int64_t)b * p.Hkv + h) * p.cap + t] = amax / 127.0f;
    }
    dst[0] = make_uint4(wd[0][0], wd[0][1], wd[1][0], wd[1][1]);
    dst[1] = make_uint4(wd[2][0], wd[2][1], wd[3][0], wd[3][1]);
}

// One wave per (b, KV head, 8-token block touched by [t0, t0 + n)): the K rows
// of the block's new tokens one by one, then the V block, lane owning
// channels 4 lane .. 4 lane + 3 (four 16-byte vectors of 8 tokens each; the
// tokens of the block outside [t0, t0 + n) keep their cached values).
// Grid (ceil(nblk * Hkv / 4), B).
__global__ __launch_bounds__(256) void kv_append_kernel(const KvAppendParams p) {
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= p.nblk * p.Hkv) return;
    const int h = item % p.Hkv, blk = (p.t0 >> 3) + item / p.Hkv, b = blockIdx.y;
    const int tb = kVBlock * blk;
    const int ta = max(tb, p.t0), te = min(tb + kVBlock, p.t0 + p.n);    // new tokens [ta, te)
    for (int t = ta; t < te; ++t) append_k_row(p, b, h, t, lane);
    if (p.v8c) {
        append_v8_block(p, b, h, blk, ta, te, lane);
        return;
    }

    uint4 *dst = reinterpret_cast<uint4 *>(
        p.vc + ((((int64_t)b * p.Hkv + h) * (p.cap / kVBlock) + blk) * 256 + 4 * lane) * kVBlock);
    uint32_t w[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint4 old = make_uint4(0, 0, 0, 0);
        if (te - ta < kVBlock) old = dst[i];
        w[i][0] = old.x; w[i][1] = old.y; w[i][2] = old.z; w[i][3] = old.w;
    }
#pragma unroll
    for (int e = 0; e < kVBlock; ++e) {
        const int t = tb + e;
        if (t >= ta && t < te) {
            const uint2 s = *reinterpret_cast<const uint2 *>(p.v.ptr + (int64_t)b * p.v.sb +
                                                             (int64_t)(t - p.t0) * p.v.sn +
                                                             (int64_t)h * p.v.sh + 4 * lane);
            const uint32_t hv[4] = {s.x & 0xffffu, s.x >> 16, s.y & 0xffffu, s.y >> 16};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t &x = w[i][e >> 1];
                x = (e & 1) ? ((x & 0x0000ffffu) | (hv[i] << 16)) : ((x & 0xffff0000u) | hv[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(w[i][0], w[i][1], w[i][2], w[i][3]);
}

constexpr int kQRow = 272;      // LDS bytes per head row of the query parts (rows 4 banks apart)

// The A operands (K rows) and K scales of the 32-token step starting at ts:
// MFMA block bb row m is token ts + 8 (m / 4) + 4 bb + m % 4 (clamped to the
// last valid row), so that accumulator register i of lane group q4 is token
// ts + 8 q4 + 4 bb + i; k0, k1 get the scales of tokens ts + 8 q4 .. + 7.
struct KStep {
    v4i a[2][4];
    float4 k0, k1;
};

__device__ __forceinline__ void load_k_rows(KStep &k, const int8_t *kb, int ts, int T, int q4, int r16) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        const int tok = min(ts + 8 * (r16 >> 2) + 4 * bb + (r16 & 3), T - 1);
        const int8_t *kr = kb + (int64_t)tok * 256 + 16 * q4;
#pragma unroll
        for (int s = 0; s < 4; ++s) k.a[bb][s] = *reinterpret_cast<const v4i *>(kr + 64 * s);
    }
}
__device__ __forceinline__ void load_k_scales(KStep &k, const float *ksb, int ts, int T, int q4) {
    // a group of 8 past T reads the last valid group (its scores are masked);
    // t8 + 8 <= capacity since both are multiples of 8
    const int t8 = min(ts + 8 * q4, ((T - 1) / 8) * 8);
    const v4f s0 = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(ksb + t8));
    const v4f s1 = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(ksb + t8 + 4));
    k.k0 = make_float4(s0[0], s0[1], s0[2], s0[3]);
    k.k1 = make_float4(s1[0], s1[1], s1[2], s1[3]);
}
__device__ __forceinline__ void load_k_step(KStep &k, const int8_t *kb, const float *ksb, int ts, int T,
                                            int q4, int r16) {
    load_k_rows(k, kb, ts, T, q4, r16);
    load_k_scales(k, ksb, ts, T, q4);
}

// The V block of tokens ts + 8 q4 .. + 7 for channels 16 nb + r16 (the B
// operands of the step); a block past T reads the last valid block and is
// masked to zero before use.
__device__ __forceinline__ void load_v_step(uint4 vv[16], const uint16_t *vb, int ts, int T, int q4, int r16) {
    const int blk = min(ts / kVBlock + q4, (T - 1) / kVBlock);
    const uint16_t *vr = vb + ((int64_t)blk * 256 + r16) * kVBlock;
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) {
        const v4i x = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(vr + nb * 16 * kVBlock));
        vv[nb] = make_uint4(x[0], x[1], x[2], x[3]);
    }
}

// INT8 V: the 8 bytes (tokens ts + 8 q4 .. + 7) of channels 16 nb + r16 and
// the V scales of those tokens; a block past T reads the last valid block
// (its weights are zero and its scales are not used).
__device__ __forceinline__ void load_v8_step(uint4 vv[16], float4 &s0, float4 &s1, const int8_t *vb,
                                             const float *vsb, int ts, int T, int q4, int r16) {
    const int blk = min(ts / kVBlock + q4, (T - 1) / kVBlock);
    const int8_t *vr = vb + ((int64_t)blk * 256 + r16) * kVBlock;
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) {
        typedef int v2i __attribute__((ext_vector_type(2)));
        const v2i x = __builtin_nontemporal_load(reinterpret_cast<const v2i *>(vr + nb * 16 * kVBlock));
        vv[nb] = make_uint4(x[0], x[1], 0u, 0u);
    }
    const v4f a = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(vsb + blk * kVBlock));
    const v4f c = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(vsb + blk * kVBlock + 4));
    s0 = make_float4(a[0], a[1], a[2], a[3]);
    s1 = make_float4(c[0], c[1], c[2], c[3]);
}

// Two INT8 values (bytes 2 j and 2 j + 1 of w) as a BF16 pair, exactly
// (integers of magnitude <= 128 have at most 8 significant bits).
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int j) {
    const float a = (float)(int8_t)(w >> (16 * j)), c = (float)(int8_t)(w >> (16 * j + 8));
    // the high halves of a (bytes 2, 3) and c (bytes 6, 7 of the pair c:a)
    return __builtin_amdgcn_perm(__float_as_uint(c), __float_as_uint(a), 0x07060302u);
}

// Chunk partial of the grp (<= 16) query heads of one KV head over tokens
// [128 ns chunk, 128 ns (chunk + 1)).  Grid (nchunk * Hkv, B), 256 threads;
// step st of wave w covers tokens 128 ns chunk + 128 st + 32 w + [0, 32), so
// the four waves of a step read adjacent tokens and the work-group streams
// one contiguous range of the cache.  Each wave runs an online softmax over
// its steps (each step's V loads are issued before its K loads, so they are
// in flight while the scores compute), and the four waves' partials are
// merged in order.  The query expansion runs while the first step's loads are
// in flight.  The cache is read once: the V and scale loads are
// nontemporal.  The K loads are not: each reads 64 bytes of each of 16 rows
// (half a cache line per row), and with that shape a nontemporal hint made
// the step slower (87 against 80 us on the decode workload).
template <bool kInt8V>
__global__ __launch_bounds__(256, 2) void decode_chunk_kernel(const DecodeParams p) {
    __shared__ __attribute__((aligned(16))) int8_t qp[3][kDecodeMaxGroup][kQRow];   // query parts
    __shared__ float qsc[3][kDecodeMaxGroup];                                        // their scales
    __shared__ float wm[4][kDecodeMaxGroup];                                         // per-wave maxima
    __shared__ float wl[4][kDecodeMaxGroup];                                         // per-wave sums
    __shared__ __attribute__((aligned(16))) float osum[kDecodeMaxGroup][260];

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q4 = lane >> 4, r16 = lane & 15;
    const int hk = blockIdx.x % p.Hkv, chunk = blockIdx.x / p.Hkv, b = blockIdx.y;
    const int64_t bh = (int64_t)b * p.Hkv + hk;
    const int T = p.T;

    const int tw = chunk * 128 * p.ns + 32 * wave;          // the wave's first token
    const int nst = T > tw ? min((T - tw + 127) / 128, p.ns) : 0;
    const int8_t *kb = p.k8 + bh * p.cap * 256;
    const float *ksb = p.k_scale + bh * p.cap;
    const uint16_t *vb = p.vc + bh * p.cap * 256;
    const int8_t *vb8 = p.v8c + bh * p.cap * 256;
    const float *vsb = p.v_scale + bh * p.cap;
    // the query rows of this wave's heads g = wave + 4 i are loaded first, so
    // that waiting for them does not wait for the step loads issued after
    // (unconditionally: heads g >= grp read head grp - 1, are expanded like
    // the others and then zeroed, so no load is sunk into a conditional block
    // whose wait would also wait for the step loads)
    float xq[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = min(wave + 4 * i, p.grp - 1);
        load4(p.q.ptr + (int64_t)b * p.q.sb + (int64_t)(hk * p.grp + g) * p.q.sh, lane, xq[i]);
    }
    // the first step's loads, unconditionally (a wave with no tokens reads
    // clamped, valid rows and does not use them)
    KStep k;
    uint4 vv[16];
    float4 vs0, vs1;                        // INT8 V: scales of the lane's 8 tokens
    load_k_step(k, kb, ksb, tw, T, q4, r16);
    if constexpr (kInt8V) load_v8_step(vv, vs0, vs1, vb8, vsb, tw, T, q4, r16);
    else load_v_step(vv, vb, tw, T, q4, r16);
    __builtin_amdgcn_sched_barrier(0);      // every load above is issued before the expansion

    // rotated queries -> three INT8 parts q_j with scales s_j (s_{j+1} =
    // s_j / 128), qr = sum_j s_j q_j + r, |r| <= s3 / 2; zero rows for the
    // unused MFMA columns g >= grp
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = wave + 4 * i;
        uint32_t wd[3] = {0u, 0u, 0u};
        float sj[3] = {0.0f, 0.0f, 0.0f};
        float *x = xq[i];
        wht256(x, lane);
        float a = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(x[0]), __builtin_fabsf(x[1])),
                                  __builtin_fmaxf(__builtin_fabsf(x[2]), __builtin_fabsf(x[3])));
        a = wave_max_x(a);
        float sc = a / 127.0f, mu = 127.0f / a;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const bool ok = a > 0.0f && mu <= 3.0e38f;      // a nonzero row, a finite multiplier
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int qv = ok ? to_i8(x[e] * mu) : 0;
                wd[j] |= (uint32_t)(qv & 0xff) << (8 * e);
                x[e] = __builtin_fmaf(-(float)qv, sc, x[e]);
            }
            sj[j] = a > 0.0f ? sc : 0.0f;
            sc = sc * 0.0078125f;
            mu = mu * 128.0f;
        }
        const bool used = g < p.grp;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            *reinterpret_cast<uint32_t *>(&qp[j][g][4 * lane]) = used ? wd[j] : 0u;
            if (lane == 0) qsc[j][g] = used ? sj[j] : 0.0f;
        }
    }
    __syncthreads();
    const float s1 = qsc[0][r16], s2 = qsc[1][r16], s3 = qsc[2][r16];

    float m = -INFINITY, l = 0.0f;          // running max and lane-partial sum of head r16
    v4f o[16];                              // register i: head 4 q4 + i, channel 16 nb + r16
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) o[nb] = v4f{0.f, 0.f, 0.f, 0.f};
    // Step st finds in flight, in this order: its K rows, its K scales and
    // its V.  The K rows of step st + 1 go out once the scores have read this
    // step's, its K scales once the dequantization has read this step's, and
    // its V once the PV products have read this step's.  Every step issues
    // the same loads, so that the compiler's waits count them exactly: on the
    // last step they are dummies, every lane reading the first row or block
    // of the step (one cache line per load), and nothing uses them.
#pragma unroll 1
    for (int st = 0; st < nst; ++st) {
        const int ts = tw + 128 * st;
        const bool more = st + 1 < nst;
        const int tn = more ? ts + 128 : ts;
        const int q4n = more ? q4 : 0, r16n = more ? r16 : 0;

        // scores of tokens ts + 8 q4 + e, head r16: B operand (part j, d-step
        // s) = bytes 16 q4 + 64 s .. + 15 of part j of head r16
        float sc[8];
        const int t8 = ts + 8 * q4;
        const float ks[8] = {k.k0.x, k.k0.y, k.k0.z, k.k0.w, k.k1.x, k.k1.y, k.k1.z, k.k1.w};
        v4i acc[2][3];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int j = 0; j < 3; ++j) acc[bb][j] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                // volatile: read at its use each step, not hoisted out of the loop
                typedef const volatile v4i __attribute__((address_space(3))) *lds_v4i;
                const v4i qb = *(lds_v4i)(uintptr_t)(uint32_t)(uintptr_t)&qp[j][r16][16 * q4 + 64 * s];
#pragma unroll
                for (int bb = 0; bb < 2; ++bb)
                    acc[bb][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k.a[bb][s], qb, acc[bb][j], 0, 0, 0);
            }
        // the next step's K rows into the registers the scores just read
        load_k_rows(k, kb, tn, T, q4n, r16n);
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * bb + i;
                float x = (float)acc[bb][0][i] * s1;
                x = __builtin_fmaf((float)acc[bb][1][i], s2, x);
                x = __builtin_fmaf((float)acc[bb][2][i], s3, x);
                sc[e] = (t8 + e < T) ? x * (ks[e] * 0.0625f) : -INFINITY;
            }
        // and its K scales into the registers the dequantization just read
        load_k_scales(k, ksb, tn, T, q4n);

        // online softmax over the step (its first token is valid: mx is finite)
        float mx = sc[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = __builtin_fmaxf(mx, sc[e]);
        mx = __builtin_fmaxf(mx, xor_lane<16>(mx));
        mx = __builtin_fmaxf(mx, xor_lane<32>(mx));
        const float mn = __builtin_fmaxf(m, mx);
        const float alpha = expf(m - mn);                   // 0 on the first step
        l = l * alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sc[e] = expf(sc[e] - mn);                       // invalid tokens: exp(-inf) = 0
            l = l + sc[e];
        }
        m = mn;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
            float al[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * q4 + i, 64);
#pragma unroll
            for (int nb = 0; nb < 16; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[nb][i] = o[nb][i] * al[i];
        }

        // PV: A = weights (head r16, tokens ts + 8 q4 + e) as BF16 hi + lo,
        // B = the V block of the same tokens; V slots past T zeroed
        const int nv = T - (ts + 8 * q4);
        uint32_t mk[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) mk[c] = nv >= 2 * c + 2 ? 0xffffffffu : (nv == 2 * c + 1 ? 0x0000ffffu : 0u);
        if constexpr (kInt8V) {
            // INT8 V: each token's V scale goes into its weight (tokens past
            // T get weight 0 whatever their scale slot holds)
            const float vsc[8] = {vs0.x, vs0.y, vs0.z, vs0.w, vs1.x, vs1.y, vs1.z, vs1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[e] = e < nv ? sc[e] * vsc[e] : 0.0f;
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float a = sc[2 * c], d = sc[2 * c + 1];
            hi[c] = pack_bf16x2(a, d);
            lo[c] = pack_bf16x2(a - bf16_lo(hi[c]), d - bf16_hi(hi[c]));
        }
        const v8bf wh = __builtin_bit_cast(v8bf, hi), wl8 = __builtin_bit_cast(v8bf, lo);
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) {
            uint4 v = vv[nb];
            if constexpr (kInt8V) {
                v = make_uint4(i8x2_to_bf16x2(v.x, 0), i8x2_to_bf16x2(v.x, 1), i8x2_to_bf16x2(v.y, 0),
                               i8x2_to_bf16x2(v.y, 1));
            } else {
                v.x &= mk[0]; v.y &= mk[1]; v.z &= mk[2]; v.w &= mk[3];
            }
            const v8bf bv = __builtin_bit_cast(v8bf, v);
            o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, bv, o[nb], 0, 0, 0);
            o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl8, bv, o[nb], 0, 0, 0);
        }
        if constexpr (kInt8V) load_v8_step(vv, vs0, vs1, vb8, vsb, tn, T, q4n, r16n);
        else load_v_step(vv, vb, tn, T, q4n, r16n);
    }

    // merge the four waves: M = max_w m_w, o = sum_w o_w e^(m_w - M) in the
    // order 0, 1, 2, 3 (wave 0 starts at the chunk's first token, which is
    // valid; a wave with no tokens has m = -inf and adds zero)
    l = l + xor_lane<16>(l);
    l = l + xor_lane<32>(l);
    if (q4 == 0) {
        wm[wave][r16] = m;
        wl[wave][r16] = l;
    }
    __syncthreads();
    float fo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = 4 * q4 + i;
        const float M = __builtin_fmaxf(__builtin_fmaxf(wm[0][g], wm[1][g]), __builtin_fmaxf(wm[2][g], wm[3][g]));
        fo[i] = expf(wm[wave][g] - M);
    }
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int nb = 0; nb < 16; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int g = 4 * q4 + i;
                    if (g < p.grp) {
                        float &s = osum[g][16 * nb + r16];
                        const float x = o[nb][i] * fo[i];
                        s = (w == 0) ? x : s + x;
                    }
                }
        }
        __syncthreads();
    }
    for (int idx = threadIdx.x; idx < p.grp * 256; idx += 256) {
        const int g = idx >> 8, d = idx & 255;
        p.part[(((int64_t)b * p.Hq + hk * p.grp + g) * p.nchunk + chunk) * kPartStride + d] = osum[g][d];
    }
    if ((int)threadIdx.x < p.grp) {
        const int g = threadIdx.x;
        float *dst = p.part + (((int64_t)b * p.Hq + hk * p.grp + g) * p.nchunk + chunk) * kPartStride;
        const float M = __builtin_fmaxf(__builtin_fmaxf(wm[0][g], wm[1][g]), __builtin_fmaxf(wm[2][g], wm[3][g]));
        float L = 0.0f;
        for (int w = 0; w < 4; ++w) L = L + wl[w][g] * expf(wm[w][g] - M);
        dst[256] = M;
        dst[257] = L;
    }
}

// Combines the chunk partials of one query head: M = max_c m_c,
// f_c = e^(m_c - M), L = sum_c l_c f_c, O = (sum_c o_c f_c) / L.  Thread
// (group cg, channel d) of the 1024 sums o_c[d] f_c over the chunks c = cg,
// cg + 4, ... in increasing order; the four group sums are added in the order
// 0, 1, 2, 3, and L is summed in increasing c (a fixed order: the result is
// deterministic).  The first partials a thread needs are loaded together with
// the maxima, so a short combine takes one round trip to memory.
// Grid (Hq, B), 1024 threads.
constexpr int kCombineThreads = 1024;
constexpr int kCombineChunks = 1024;    // chunks whose weights one pass keeps in LDS
constexpr int kCombineAhead = 8;        // partials per thread loaded before the maximum

__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(const DecodeParams p) {
    __shared__ float wmax[kCombineThreads / 64];
    __shared__ float fw[kCombineChunks];
    __shared__ float lw[kCombineChunks];
    __shared__ float og[4][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
    const int d = tid & 255, cg = tid >> 8;
    const int h = blockIdx.x, b = blockIdx.y, nchunk = p.nchunk;
    const float *src = p.part + ((int64_t)b * p.Hq + h) * nchunk * kPartStride;

    float pv[kCombineAhead];
#pragma unroll
    for (int i = 0; i < kCombineAhead; ++i) {
        const int c = cg + 4 * i;
        pv[i] = c < nchunk ? src[(int64_t)c * kPartStride + d] : 0.0f;
    }
    float mc = -INFINITY, lc = 0.0f;
    if (tid < nchunk) {
        mc = src[(int64_t)tid * kPartStride + 256];
        lc = src[(int64_t)tid * kPartStride + 257];
    }
    float M = mc;
    for (int c = tid + kCombineThreads; c < nchunk; c += kCombineThreads)
        M = __builtin_fmaxf(M, src[(int64_t)c * kPartStride + 256]);
    M = wave_max_x(M);
    if (lane == 0) wmax[wave] = M;
    __syncthreads();
    M = wmax[0];
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) M = __builtin_fmaxf(M, wmax[w]);

    float L = 0.0f, o = 0.0f;
    for (int c0 = 0; c0 < nchunk; c0 += kCombineChunks) {
        const int nc = min(kCombineChunks, nchunk - c0);
        if (c0 > 0) {
            __syncthreads();                // the previous pass's weights are consumed
            if (tid < nc) {
                mc = src[(int64_t)(c0 + tid) * kPartStride + 256];
                lc = src[(int64_t)(c0 + tid) * kPartStride + 257];
            }
        }
        if (tid < nc) {
            fw[tid] = expf(mc - M);
            lw[tid] = lc;
        }
        __syncthreads();
        int c = cg;
        if (c0 == 0) {
#pragma unroll
            for (int i = 0; i < kCombineAhead; ++i, c += 4)
                if (c < nc) o = __builtin_fmaf(pv[i], fw[c], o);
        }
#pragma unroll 8
        for (; c < nc; c += 4) o = __builtin_fmaf(src[(int64_t)(c0 + c) * kPartStride + d], fw[c], o);
        if (tid == 0)
            for (int k = 0; k < nc; ++k) L = __builtin_fmaf(lw[k], fw[k], L);
    }
    og[cg][d] = o;
    __syncthreads();
    if (tid == 0) wmax[0] = L;
    __syncthreads();
    if (cg == 0) {
        const float t = (((og[0][d] + og[1][d]) + og[2][d]) + og[3][d]) * (1.0f / wmax[0]);
        if (p.v8c) {
            fw[d] = t;                                      // rotated back below
        } else {
            const float u = __shfl_xor(t, 1, 64);           // pairs of channels -> one BF16x2 store
            if ((d & 1) == 0) {
                uint32_t *dst = reinterpret_cast<uint32_t *>(p.o + ((int64_t)b * p.Hq + h) * 256 + d);
                *dst = pack_bf16x2(t, u);
            }
        }
    }
    if (p.v8c) {
        // INT8 V holds rotated rows: the normalized transform (its own
        // inverse) of the combined output gives the output, one wave
        __syncthreads();
        if (wave == 0) {
            float u[4] = {fw[4 * lane], fw[4 * lane + 1], fw[4 * lane + 2], fw[4 * lane + 3]};
            wht256(u, lane);
            *reinterpret_cast<uint2 *>(p.o + ((int64_t)b * p.Hq + h) * 256 + 4 * lane) =
                make_uint2(pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]));
        }
    }
}

}  // namespace
}  // namespace sage

hipError_t sage_launch_kv_append(const sage::KvAppendParams &p, hipStream_t s) {
    const unsigned items = (unsigned)p.nblk * (unsigned)p.Hkv;
    sage::kv_append_kernel<<<dim3((items + 3) / 4, p.B), 256, 0, s>>>(p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation-free decode: the chunk partials of one step live in a fixed
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy (kDecodeScratchBytes) until the process ends; every call
// on that GPU overwrites the partials it reads, so nothing needs clearing, and
// calls that overlap on one GPU race on the array.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[sage::kDecodeScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t sage_decode_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // the device address of this GPU's copy; the array's name on the host
        // is only a stand-in and is never passed to a kernel
        void *a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!a) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = a;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t sage_launch_decode(const sage::DecodeParams &p, hipStream_t s) {
    if (p.grp < 1 || p.grp > sage::kDecodeMaxGroup) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(p.nchunk * p.Hkv), p.B);
    if (p.v8c) sage::decode_chunk_kernel<true><<<grid, 256, 0, s>>>(p);
    else sage::decode_chunk_kernel<false><<<grid, 256, 0, s>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    sage::decode_combine_kernel<<<dim3(p.Hq, p.B), sage::kCombineThreads, 0, s>>>(p);
    return hipGetLastError();
}
