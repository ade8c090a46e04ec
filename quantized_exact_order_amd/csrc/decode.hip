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
// Decode reads the cache once: the work-group of (b, KV head, chunk of 256
// tokens) serves all Hq/Hkv query heads of that KV head.  Four lanes score one
// token (a quarter of D each, FP32 FMAs against the rotated queries read from
// LDS), so each K load instruction covers 16 rows in 64-byte runs; the
// chunk's softmax partial (max, sum, o) goes to a workspace, and a second
// kernel combines the chunks.

#include "decode.h"

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
#pragma unroll
    for (int lm = 1; lm < 64; lm <<= 1) {
        const bool upper = (lane & lm) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float other = shfl_xor_f(u[i], lm);
            u[i] = upper ? (other - u[i]) : (u[i] + other);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = u[i] * 0.0625f;
}

__device__ __forceinline__ void load4(const uint16_t *row, int lane, float x[4]) {
    const uint2 r = *reinterpret_cast<const uint2 *>(row + 4 * lane);
    x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x);
    x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
}

// One wave per appended row (b, t, h): 4 rows per 256-thread block.
// Grid (ceil(n * Hkv / 4), B).
__global__ __launch_bounds__(256) void kv_append_kernel(const KvAppendParams p) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.n * p.Hkv) return;
    const int t = row / p.Hkv, h = row % p.Hkv, b = blockIdx.y;
    const int64_t c = ((int64_t)b * p.Hkv + h) * p.cap + p.t0 + t;     // cache row

    float u[4];
    load4(p.k.ptr + (int64_t)b * p.k.sb + (int64_t)t * p.k.sn + (int64_t)h * p.k.sh, lane, u);
    wht256(u, lane);
    float m = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(u[0]), __builtin_fabsf(u[1])),
                              __builtin_fmaxf(__builtin_fabsf(u[2]), __builtin_fabsf(u[3])));
    m = wave_max_f(m);
    const float amax = (m > 1e-7f) ? m : 1e-7f;
    const float mul = 127.0f / amax;
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= (uint32_t)(to_i8(u[i] * mul) & 0xff) << (8 * i);
    reinterpret_cast<uint32_t *>(p.k8 + c * 256)[lane] = w;
    if (lane == 0) p.k_scale[c] = amax / 127.0f;

    const uint2 v = *reinterpret_cast<const uint2 *>(p.v.ptr + (int64_t)b * p.v.sb + (int64_t)t * p.v.sn +
                                                    (int64_t)h * p.v.sh + 4 * lane);
    reinterpret_cast<uint2 *>(p.vc + c * 256)[lane] = v;
}

// Chunk partial of GRP query heads.  Grid (nchunk * Hkv, B), 256 threads.
template <int GRP>
__global__ __launch_bounds__(256) void decode_chunk_kernel(const DecodeParams p) {
    __shared__ float qr[GRP][256];                 // rotated queries
    __shared__ float pw[GRP][kDecodeChunk];        // exp(s - chunk max)
    __shared__ float red[4][GRP];                  // per-wave maxima, then sums
    __shared__ float osum[GRP][256];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hk = blockIdx.x % p.Hkv, chunk = blockIdx.x / p.Hkv, b = blockIdx.y;
    const int64_t cbase = ((int64_t)b * p.Hkv + hk) * p.cap;

    for (int g = wave; g < GRP; g += 4) {
        float x[4];
        const int h = hk * GRP + g;
        load4(p.q.ptr + (int64_t)b * p.q.sb + (int64_t)h * p.q.sh, lane, x);
        wht256(x, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) qr[g][4 * lane + i] = x[i];
    }
    __syncthreads();

    // scores: four lanes per token (lane = 4 tk + qd), lane qd taking the
    // 16-byte pieces qd, qd + 4, ... of the row, 16 tokens of the wave per
    // pass; the four partial sums meet by two lane exchanges and the scores go
    // to pw (one entry per token)
    const int tl = wave * 64 + lane;                // token within the chunk (softmax, PV)
    const int t = chunk * kDecodeChunk + tl;
    const bool valid = t < p.T;
    {
        const int tk = lane >> 2, qd = lane & 3;
        for (int pass = 0; pass < 4; ++pass) {
            const int tc = wave * 64 + pass * 16 + tk;
            const int tt = chunk * kDecodeChunk + tc;
            float part[GRP];
#pragma unroll
            for (int g = 0; g < GRP; ++g) part[g] = 0.0f;
            if (tt < p.T) {
                const int8_t *kr = p.k8 + (cbase + tt) * 256 + 16 * qd;
#pragma unroll
                for (int d0 = 0; d0 < 256; d0 += 64) {        // the token's 4 lanes read 64 contiguous bytes
                    const int4 kk = *reinterpret_cast<const int4 *>(kr + d0);
                    const int w4[4] = {kk.x, kk.y, kk.z, kk.w};
                    float kf[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) kf[i] = (float)(int8_t)(w4[i >> 2] >> (8 * (i & 3)));
#pragma unroll
                    for (int g = 0; g < GRP; ++g) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) part[g] = __builtin_fmaf(qr[g][d0 + 16 * qd + i], kf[i], part[g]);
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < GRP; ++g) {
                part[g] = part[g] + shfl_xor_f(part[g], 1);
                part[g] = part[g] + shfl_xor_f(part[g], 2);
            }
            if (qd == 0 && tt < p.T) {
                const float sc = p.k_scale[cbase + tt] * 0.0625f;
#pragma unroll
                for (int g = 0; g < GRP; ++g) pw[g][tc] = part[g] * sc;
            }
        }
    }
    __syncthreads();
    float s[GRP];
#pragma unroll
    for (int g = 0; g < GRP; ++g) s[g] = valid ? pw[g][tl] : 0.0f;
    __syncthreads();

    // chunk softmax: maxima over the wave, then over the 4 waves
#pragma unroll
    for (int g = 0; g < GRP; ++g) {
        const float mw = wave_max_f(valid ? s[g] : -INFINITY);
        if (lane == 0) red[wave][g] = mw;
    }
    __syncthreads();
    float mx[GRP];
#pragma unroll
    for (int g = 0; g < GRP; ++g)
        mx[g] = __builtin_fmaxf(__builtin_fmaxf(red[0][g], red[1][g]), __builtin_fmaxf(red[2][g], red[3][g]));
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GRP; ++g) {
        const float e = valid ? expf(s[g] - mx[g]) : 0.0f;
        pw[g][tl] = e;
        float l = e;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) l = l + shfl_xor_f(l, m);
        if (lane == 0) red[wave][g] = l;
    }
    __syncthreads();

    // PV over the wave's 64 tokens: lane = 32 hf + dl takes the tokens of
    // parity hf and dimensions 8 dl .. 8 dl + 7 (16-byte V loads, two tokens
    // per instruction); the two parities are added at the end
    float o[GRP][8];
#pragma unroll
    for (int g = 0; g < GRP; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) o[g][i] = 0.0f;
    const int hf = lane >> 5, dl = lane & 31;
    const int tw = chunk * kDecodeChunk + wave * 64;
    const int nt = min(64, p.T - tw);
    for (int j = hf; j < nt; j += 2) {
        const uint4 r = *reinterpret_cast<const uint4 *>(p.vc + (cbase + tw + j) * 256 + 8 * dl);
        const float v[8] = {bf16_lo(r.x), bf16_hi(r.x), bf16_lo(r.y), bf16_hi(r.y),
                            bf16_lo(r.z), bf16_hi(r.z), bf16_lo(r.w), bf16_hi(r.w)};
#pragma unroll
        for (int g = 0; g < GRP; ++g) {
            const float e = pw[g][wave * 64 + j];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[g][i] = __builtin_fmaf(e, v[i], o[g][i]);
        }
    }
#pragma unroll
    for (int g = 0; g < GRP; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) o[g][i] = o[g][i] + shfl_xor_f(o[g][i], 32);
    // waves in order 0..3
    for (int w = 0; w < 4; ++w) {
        if (wave == w && hf == 0) {
#pragma unroll
            for (int g = 0; g < GRP; ++g)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    osum[g][8 * dl + i] = (w == 0) ? o[g][i] : osum[g][8 * dl + i] + o[g][i];
        }
        __syncthreads();
    }
    for (int g = wave; g < GRP; g += 4) {
        const int h = hk * GRP + g;
        float *dst = p.part + (((int64_t)b * p.Hq + h) * p.nchunk + chunk) * kPartStride;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[4 * lane + i] = osum[g][4 * lane + i];
        if (lane == 0) {
            dst[256] = mx[g];
            dst[257] = (red[0][g] + red[1][g]) + (red[2][g] + red[3][g]);
        }
    }
}

// Combines the chunk partials of one query head: M = max m_c,
// L = sum l_c e^(m_c - M), O = (sum o_c e^(m_c - M)) / L.  Wave w sums the
// chunks c = w, w + 4, ... in increasing order; the four wave sums are added
// in the order 0, 1, 2, 3 (a fixed order: the result is deterministic).
// Grid (Hq, B), 256 threads.
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecodeParams p) {
    __shared__ float wm[4];
    __shared__ float wl[4];
    __shared__ float wo[4][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = blockIdx.x, b = blockIdx.y;
    const float *src = p.part + ((int64_t)b * p.Hq + h) * p.nchunk * kPartStride;
    float M = -INFINITY;
    for (int c = threadIdx.x; c < p.nchunk; c += 256) M = __builtin_fmaxf(M, src[c * kPartStride + 256]);
    M = wave_max_f(M);
    if (lane == 0) wm[wave] = M;
    __syncthreads();
    M = __builtin_fmaxf(__builtin_fmaxf(wm[0], wm[1]), __builtin_fmaxf(wm[2], wm[3]));
    float L = 0.0f, o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = wave; c < p.nchunk; c += 4) {
        const float *pc = src + c * kPartStride;
        const float4 x = *reinterpret_cast<const float4 *>(pc + 4 * lane);
        const float f = expf(pc[256] - M);
        L = __builtin_fmaf(pc[257], f, L);
        o[0] = __builtin_fmaf(x.x, f, o[0]);
        o[1] = __builtin_fmaf(x.y, f, o[1]);
        o[2] = __builtin_fmaf(x.z, f, o[2]);
        o[3] = __builtin_fmaf(x.w, f, o[3]);
    }
    if (lane == 0) wl[wave] = L;
#pragma unroll
    for (int i = 0; i < 4; ++i) wo[wave][4 * lane + i] = o[i];
    __syncthreads();
    if (wave == 0) {
        const float Lt = ((wl[0] + wl[1]) + wl[2]) + wl[3];
        const float r = 1.0f / Lt;
        float t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            t[i] = (((wo[0][4 * lane + i] + wo[1][4 * lane + i]) + wo[2][4 * lane + i]) + wo[3][4 * lane + i]) * r;
        uint16_t *dst = p.o + ((int64_t)b * p.Hq + h) * 256 + 4 * lane;
        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3]));
    }
}

}  // namespace
}  // namespace sage

hipError_t sage_launch_kv_append(const sage::KvAppendParams &p, hipStream_t s) {
    const unsigned rows = (unsigned)p.n * (unsigned)p.Hkv;
    sage::kv_append_kernel<<<dim3((rows + 3) / 4, p.B), 256, 0, s>>>(p);
    return hipGetLastError();
}

hipError_t sage_launch_decode(const sage::DecodeParams &p, hipStream_t s) {
    const dim3 grid((unsigned)(p.nchunk * p.Hkv), p.B);
    switch (p.grp) {
    case 1: sage::decode_chunk_kernel<1><<<grid, 256, 0, s>>>(p); break;
    case 2: sage::decode_chunk_kernel<2><<<grid, 256, 0, s>>>(p); break;
    case 4: sage::decode_chunk_kernel<4><<<grid, 256, 0, s>>>(p); break;
    case 8: sage::decode_chunk_kernel<8><<<grid, 256, 0, s>>>(p); break;
    case 16: sage::decode_chunk_kernel<16><<<grid, 256, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    sage::decode_combine_kernel<<<dim3(p.Hq, p.B), 256, 0, s>>>(p);
    return hipGetLastError();
}
