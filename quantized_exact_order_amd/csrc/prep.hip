// prep.hip -- preparation kernels for gfx950: per-head RMSNorm and split-half
// RoPE of Q and K, the global K mean, INT8 quantization of Q and mean-smoothed
// K, and the per-channel FP8 (OCP E4M3) cast of V.
//
// Follows the page "Exact Numerical Contract", sections "Preparation",
// "Q And K Quantization" and "V And PV".  Every output of these kernels is a
// bit-exact target, so every rounding below is fixed:
//   * RMSNorm: sum of squares as a balanced pairwise tree over d in natural
//     order (8 elements per lane, then xor-butterflies over the lanes of the
//     row, which is the same tree), inv = 1/sqrt(ss/D + eps) with IEEE
//     division and square root, y = bf16((x*inv)*w);
//   * RoPE: z_i = bf16(a*c - b*s), z_{i+R/2} = bf16(b*c + a*s) on BF16 y and
//     BF16 coefficients (products exact in FP32);
//   * K mean: pairwise tree over the sequence padded with +0 to
//     2^ceil(log2 N) leaves: an in-tile tree over 64 rows here (cut short for
//     a sequence of one tile), a tree over tiles in prep_reduce_kernel;
//   * quantization: amax = max(1e-7, max|u|), scale = amax/127,
//     q = rni_sat(u * (127/amax)); V: v_scale = amax/2.25,
//     v8 = e4m3_rn_satfinite(v * (2.25/amax)).
// The file is built with -ffp-contract=off: no multiply-add is fused.
//
// Two passes over the rows: prep_stats_kernel (K tile sums, V tile maxima)
// and prep_reduce_kernel, then quant_kernel, one launch for the quantization
// of Q, K and V.  Each kernel streams its rows once with 16-byte loads (one
// row of D BF16 values is D/8 lanes), keeps per-row work in registers and
// uses LDS only for the RoPE partner exchange, the 64-row column reductions
// and the V tile transpose.

#include <algorithm>

#include "device.h"
#include "lanes.h"

namespace sage {
namespace {

constexpr int kThreads = 256;

// Loads 8 consecutive BF16 values (16 bytes) of row (b, n, h) starting at
// element 8*j.  The load is unconditional (an invalid row reads row 0, which
// always exists), so the kernels can issue every row load of a work-group
// before using the first; no select depends on the loaded value, so the
// compiler keeps the load where it is written instead of moving it into a
// branch on the row's validity (a load issued in a branch makes every later
// wait for it a wait for all loads).  Each pass streams its rows once, far
// more bytes than the caches hold, so the load is nontemporal.
__device__ __forceinline__ uint4 load_row8(const View &v, int b, int n, int h, int j, bool valid) {
    const int nn = valid ? n : 0;
    const uint16_t *p = v.ptr + (int64_t)b * v.sb + (int64_t)nn * v.sn + (int64_t)h * v.sh + 8 * j;
    const v4i x = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}

// x, or zeros when the row is invalid: an AND with a mask the compiler cannot
// see through (a select would make it move the row's load into a branch),
// applied where the row is used, so that it waits for the load there.
__device__ __forceinline__ uint4 zero_unless(uint4 x, bool valid) {
    uint32_t m = valid ? 0xffffffffu : 0u;
    asm("" : "+v"(m));
    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
}

__device__ __forceinline__ void unpack8(uint4 r, float x[8]) {
    x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x);
    x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
    x[4] = bf16_lo(r.z); x[5] = bf16_hi(r.z);
    x[6] = bf16_lo(r.w); x[7] = bf16_hi(r.w);
}

__device__ __forceinline__ uint4 pack8(const float y[8]) {
    return make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                      pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
}

// Row 0, elements [8j, 8j+8), of head h of batch b: a readable 16-byte
// aligned address for loads whose value is not used.
__device__ __forceinline__ const uint16_t *row0_8(const View &v, int b, int h, int j) {
    return v.ptr + (int64_t)b * v.sb + (int64_t)h * v.sh + 8 * j;
}

// RMSNorm weights of elements [8j, 8j+8), as their BF16 pairs (BF16 ones,
// 0x3F80, when w is NULL), loaded once per kernel; unpack8 makes them FP32.
// Kept packed until first use, so that issuing the load does not wait for it;
// the load is issued in either case (from `any`, a readable address, when w
// is NULL) and the ones are merged in with a mask the compiler cannot see
// through, which keeps the load out of a branch.
__device__ __forceinline__ uint4 load_w8(const uint16_t *w, int j, const uint16_t *any) {
    const uint4 x = *reinterpret_cast<const uint4 *>(w ? w + 8 * j : any);
    uint32_t m = w ? 0xffffffffu : 0u;
    asm("" : "+v"(m));
    const uint32_t one = 0x3F803F80u & ~m;
    return make_uint4((x.x & m) | one, (x.y & m) | one, (x.z & m) | one, (x.w & m) | one);
}

// RoPE coefficients for elements [8j, 8j+8) at position n when R/2 is a
// multiple of 8, so that 8-element blocks pair up whole: 16 bytes of cos and
// of sin at the pair's lower block (lanes past R read block 0 and do not use
// it).
struct Coef8 {
    uint4 c, s;
};

// The two loads are issued whatever R is, from `any` (a readable 16-byte
// aligned address) when the block form does not apply: a load in a branch
// would make the compiler's later waits count conservatively.  The values are
// then meaningless, and rope8 does not read them.
__device__ __forceinline__ Coef8 rope_coef8(const uint16_t *cos_t, const uint16_t *sin_t, int n, int j, int R,
                                            const uint16_t *any) {
    const int half = R >> 1, d0 = 8 * j;
    const bool use = R > 0 && (half & 7) == 0;
    const int64_t off = (int64_t)n * half + (d0 < half ? d0 : (d0 < R ? d0 - half : 0));
    const uint16_t *pc = use ? cos_t + off : any;
    const uint16_t *ps = use ? sin_t + off : any;
    return Coef8{*reinterpret_cast<const uint4 *>(pc), *reinterpret_cast<const uint4 *>(ps)};
}

// RMSNorm of one row held by L consecutive lanes (8 elements each).  Every
// lane of the wave must call this (lane exchanges).  Result rounded to BF16
// and packed (one RNE conversion per element).
template <int L>
__device__ __forceinline__ uint4 rmsnorm8(const float x[8], const float wv[8], float eps, int D) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = x[i] * x[i];
    float a0 = t[0] + t[1], a1 = t[2] + t[3], a2 = t[4] + t[5], a3 = t[6] + t[7];
    float b0 = a0 + a1, b1 = a2 + a3;
    float ss = b0 + b1;
    for_pow2<1, L>([&](auto m) { ss = ss + xor_lane<decltype(m)::value>(ss); });
    float inv = 1.0f / sqrtf(ss / (float)D + eps);
    float n2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float n1 = x[i] * inv;
        n2[i] = n1 * wv[i];
    }
    return pack8(n2);
}

// Split-half RoPE of the 8 elements [8j, 8j+8) of row `r` whose normalized
// values (BF16) sit in LDS row `yrow`; n is the position and k its
// coefficients from rope_coef8 (used when R/2 is a multiple of 8; other
// widths load per element).
__device__ __forceinline__ void rope8(const uint16_t *yrow, int j, int n, int R, const uint16_t *cos_t,
                                      const uint16_t *sin_t, const Coef8 &k, float z[8]) {
    const int half = R >> 1;
    const int d0 = 8 * j;
    float y[8];
    unpack8(*reinterpret_cast<const uint4 *>(yrow + d0), y);
    if (d0 >= R) {
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = y[i];
        return;
    }
    if ((half & 7) == 0) {
        // whole 8-element blocks pair up: block j with block j +- half/8
        const bool lower = d0 < half;
        const int pd = lower ? d0 + half : d0 - half;     // partner block start
        // a*c - b*s (lower) and b*c + a*s (upper) are both y*c + partner*s'
        // with s' = -s for the lower half: the products are exact, so
        // negating s before the single rounding of the sum changes nothing
        float pv[8], c[8], s[8], r[8];
        unpack8(*reinterpret_cast<const uint4 *>(yrow + pd), pv);
        unpack8(k.c, c);
        uint4 sw = k.s;
        const uint32_t flip = lower ? 0x80008000u : 0u;
        sw.x ^= flip; sw.y ^= flip; sw.z ^= flip; sw.w ^= flip;
        unpack8(sw, s);
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = y[i] * c[i] + pv[i] * s[i];
        unpack8(pack8(r), z);                            // round to BF16 (RNE), as FP32
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int d = d0 + i;
        float r;
        if (d < half) {
            float a = y[i], b = __uint_as_float((uint32_t)yrow[d + half] << 16);
            float c = __uint_as_float((uint32_t)cos_t[(int64_t)n * half + d] << 16);
            float s = __uint_as_float((uint32_t)sin_t[(int64_t)n * half + d] << 16);
            r = round_bf16(a * c - b * s);
        } else if (d < R) {
            float b = y[i], a = __uint_as_float((uint32_t)yrow[d - half] << 16);
            float c = __uint_as_float((uint32_t)cos_t[(int64_t)n * half + d - half] << 16);
            float s = __uint_as_float((uint32_t)sin_t[(int64_t)n * half + d - half] << 16);
            r = round_bf16(b * c + a * s);
        } else {
            r = y[i];
        }
        z[i] = r;
    }
}

// Normalized Walsh-Hadamard transform of a row held by L lanes (8 consecutive
// elements each), in place, FP32.  Butterfly spans 1, 2, 4 inside the lane,
// then 8 .. 4L across lanes; pair (a at i, b at i+span) -> (a+b, a-b); finally
// times 1/sqrt(8L) (1/16 for the supported 256-wide rows, exact).
template <int L>
__device__ __forceinline__ void wht8(float u[8], int j) {
#pragma unroll
    for (int span = 1; span < 8; span <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if ((i & span) == 0) {
                float a = u[i], b = u[i + span];
                u[i] = a + b;
                u[i + span] = a - b;
            }
        }
    }
    for_pow2<1, L>([&](auto m) {
        constexpr int lm = decltype(m)::value;
        const bool upper = (j & lm) != 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float other = xor_lane<lm>(u[i]);
            u[i] = upper ? (other - u[i]) : (u[i] + other);
        }
    });
    const float s = (L == 32) ? 0.0625f : 1.0f / sqrtf((float)(8 * L));
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = u[i] * s;
}

// ---------------------------------------------------------------------------
// Pass 1: K rows -> per-tile column sums (pairwise over 64 rows); V rows ->
// per-tile column maxima of |v|.  Grid (nk * Hkv, B), x = tile * Hkv + head,
// 256 threads.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void prep_stats_kernel(const PrepParams p) {
    constexpr int L = D / 8;               // lanes per row
    constexpr int RPP = kThreads / L;      // rows per pass
    constexpr int NPASS = 64 / RPP;
    __shared__ __attribute__((aligned(16))) uint16_t ybuf[64 * D];
    __shared__ __attribute__((aligned(16))) uint16_t zbuf[64 * D];
    // V partial maxima reuse ybuf once the RoPE pass has consumed it
    float *vpart = reinterpret_cast<float *>(ybuf);
    static_assert(RPP * D * sizeof(float) <= sizeof(ybuf), "vpart must fit in ybuf");

    const int h = blockIdx.x % p.Hkv, t = blockIdx.x / p.Hkv, b = blockIdx.y;
    const int tid = threadIdx.x, j = tid % L, rr = tid / L;

    // every global load of the work-group first, none of them in a branch
    // (that would make the compiler's waits count conservatively), in the
    // order of first use: RMSNorm weights, RoPE coefficients, K rows, V rows
    // (vmcnt counts in order: waiting for a K row never waits for V)
    const uint16_t *any = row0_8(p.k, b, h, j);
    const uint4 wraw = load_w8(p.w_k, j, any);
    uint4 kraw[NPASS], vraw[NPASS];
    Coef8 cf[NPASS];
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int n = t * 64 + pass * RPP + rr;
        cf[pass] = rope_coef8(p.cos_t, p.sin_t, n < p.N ? n : 0, j, p.R, any);
    }
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int n = t * 64 + pass * RPP + rr;
        kraw[pass] = load_row8(p.k, b, n, h, j, n < p.N);     // rows >= N are zeroed after RoPE
    }
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int n = t * 64 + pass * RPP + rr;
        vraw[pass] = load_row8(p.v, b, n, h, j, n < p.N);
    }
    // (the compiler's scheduler would otherwise interleave the first passes'
    // arithmetic with the loads, and their waits with the issue of the rest)
    __builtin_amdgcn_sched_barrier(0);
    float wv[8];
    unpack8(wraw, wv);
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int r = pass * RPP + rr;
        float x[8];
        unpack8(kraw[pass], x);
        *reinterpret_cast<uint4 *>(&ybuf[r * D + 8 * j]) = rmsnorm8<L>(x, wv, p.eps, D);
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int r = pass * RPP + rr, n = t * 64 + r;
        float z[8];
        rope8(&ybuf[r * D], j, n < p.N ? n : 0, p.R, p.cos_t, p.sin_t, cf[pass], z);
        if (n >= p.N) {
#pragma unroll
            for (int i = 0; i < 8; ++i) z[i] = 0.0f;       // padding leaves are +0
        }
        *reinterpret_cast<uint4 *>(&zbuf[r * D + 8 * j]) = pack8(z);
    }
    // V: running max |v| of this thread's 8 channels over its rows
    float vm[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vm[i] = 0.0f;
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        float x[8];
        const int n = t * 64 + pass * RPP + rr;
        unpack8(zero_unless(vraw[pass], n < p.N), x);     // invalid rows are zeros
#pragma unroll
        for (int i = 0; i < 8; ++i) vm[i] = __builtin_fmaxf(vm[i], __builtin_fabsf(x[i]));
    }
    __syncthreads();                       // every RoPE read of ybuf is done
#pragma unroll
    for (int i = 0; i < 8; ++i) vpart[rr * D + 8 * j + i] = vm[i];
    __syncthreads();

    const int64_t wsoff = (((int64_t)b * p.Hkv + h) * p.nk + t) * D;
    // The tree has 2^ceil(log2 N) leaves: a sequence of one tile stops after
    // log2 of that many levels (the value then at v[0] is the whole sum, the
    // rest of the 64-leaf tree would only add +0 leaves to it).
    int stop = 1;
    if (p.nk == 1)
        while (64 / stop > 1 && 64 / stop >= 2 * p.N) stop *= 2;
    for (int d = tid; d < D; d += kThreads) {
        float v[64];
#pragma unroll
        for (int r = 0; r < 64; ++r) v[r] = __uint_as_float((uint32_t)zbuf[r * D + d] << 16);
#pragma unroll
        for (int w = 64; w > 1; w >>= 1) {
            if (w > stop) {
#pragma unroll
                for (int i = 0; i < w / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
            }
        }
        p.ws_ksum[wsoff + d] = v[0];
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < RPP; ++r) m = __builtin_fmaxf(m, vpart[r * D + d]);
        p.ws_vmax[wsoff + d] = m;
    }
}

// ---------------------------------------------------------------------------
// Pass 1b: per (b, h, d) the pairwise tree over the tile sums (padded with +0
// to P = a power of two), mean = S/N; V channel maximum over tiles, floored at
// 1e-7, and v_scale = amax/2.25.  Grid (B*Hkv, D/32), 32 G threads: a block
// owns 32 columns, thread group g (G of them) the chunks g, g+G, ... of C
// consecutive tiles.  The tree over P leaves is the tree over the P/C aligned
// chunk subtrees, so each thread builds whole chunk subtrees and the block
// finishes the tree over the (at most 64) chunk sums level by level in LDS.
// The kernel is latency-bound (34 MB at the canonical size), so the host
// gives a block one thread group per chunk (G = NC, within 2..32) and each
// chunk's loads are issued together.
// ---------------------------------------------------------------------------
constexpr int kRedCols = 32;
constexpr int kRedMaxGroups = 32;

// Leaves P (nk rounded up to a power of two), tiles per chunk C and chunks NC
// of the tree over nk tile sums; the same on the host and in the kernel.
struct RedShape {
    int P, C, NC;
};
__host__ __device__ inline RedShape red_shape(int nk) {
    int P = 1;
    while (P < nk) P <<= 1;
    const int C = (P <= 1024) ? (P < 16 ? P : 16) : P / 64;
    return RedShape{P, C, P / C};
}

// Pairwise tree over the C leaves (C a power of two, at most 16) of tiles
// t0 .. t0+C-1; tiles >= nk are +0.  The loads are unconditional (a leaf past
// the column reads tile 0, which always exists), so all of them are in flight
// before the first add.
__device__ __forceinline__ float chunk_tree16(const float *col, int D, int t0, int C, int nk) {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const bool in = k < C && t0 + k < nk;
        const float x = col[(int64_t)(in ? t0 + k : 0) * D];
        v[k] = in ? x : 0.0f;
    }
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1) {
        if (w < C) {
#pragma unroll
            for (int k = 0; k < w; ++k) v[k] = v[2 * k] + v[2 * k + 1];
        }
    }
    return v[0];
}

// Maximum of the column over tiles t0 .. min(t0 + C, nk) - 1 (C at most 16),
// starting from m; every load is issued before the first maximum.
__device__ __forceinline__ float chunk_max16(const float *col, int D, int t0, int C, int nk, float m) {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const bool in = k < C && t0 + k < nk;
        const float x = col[(int64_t)(in ? t0 + k : 0) * D];     // tile 0 always exists
        v[k] = in ? x : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) m = __builtin_fmaxf(m, v[k]);
    return m;
}

// The same tree for any power of two C: the binary-counter evaluation (after
// leaf i, ctz(i+1) merges of left + right) over 16-leaf subtrees.
__device__ float chunk_tree(const float *col, int D, int t0, int C, int nk) {
    if (C <= 16) return chunk_tree16(col, D, t0, C, nk);
    float stack[32];
    int top = 0;
    const int n16 = C / 16;
    for (int i = 0; i < n16; ++i) {
        float x = chunk_tree16(col, D, t0 + 16 * i, 16, nk);
        for (int m = __builtin_ctz((unsigned)(i + 1)); m > 0; --m) x = stack[--top] + x;
        stack[top++] = x;
    }
    return stack[0];
}

__global__ __launch_bounds__(kRedCols * kRedMaxGroups) void prep_reduce_kernel(const PrepParams p) {
    __shared__ float tree[2][64][kRedCols + 1];
    __shared__ float vmx[kRedMaxGroups][kRedCols];
    const int bh = blockIdx.x, D = p.D, nk = p.nk;
    const int G = blockDim.x / kRedCols;                      // thread groups
    const int c = threadIdx.x % kRedCols, g = threadIdx.x / kRedCols;
    const int d = blockIdx.y * kRedCols + c;
    const float *ks = p.ws_ksum + (int64_t)bh * nk * D + d;
    const float *vm = p.ws_vmax + (int64_t)bh * nk * D + d;
    const RedShape rs = red_shape(nk);
    const int C = rs.C, NC = rs.NC;                           // tiles per chunk, chunks (<= 64)
    float m = 0.0f;
    for (int j = g; j < NC; j += G) {
        tree[0][j][c] = chunk_tree(ks, D, j * C, C, nk);
        for (int t = j * C; t < (j + 1) * C && t < nk; t += 16) m = chunk_max16(vm, D, t, min(16, (j + 1) * C - t), nk, m);
    }
    vmx[g][c] = m;
    __syncthreads();
    int src = 0;
    for (int w = NC / 2; w >= 1; w >>= 1) {           // one tree level: left + right
        for (int j = g; j < w; j += G) tree[src ^ 1][j][c] = tree[src][2 * j][c] + tree[src][2 * j + 1][c];
        src ^= 1;
        __syncthreads();
    }
    if (g == 0) {
        p.k_mean[(int64_t)bh * D + d] = tree[src][0][c] / (float)p.N;
        for (int i = 1; i < G; ++i) m = __builtin_fmaxf(m, vmx[i][c]);
        const float amax = (m > 1e-7f) ? m : 1e-7f;
        p.v_scale[(int64_t)bh * D + d] = amax / 2.25f;
        p.ws_vamax[(int64_t)bh * D + d] = amax;
    }
}

// ---------------------------------------------------------------------------
// Pass 2a: Q -> INT8, one scale per 32 rows.  Work-group x of batch b
// (x < q_rows/128 * Hq): x = (row block) * Hq + head; wave w of row block r
// owns group g = 4r + w (rows [32g, 32g+32)).  LDS: kQLds(D) bytes.
// ---------------------------------------------------------------------------
constexpr int kQLds(int D) { return 4 * 32 * D * 2; }

template <int D>
__device__ __forceinline__ void quant_q_tile(const PrepParams &p, int x, int b, uint8_t *lds) {
    constexpr int L = D / 8;
    constexpr int RPW = 64 / L;            // rows per wave pass
    constexpr int NP = 32 / RPW;

    const int h = x % p.Hq;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane % L, rr = lane / L;
    const int g = (x / p.Hq) * 4 + wave;
    uint16_t *yb = reinterpret_cast<uint16_t *>(lds) + wave * 32 * D;

    // every row load of the wave first; the RoPE coefficients with them when
    // there are at most 4 passes, else in groups of CG = 4 passes, each
    // group's loads issued together ahead of its passes (a load per pass,
    // next to a store that may alias it, would cost a round trip per pass).
    // Loading all 8 groups of D = 128 up front takes 136 VGPRs, which leaves
    // the launch shared with the K/V work-groups at 3 work-groups per CU
    // instead of 4, and measured 5% slower.
    constexpr bool PRE = NP <= 4;
    constexpr int CG = PRE ? NP : 4;
    // (the RMSNorm weights, and the coefficients when loaded up front, before
    // the rows, in the order of first use, none in a branch)
    const uint16_t *any = row0_8(p.q, b, h, j);
    const uint4 wraw = load_w8(p.w_q, j, any);
    uint4 qraw[NP];
    Coef8 cf[CG];
    if constexpr (PRE) {
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
            const int n = 32 * g + pass * RPW + rr;
            cf[pass] = rope_coef8(p.cos_t, p.sin_t, n < p.N ? n : 0, j, p.R, any);
        }
    }
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const int n = 32 * g + pass * RPW + rr;
        qraw[pass] = load_row8(p.q, b, n, h, j, n < p.N);   // rows >= N are masked below
    }
    // (the compiler's scheduler would otherwise interleave the first passes'
    // arithmetic with the loads, and their waits with the issue of the rest)
    __builtin_amdgcn_sched_barrier(0);
    float wv[8];
    unpack8(wraw, wv);
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const int r = pass * RPW + rr;
        float x[8];
        unpack8(qraw[pass], x);
        *reinterpret_cast<uint4 *>(&yb[r * D + 8 * j]) = rmsnorm8<L>(x, wv, p.eps, D);
    }
    __syncthreads();
    float u[NP][8];
    float amax = 0.0f;
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const int r = pass * RPW + rr, n = 32 * g + r;
        const int nc = n < p.N ? n : 0;
        if constexpr (!PRE) {
            if (pass % CG == 0) {
#pragma unroll
                for (int i = 0; i < CG; ++i) {
                    const int ni = 32 * g + (pass + i) * RPW + rr;
                    cf[i] = rope_coef8(p.cos_t, p.sin_t, ni < p.N ? ni : 0, j, p.R, any);
                }
            }
        }
        const Coef8 k = cf[pass % CG];
        rope8(&yb[r * D], j, nc, p.R, p.cos_t, p.sin_t, k, u[pass]);
        if (p.q_prep && n < p.N)
            *reinterpret_cast<uint4 *>(p.q_prep + (((int64_t)b * p.Hq + h) * p.N + n) * D + 8 * j) = pack8(u[pass]);
        if (p.hadamard) wht8<L>(u[pass], j);
        if (n < p.N) {
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(u[pass][i]));
        }
    }
    amax = wave_max_x(amax);
    amax = (amax > 1e-7f) ? amax : 1e-7f;
    const float scale = amax / 127.0f;
    const float mul = 127.0f / amax;
    int8_t *dst = p.q8 + (((int64_t)b * p.Hq + h) * p.q_rows + 32 * g) * D;
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const int r = pass * RPW + rr, n = 32 * g + r;
        uint32_t lo = 0, hi = 0;
        if (n < p.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) lo |= (uint32_t)(to_i8(u[pass][i] * mul) & 0xff) << (8 * i);
#pragma unroll
            for (int i = 0; i < 4; ++i) hi |= (uint32_t)(to_i8(u[pass][4 + i] * mul) & 0xff) << (8 * i);
        }
        *reinterpret_cast<uint2 *>(dst + (int64_t)r * D + 8 * j) = make_uint2(lo, hi);
    }
    if (lane == 0 && g < p.nq) p.q_scale[((int64_t)b * p.Hq + h) * p.nq + g] = scale;
}

// ---------------------------------------------------------------------------
// Pass 2b: one 64-row tile of K and of V per work-group.  Work-group x of
// batch b (x < nk * Hkv): x = tile * Hkv + head.  LDS: kKVLds(D) bytes.
//   K -> subtract k_mean -> INT8, one scale per tile;
//   V -> E4M3 into tiles [D][64], keys of a tile in the slot order of
//        sage_v8_slot_key (the key order in which the attention kernel holds
//        its probabilities), one scale per channel (from pass 1).
// The two share a work-group so that the V rows, which need no arithmetic
// before their conversion, stream in while the K rows are normalized and
// rotated.
// ---------------------------------------------------------------------------
constexpr int kKVLds(int D) { return 2 * 64 * D * 2 + 16 * (kThreads / 64); }

template <int D>
__device__ __forceinline__ void quant_kv_tile(const PrepParams &p, int x, int b, uint8_t *lds) {
    constexpr int L = D / 8;
    constexpr int RPP = kThreads / L;
    constexpr int NPASS = 64 / RPP;
    constexpr int NE = 2 * D / kThreads;      // V conversion items per thread
    static_assert(NE * kThreads == 2 * D, "whole conversion items per thread");
    uint16_t *ybuf = reinterpret_cast<uint16_t *>(lds);
    uint16_t *vbuf = ybuf + 64 * D;
    float *wmax = reinterpret_cast<float *>(vbuf + 64 * D);

    const int h = x % p.Hkv, t = x / p.Hkv;
    const int tid = threadIdx.x, j = tid % L, rr = tid / L;

    // every global load of the work-group first, none of them in a branch,
    // in the order of first use: RMSNorm weights, RoPE coefficients, K rows,
    // the K mean, V rows, the V channel maxima (vmcnt counts in order:
    // waiting for a K row never waits for V)
    const uint16_t *any = row0_8(p.k, b, h, j);
    const uint4 wraw = load_w8(p.w_k, j, any);
    uint4 kraw[NPASS], vraw[NPASS];
    Coef8 cf[NPASS];
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int n = t * 64 + pass * RPP + rr;
        cf[pass] = rope_coef8(p.cos_t, p.sin_t, n < p.N ? n : 0, j, p.R, any);
    }
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int n = t * 64 + pass * RPP + rr;
        kraw[pass] = load_row8(p.k, b, n, h, j, n < p.N);   // rows >= N are masked below
    }
    const float *mu = p.k_mean + ((int64_t)b * p.Hkv + h) * D + 8 * j;
    float mean[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) mean[i] = mu[i];
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int n = t * 64 + pass * RPP + rr;
        vraw[pass] = load_row8(p.v, b, n, h, j, n < p.N);
    }
    // thread: channel pair (2 dp, 2 dp + 1) and a quarter qr of the 64 slots
    // for each of its NE items e = tid + kThreads * i
    const float *vam = p.ws_vamax + ((int64_t)b * p.Hkv + h) * D;
    float2 am[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) am[i] = *reinterpret_cast<const float2 *>(vam + 2 * ((tid + kThreads * i) % (D / 2)));
    // (the compiler's scheduler would otherwise interleave the first passes'
    // arithmetic with the loads, and their waits with the issue of the rest)
    __builtin_amdgcn_sched_barrier(0);
    float wv[8];
    unpack8(wraw, wv);
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int r = pass * RPP + rr;
        float x[8];
        unpack8(kraw[pass], x);
        *reinterpret_cast<uint4 *>(&ybuf[r * D + 8 * j]) = rmsnorm8<L>(x, wv, p.eps, D);
    }
    // (the V rows go to LDS after the K passes: stored first, their waits
    // would be every load's)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int n = t * 64 + pass * RPP + rr;
        *reinterpret_cast<uint4 *>(&vbuf[(pass * RPP + rr) * D + 8 * j]) = zero_unless(vraw[pass], n < p.N);
    }
    __syncthreads();

    // K
    float u[NPASS][8];
    float amax = 0.0f;
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int r = pass * RPP + rr, n = t * 64 + r;
        float z[8];
        rope8(&ybuf[r * D], j, n < p.N ? n : 0, p.R, p.cos_t, p.sin_t, cf[pass], z);
        if (p.k_prep && n < p.N)
            *reinterpret_cast<uint4 *>(p.k_prep + (((int64_t)b * p.Hkv + h) * p.N + n) * D + 8 * j) = pack8(z);
#pragma unroll
        for (int i = 0; i < 8; ++i) u[pass][i] = z[i] - mean[i];
        if (p.hadamard) wht8<L>(u[pass], j);
        if (n < p.N) {
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(u[pass][i]));
        }
    }
    amax = wave_max_x(amax);
    if ((tid & 63) == 0) wmax[tid >> 6] = amax;
    __syncthreads();
    amax = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
    amax = (amax > 1e-7f) ? amax : 1e-7f;
    const float scale = amax / 127.0f;
    const float mul = 127.0f / amax;
    int8_t *dst = p.k8 + (((int64_t)b * p.Hkv + h) * p.k_rows + 64 * t) * D;
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int r = pass * RPP + rr, n = t * 64 + r;
        uint32_t lo = 0, hi = 0;
        if (n < p.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) lo |= (uint32_t)(to_i8(u[pass][i] * mul) & 0xff) << (8 * i);
#pragma unroll
            for (int i = 0; i < 4; ++i) hi |= (uint32_t)(to_i8(u[pass][4 + i] * mul) & 0xff) << (8 * i);
        }
        *reinterpret_cast<uint2 *>(dst + (int64_t)r * D + 8 * j) = make_uint2(lo, hi);
    }
    if (tid == 0) p.k_scale[((int64_t)b * p.Hkv + h) * p.nk + t] = scale;

    // V: for each slot, one 4-byte LDS read gives both channels of its key
    uint8_t *vdst = p.v8 + (((int64_t)b * p.Hkv + h) * p.nk + t) * (int64_t)D * 64;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int e = tid + kThreads * i;
        const int dp = e % (D / 2), qr = e / (D / 2);
        const int d = 2 * dp;
        const float mul0 = 2.25f / am[i].x, mul1 = 2.25f / am[i].y;
        uint32_t w0[4], w1[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float x0[4], x1[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int key = sage_v8_slot_key(16 * qr + 4 * k + q);
                const uint32_t pair = *reinterpret_cast<const uint32_t *>(&vbuf[key * D + d]);
                x0[q] = bf16_lo(pair) * mul0;
                x1[q] = bf16_hi(pair) * mul1;
            }
            w0[k] = pack4_e4m3_bounded(x0);
            w1[k] = pack4_e4m3_bounded(x1);
        }
        *reinterpret_cast<uint4 *>(vdst + (int64_t)d * 64 + 16 * qr) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
        *reinterpret_cast<uint4 *>(vdst + (int64_t)(d + 1) * 64 + 16 * qr) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
    }
}

// ---------------------------------------------------------------------------
// Pass 2 as one launch.  Grid (nq_wg + nkv_wg, B) with nq_wg = q_rows/128 * Hq
// Q work-groups and nkv_wg = nk * Hkv K/V work-groups, interleaved in runs of
// one Q and two K/V work-groups while both last (then the rest of either
// kind), so that the Q passes' arithmetic and the K/V streams share the CUs
// throughout the launch.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void quant_kernel(const PrepParams p, int nq_wg, int nkv_wg) {
    constexpr int kLds = kQLds(D) > kKVLds(D) ? kQLds(D) : kKVLds(D);
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
    const int i = blockIdx.x, b = blockIdx.y;
    const int u = min(nq_wg, nkv_wg / 2);     // runs of (Q, K/V, K/V)
    if (i < 3 * u) {
        const int run = i / 3, r = i - 3 * run;
        if (r == 0) quant_q_tile<D>(p, run, b, lds);
        else quant_kv_tile<D>(p, 2 * run + r - 1, b, lds);
    } else if (i < 3 * u + (nq_wg - u)) {
        quant_q_tile<D>(p, u + (i - 3 * u), b, lds);
    } else {
        quant_kv_tile<D>(p, 2 * u + (i - 3 * u - (nq_wg - u)), b, lds);
    }
}

}  // namespace
}  // namespace sage

using sage::PrepParams;

hipError_t sage_launch_prep_stats(const PrepParams &p, hipStream_t s) {
    // x = tile * H + head: concurrent work-groups read neighbouring heads of
    // the same rows, i.e. long contiguous runs of an interleaved QKV row
    const dim3 grid((unsigned)(p.nk * p.Hkv), p.B);
    if (p.D == 128) sage::prep_stats_kernel<128><<<grid, sage::kThreads, 0, s>>>(p);
    else sage::prep_stats_kernel<256><<<grid, sage::kThreads, 0, s>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int groups = std::min(sage::kRedMaxGroups, std::max(2, sage::red_shape(p.nk).NC));
    sage::prep_reduce_kernel<<<dim3(p.B * p.Hkv, p.D / sage::kRedCols), sage::kRedCols * groups, 0, s>>>(p);
    return hipGetLastError();
}

hipError_t sage_launch_quant(const PrepParams &p, hipStream_t s) {
    const int nq_wg = (int)(p.q_rows / 128 * p.Hq), nkv_wg = p.nk * p.Hkv;
    const dim3 grid((unsigned)(nq_wg + nkv_wg), p.B);
    if (p.D == 128) sage::quant_kernel<128><<<grid, sage::kThreads, 0, s>>>(p, nq_wg, nkv_wg);
    else sage::quant_kernel<256><<<grid, sage::kThreads, 0, s>>>(p, nq_wg, nkv_wg);
    return hipGetLastError();
}
