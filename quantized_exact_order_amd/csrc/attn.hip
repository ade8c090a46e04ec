// attn.hip -- fused quantized attention forward for gfx950 (CDNA4).
//
// Computes, per query row, the sequence of the page "Exact Numerical
// Contract", sections "INT8 QK And Score Domain", "Online Softmax", "V And PV"
// and "Finalization And Tails":
//   S    = q8 . k8 over D in INT32 (exact)             v_mfma_i32_32x32x32_i8
//   f    = (q_scale * c) * k_scale[t],  c = log2(e)/sqrt(D)
//   M    = float(max S) * f - 8.807;  m' = max(m, M);  alpha = 2^(m - m')
//   d    = d*alpha,  RO = RO*alpha   (RO rescale skipped when no row of the
//                                     wave moved; alpha is then exactly 1)
//   p    = 2^(fma(float(S), f, -m')),  d += p,  p8 = e4m3(p)
//   RO  += p8 . v8 (FP32 accumulate)                   v_mfma_f32_32x32x64_f8f6f4
//   O    = bf16((RO * (1/d)) * v_scale)
// with m0 = -5e6, d0 = 1, KV tiles of 64 keys visited in increasing order and
// one work-group owning a query tile for the whole sequence (no split over
// keys).  Keys >= N in the last tile get p = 0 (their score would be -5e6)
// and never win the maximum.
//
// Register layout: the score tile is computed transposed, S^T = K Q^T, so a
// lane holds 32 keys of ONE query row (column lane%32 of the accumulator;
// rows 8*(r/4) + 4*(lane/32) + r%4 of block c for register r).  Per-row state
// (m, d) is per lane, the row maximum needs one exchange between the two lane
// halves, and the packed FP8 probabilities of the lane are directly the B
// operand (P^T) of the PV MFMA.  The prep pass stores each V tile as [D][64]
// with the keys permuted into exactly that register order
// (sage_v8_slot_key), so the A operand (V^T) is a plain 32-byte LDS read.
// The contract page's own PV accumulates each tile in FP16 on its hardware;
// the gfx950 FP8 MFMA accumulates in FP32 directly into RO.
//
// INT32 -> FP32 without a conversion instruction: the QK accumulator starts at
// the bit pattern of 1.5 * 2^23 (0x4B400000).  Since |S| <= D * 127^2 < 2^22,
// the finished accumulator is the FP32 encoding of 12582912 + S, so
// float(S) = bits - 12582912.0f exactly (one subtraction), and the integer
// maximum of the biased values is the maximum of S.
//
// Schedule (PIPE, per wave, tile t): issue the QK MFMAs of tile t+1, then the
// softmax VALU work of tile t runs while they execute, then the PV MFMAs of
// tile t.  K is therefore staged in LDS one tile ahead of V (two K buffers,
// two V buffers, register-staged global loads issued a full tile ahead).
// Wide heads (D = 256) keep one tile of scores live instead (!PIPE) to stay
// within the register file.
// Work-groups are renumbered so that consecutive query tiles of a head run on
// the same XCD and share its L2.

#include "device.h"

namespace sage {
namespace {

constexpr int kBias = 0x4B400000;         // FP32 bits of 12582912 = 1.5 * 2^23
constexpr float kBiasF = 12582912.0f;

// LDS byte offset of 16-byte chunk `j` of K row `r` (row length D bytes).
// The XOR swizzle spreads the 16 lanes that read chunk j of rows r..r+15
// over distinct 16-byte bank groups, whether the LDS serves 8 lanes from 32
// banks or 16 lanes from 64 banks per cycle.
template <int D>
__device__ __forceinline__ int k_lds(int r, int j) {
    const int h = (D == 128) ? ((r & 7) ^ ((r >> 3) & 1)) : (r & 15);
    return r * D + 16 * (j ^ h);
}

// LDS byte offset of 16-byte chunk `j` (0..3) of V^T row `d` (64 bytes),
// swizzled the same way for rows d..d+15.
__device__ __forceinline__ int v_lds(int d, int j) {
    const int h = ((d >> 1) & 1) ^ (((d >> 2) & 1) << 1) ^ ((d >> 3) & 1);
    return d * 64 + 16 * (j ^ h);
}

__device__ __forceinline__ int imax3(int a, int b, int c) { return max(max(a, b), c); }

// S^T (biased) of one 64-key tile for the wave's 32 queries.
template <int D>
__device__ __forceinline__ void qk_tile(const uint8_t *kt, const v4i (&qf)[D / 32], int col, int hi,
                                        v16i &s0, v16i &s1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = kBias; s1[r] = kBias; }
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        const v4i k0 = *reinterpret_cast<const v4i *>(kt + k_lds<D>(col, 2 * s + hi));
        const v4i k1 = *reinterpret_cast<const v4i *>(kt + k_lds<D>(32 + col, 2 * s + hi));
        s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(k0, qf[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(k1, qf[s], s1, 0, 0, 0);
    }
}

// Online-softmax update and PV for one tile.  TAIL: keys >= nvalid masked.
template <int D, bool TAIL>
__device__ __forceinline__ void softmax_pv(const v16i &s0, const v16i &s1, const uint8_t *vt, float f,
                                           int col, int hi, int nvalid, float &m, float &dsum,
                                           v16f (&acc)[D / 32]) {
    int a[32];
#pragma unroll
    for (int r = 0; r < 16; ++r) { a[r] = s0[r]; a[16 + r] = s1[r]; }
    if (TAIL) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int key = 32 * (i >> 4) + 8 * ((i & 15) >> 2) + 4 * hi + (i & 3);
            if (key >= nvalid) a[i] = -2147483647 - 1;
        }
    }
    // row maximum of the biased integers (order-preserving), then both halves
    int t[11];
#pragma unroll
    for (int i = 0; i < 10; ++i) t[i] = imax3(a[3 * i], a[3 * i + 1], a[3 * i + 2]);
    t[10] = max(a[30], a[31]);
    int mx = imax3(imax3(t[0], t[1], t[2]), imax3(t[3], t[4], t[5]), imax3(t[6], t[7], t[8]));
    mx = imax3(mx, t[9], t[10]);
    mx = max(mx, shfl_xor_i(mx, 32));
    const float M = (__int_as_float(mx) - kBiasF) * f - 8.807f;
    const float mnew = __builtin_fmaxf(m, M);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    const bool moved = __any(mnew != m);
    m = mnew;
    dsum = dsum * alpha;
    const float nm = -mnew;

    int pk[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = 4 * q + i;
            float e = __builtin_amdgcn_exp2f(__builtin_fmaf(__int_as_float(a[idx]) - kBiasF, f, nm));
            if (TAIL) {
                const int key = 32 * (idx >> 4) + 8 * ((idx & 15) >> 2) + 4 * hi + (idx & 3);
                if (key >= nvalid) e = 0.0f;
            }
            pr[i] = e;
            dsum = dsum + e;
        }
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(pr[0], pr[1], 0, false);
        pk[q] = __builtin_amdgcn_cvt_pk_fp8_f32(pr[2], pr[3], w, true);
    }
    const v8i pb = {pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]};

    if (moved) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] = acc[i] * alpha;
    }
#pragma unroll
    for (int blk = 0; blk < D / 32; ++blk) {
        const int d = 32 * blk + col;
        const v4i va0 = *reinterpret_cast<const v4i *>(vt + v_lds(d, 2 * hi));
        const v4i va1 = *reinterpret_cast<const v4i *>(vt + v_lds(d, 2 * hi + 1));
        const v8i va = {va0[0], va0[1], va0[2], va0[3], va1[0], va1[1], va1[2], va1[3]};
        acc[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, acc[blk], 0, 0, 0, 0, 0, 0);
    }
}

// Register staging of one K or V tile: thread tid moves 16-byte chunks
// tid, tid + THREADS, ... between global memory and the swizzled LDS layout.
template <int CH, int THREADS>
__device__ __forceinline__ void stage_load(v4i (&dst)[CH], const uint8_t *src, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) dst[i] = *reinterpret_cast<const v4i *>(src + 16 * (tid + THREADS * i));
}
template <int D, int CH, int THREADS>
__device__ __forceinline__ void stage_store_k(const v4i (&src)[CH], uint8_t *kb, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = tid + THREADS * i;
        *reinterpret_cast<v4i *>(kb + k_lds<D>(c / (D / 16), c % (D / 16))) = src[i];
    }
}
template <int CH, int THREADS>
__device__ __forceinline__ void stage_store_v(const v4i (&src)[CH], uint8_t *vb, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = tid + THREADS * i;
        *reinterpret_cast<v4i *>(vb + v_lds(c >> 2, c & 3)) = src[i];
    }
}

template <int D, int WAVES, bool PIPE>
__global__ __launch_bounds__(64 * WAVES, 1) void attn_fwd_kernel(const AttnParams p) {
    constexpr int THREADS = 64 * WAVES;
    constexpr int QTILE = 32 * WAVES;                // query rows per work-group
    constexpr int KS = D / 32;                       // QK k-steps == PV output blocks
    constexpr int KT = 64 * D;                       // bytes of one K (or V) tile
    constexpr int CH = KT / 16 / THREADS;            // 16-byte chunks per thread per tile
    static_assert(CH >= 1 && CH * 16 * THREADS == KT, "tile must split evenly");
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][KT];
    __shared__ __attribute__((aligned(16))) uint8_t vbuf[2][KT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, col = lane & 31;

    // XCD-aware renumbering: hardware block i runs on XCD i % 8; give each XCD
    // a contiguous range of (b, h, query tile) so a head's tiles share an L2.
    const int total = gridDim.x, nxcd = 8;
    const int xq = total / nxcd, xr = total % nxcd;
    const int x = blockIdx.x % nxcd, k = blockIdx.x / nxcd;
    const int lid = x * xq + min(x, xr) + k;
    const int nqt = (p.N + QTILE - 1) / QTILE;
    const int qt = lid % nqt, h = (lid / nqt) % p.Hq, b = lid / (nqt * p.Hq);
    const int hk = h / p.grp;
    const int q0 = qt * QTILE + 32 * wave;           // first query row of the wave
    const int g = q0 >> 5;                           // its Q scale group

    // Q fragment (B operand of the QK MFMA): query q0+col, 16 bytes per k-step.
    const int8_t *qrow = p.q8 + (((int64_t)b * p.Hq + h) * p.q_rows + q0 + col) * D + 16 * hi;
    v4i qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const v4i *>(qrow + 32 * s);
    const float qs = (g < p.nq) ? p.q_scale[((int64_t)b * p.Hq + h) * p.nq + g] : 1.0f;
    const float qc = qs * p.c;

    const uint8_t *kbase = reinterpret_cast<const uint8_t *>(p.k8) + ((int64_t)b * p.Hkv + hk) * p.k_rows * D;
    const uint8_t *vbase = p.v8 + ((int64_t)b * p.Hkv + hk) * (int64_t)p.nk * D * 64;
    const float *ksc = p.k_scale + ((int64_t)b * p.Hkv + hk) * p.nk;
    const int nk = p.nk;
    const int tail_valid = p.N - 64 * (nk - 1);      // valid keys of the last tile (1..64)

    v4i stk[CH], stv[CH];
    auto tile_src = [&](const uint8_t *base, int t) { return base + (int64_t)min(t, nk - 1) * KT; };
#define SAGE_LOAD(dst, base, T) stage_load<CH, THREADS>(dst, tile_src(base, T), tid)
#define SAGE_STORE_K(buf) stage_store_k<D, CH, THREADS>(stk, kbuf[buf], tid)
#define SAGE_STORE_V(buf) stage_store_v<CH, THREADS>(stv, vbuf[buf], tid)

    v16f acc[KS];
#pragma unroll
    for (int i = 0; i < KS; ++i) acc[i] = v16f{};
    float m = -5000000.0f;
    float dsum = hi ? 0.0f : 1.0f;                   // d0 = 1 once per row

    if constexpr (PIPE) {
        // prologue: K0, V0, K1 into LDS; S(0); then K2 / V1 in flight
        SAGE_LOAD(stk, kbase, 0);
        SAGE_LOAD(stv, vbase, 0);
        SAGE_STORE_K(0);
        SAGE_STORE_V(0);
        SAGE_LOAD(stk, kbase, 1);
        SAGE_STORE_K(1);
        __syncthreads();
        v16i sc0, sc1;
        qk_tile<D>(kbuf[0], qf, col, hi, sc0, sc1);
        SAGE_LOAD(stk, kbase, 2);
        SAGE_LOAD(stv, vbase, 1);
        __syncthreads();                             // every wave has read K0

#define SAGE_PIPE_STEP(T, CUR, SC0, SC1, SN0, SN1)                                          \
    do {                                                                                    \
        qk_tile<D>(kbuf[(CUR) ^ 1], qf, col, hi, SN0, SN1);      /* S(T+1) in flight */     \
        softmax_pv<D, false>(SC0, SC1, vbuf[CUR], qc * ksc[T], col, hi, 64, m, dsum, acc);  \
        SAGE_STORE_K(CUR);                                       /* K(T+2) over K(T)   */   \
        SAGE_STORE_V((CUR) ^ 1);                                 /* V(T+1) over V(T-1) */   \
        __syncthreads();                                                                    \
        SAGE_LOAD(stk, kbase, (T) + 3);                                                     \
        SAGE_LOAD(stv, vbase, (T) + 2);                                                     \
    } while (0)
        v16i sn0, sn1;
        int t = 0;
        for (; t + 2 < nk; t += 2) {                 // tiles t, t+1 (both before the last)
            SAGE_PIPE_STEP(t, 0, sc0, sc1, sn0, sn1);
            SAGE_PIPE_STEP(t + 1, 1, sn0, sn1, sc0, sc1);
        }
        if (t < nk - 1) {
            SAGE_PIPE_STEP(t, 0, sc0, sc1, sn0, sn1);
            sc0 = sn0;
            sc1 = sn1;
        }
#undef SAGE_PIPE_STEP
        const int tl = nk - 1;
        const float f = qc * ksc[tl];
        if (tail_valid < 64)
            softmax_pv<D, true>(sc0, sc1, vbuf[tl & 1], f, col, hi, tail_valid, m, dsum, acc);
        else
            softmax_pv<D, false>(sc0, sc1, vbuf[tl & 1], f, col, hi, 64, m, dsum, acc);
    } else {
        // one tile of scores live at a time (wide heads): K(t), V(t) share a
        // buffer index; tile t+1 is staged while tile t is processed
        SAGE_LOAD(stk, kbase, 0);
        SAGE_LOAD(stv, vbase, 0);
        SAGE_STORE_K(0);
        SAGE_STORE_V(0);
        SAGE_LOAD(stk, kbase, 1);
        SAGE_LOAD(stv, vbase, 1);
        __syncthreads();
        for (int t = 0; t < nk - 1; ++t) {
            const int cur = t & 1;
            v16i sc0, sc1;
            qk_tile<D>(kbuf[cur], qf, col, hi, sc0, sc1);
            softmax_pv<D, false>(sc0, sc1, vbuf[cur], qc * ksc[t], col, hi, 64, m, dsum, acc);
            SAGE_STORE_K(cur ^ 1);                   // K(t+1), V(t+1) over tile t-1
            SAGE_STORE_V(cur ^ 1);
            __syncthreads();
            SAGE_LOAD(stk, kbase, t + 2);
            SAGE_LOAD(stv, vbase, t + 2);
        }
        const int t = nk - 1;
        v16i sc0, sc1;
        qk_tile<D>(kbuf[t & 1], qf, col, hi, sc0, sc1);
        if (tail_valid < 64)
            softmax_pv<D, true>(sc0, sc1, vbuf[t & 1], qc * ksc[t], col, hi, tail_valid, m, dsum, acc);
        else
            softmax_pv<D, false>(sc0, sc1, vbuf[t & 1], qc * ksc[t], col, hi, 64, m, dsum, acc);
    }
#undef SAGE_LOAD
#undef SAGE_STORE_K
#undef SAGE_STORE_V

    // ---- finalize: d over both lane halves, O = bf16((RO * (1/d)) * v_scale)
    const float dt = dsum + shfl_xor_f(dsum, 32);
    const float rinv = 1.0f / dt;
    const int n = q0 + col;
    if (n < p.N) {
        uint16_t *orow = p.o + (int64_t)b * p.osb + (int64_t)n * p.osn + (int64_t)h * p.osh;
        const float *vs = p.v_scale + ((int64_t)b * p.Hkv + hk) * D;
#pragma unroll
        for (int blk = 0; blk < KS; ++blk) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * blk + 8 * r4 + 4 * hi;
                const float4 sc = *reinterpret_cast<const float4 *>(vs + d0);
                const float o0 = (acc[blk][4 * r4 + 0] * rinv) * sc.x;
                const float o1 = (acc[blk][4 * r4 + 1] * rinv) * sc.y;
                const float o2 = (acc[blk][4 * r4 + 2] * rinv) * sc.z;
                const float o3 = (acc[blk][4 * r4 + 3] * rinv) * sc.w;
                *reinterpret_cast<uint2 *>(orow + d0) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
            }
        }
    }
}

}  // namespace
}  // namespace sage

hipError_t sage_launch_attn(const sage::AttnParams &p, int D, hipStream_t s) {
    if (D == 128) {
        constexpr int W = 8;
        const unsigned nqt = (unsigned)((p.N + 32 * W - 1) / (32 * W));
        sage::attn_fwd_kernel<128, W, true><<<dim3(nqt * p.Hq * p.B), 64 * W, 0, s>>>(p);
    } else {
        constexpr int W = 4;
        const unsigned nqt = (unsigned)((p.N + 32 * W - 1) / (32 * W));
        sage::attn_fwd_kernel<256, W, false><<<dim3(nqt * p.Hq * p.B), 64 * W, 0, s>>>(p);
    }
    return hipGetLastError();
}
