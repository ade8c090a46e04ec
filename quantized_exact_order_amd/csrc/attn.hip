// attn.hip -- fused quantized attention forward for gfx950 (CDNA4).
//
// Computes, per query row, the sequence of the page "Exact Numerical
// Contract", sections "INT8 QK And Score Domain", "Online Softmax", "V And PV"
// and "Finalization And Tails":
//   S    = q8 . k8 over D in INT32 (exact)             v_mfma_i32_32x32x32_i8
//   f    = (q_scale * c) * k_scale[t],  c = log2(e)/sqrt(D)
//   M    = float(max S) * f - 8.807;  m' = max(m, M);  alpha = 2^(m - m')
//   d    = d*alpha,  RO = RO*alpha   (skipped when no row of the wave moved;
//                                     alpha is then exactly 1)
//   p    = 2^(fma(float(S), f, -m')),  d += p,  p8 = e4m3(p)
//   RO  += p8 . v8 (FP32 accumulate)                   v_mfma_f32_32x32x64_f8f6f4
//   O    = bf16((RO * (1/d)) * v_scale)
// with m0 = -5e6, d0 = 1, KV tiles of 64 keys visited in increasing order and
// one work-group owning a 128-row query tile for the whole sequence (no split
// over keys).  Keys >= N in the last tile get p = 0 (their score would be
// -5e6) and never win the maximum.
//
// Layout on the wave: the score tile is computed transposed, S^T = K Q^T, so a
// lane holds 32 keys of ONE query row (column j = lane%32 of the accumulator;
// rows 8*(r/4) + 4*(lane/32) + r%4 of block c for register r).  Per-row state
// (m, d) is then per lane, the row maximum needs one exchange between the two
// lane halves, and the packed FP8 probabilities of the lane are directly the
// B operand (P^T) of the PV MFMA.  The prep pass stores each V tile as
// [D][64] with the keys permuted into exactly that register order
// (sage_v8_slot_key), so the A operand (V^T) is a plain 32-byte read.  The
// contract page's own PV accumulates each tile in FP16 on its hardware; the
// gfx950 FP8 MFMA accumulates in FP32 directly into RO.
//
// LDS: K and V tiles (64*D bytes each) double-buffered; 16-byte chunks are
// XOR-swizzled so that the MFMA operand reads are bank-conflict free.

#include "device.h"

namespace sage {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQTile = 32 * kWaves;       // query rows per work-group

// LDS byte offset of 16-byte chunk `j` of K row `r` (row length D bytes).
template <int D>
__device__ __forceinline__ int k_lds(int r, int j) { return r * D + 16 * (j ^ (r & 7)); }

// LDS byte offset of 16-byte chunk `j` (0..3) of V^T row `d` (64 bytes).
__device__ __forceinline__ int v_lds(int d, int j) { return d * 64 + 16 * (j ^ ((d >> 1) & 3)); }

template <int D>
__global__ __launch_bounds__(kThreads, D == 128 ? 2 : 1) void attn_fwd_kernel(const AttnParams p) {
    constexpr int KS = D / 32;                       // QK k-steps == PV output blocks
    constexpr int KT = 64 * D;                       // K tile bytes
    constexpr int TILE = 2 * KT;                     // K + V tile bytes
    constexpr int CH = TILE / 16 / kThreads;         // 16-byte chunks per thread per tile
    constexpr int KCH = KT / 16;                     // K chunks per tile
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, col = lane & 31;
    const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int hk = h / p.grp;
    const int q0 = qt * kQTile + 32 * wave;          // first query row of the wave
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

    v16f acc[KS];
#pragma unroll
    for (int i = 0; i < KS; ++i) acc[i] = v16f{};
    float m = -5000000.0f;
    float dsum = hi ? 0.0f : 1.0f;                   // d0 = 1 once per row

    // global -> registers -> LDS staging of one tile (K rows, then V^T rows)
    uint4 stage[CH];

#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = tid + kThreads * i;
        const uint8_t *src = (c < KCH) ? kbase + (int64_t)0 * KT + 16 * c
                                       : vbase + (int64_t)0 * KT + 16 * (c - KCH);
        stage[i] = *reinterpret_cast<const uint4 *>(src);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = tid + kThreads * i;
        const int off = (c < KCH) ? k_lds<D>(c / (D / 16), c % (D / 16))
                                  : KT + v_lds((c - KCH) >> 2, (c - KCH) & 3);
        *reinterpret_cast<uint4 *>(smem + 0 * TILE + off) = stage[i];
    }
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
        const int buf = t & 1;
        {
            // prefetch tile t+1 (the last tile is re-read harmlessly at the end)
            const int tn = (t + 1 < nk) ? t + 1 : t;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int c = tid + kThreads * i;
                const uint8_t *src = (c < KCH) ? kbase + (int64_t)tn * KT + 16 * c
                                               : vbase + (int64_t)tn * KT + 16 * (c - KCH);
                stage[i] = *reinterpret_cast<const uint4 *>(src);
            }
        }
        const uint8_t *kt = smem + buf * TILE;
        const uint8_t *vt = kt + KT;

        // ---- S^T = K Q^T (INT32) ------------------------------------------
        v16i s0 = v16i{}, s1 = v16i{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const v4i k0 = *reinterpret_cast<const v4i *>(kt + k_lds<D>(col, 2 * s + hi));
            const v4i k1 = *reinterpret_cast<const v4i *>(kt + k_lds<D>(32 + col, 2 * s + hi));
            s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(k0, qf[s], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(k1, qf[s], s1, 0, 0, 0);
        }

        // ---- row maximum (integer domain; x -> fl(x*f) is monotone) --------
        const bool tail = (t == nk - 1) && (tail_valid < 64);
        int mx = -2147483647 - 1;
        if (!tail) {
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = max(mx, max(s0[r], s1[r]));
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * hi + (r & 3);
                if (key < tail_valid) mx = max(mx, s0[r]);
                if (key + 32 < tail_valid) mx = max(mx, s1[r]);
            }
        }
        mx = max(mx, shfl_xor_i(mx, 32));
        const float f = qc * ksc[t];
        const float M = (float)mx * f - 8.807f;
        const float mnew = __builtin_fmaxf(m, M);
        if (__any(mnew != m)) {
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);
            dsum = dsum * alpha;
#pragma unroll
            for (int i = 0; i < KS; ++i) acc[i] = acc[i] * alpha;
        }
        m = mnew;
        const float nm = -mnew;

        // ---- probabilities -> E4M3, packed as the PV B operand -------------
        int pk[8];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float pr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * q + i;
                    const int sv = c ? s1[r] : s0[r];
                    float e = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sv, f, nm));
                    if (tail) {
                        const int key = 32 * c + 8 * q + 4 * hi + i;
                        if (key >= tail_valid) e = 0.0f;
                    }
                    pr[i] = e;
                    dsum = dsum + e;
                }
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(pr[0], pr[1], 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(pr[2], pr[3], w, true);
                pk[4 * c + q] = w;
            }
        }
        const v8i pb = {pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]};

        // ---- RO^T += V^T P^T (FP8 x FP8 -> FP32) ---------------------------
#pragma unroll
        for (int blk = 0; blk < KS; ++blk) {
            const int d = 32 * blk + col;
            const v4i va0 = *reinterpret_cast<const v4i *>(vt + v_lds(d, 2 * hi));
            const v4i va1 = *reinterpret_cast<const v4i *>(vt + v_lds(d, 2 * hi + 1));
            const v8i va = {va0[0], va0[1], va0[2], va0[3], va1[0], va1[1], va1[2], va1[3]};
            acc[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, acc[blk], 0, 0, 0, 0, 0, 0);
        }

#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + kThreads * i;
            const int off = (c < KCH) ? k_lds<D>(c / (D / 16), c % (D / 16))
                                      : KT + v_lds((c - KCH) >> 2, (c - KCH) & 3);
            *reinterpret_cast<uint4 *>(smem + (buf ^ 1) * TILE + off) = stage[i];
        }
        __syncthreads();
    }

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
    dim3 grid((unsigned)((p.N + sage::kQTile - 1) / sage::kQTile), p.Hq, p.B);
    if (D == 128) sage::attn_fwd_kernel<128><<<grid, sage::kThreads, 0, s>>>(p);
    else sage::attn_fwd_kernel<256><<<grid, sage::kThreads, 0, s>>>(p);
    return hipGetLastError();
}
