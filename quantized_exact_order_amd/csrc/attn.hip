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
// Schedules.  Heads of D = 128 run attn_ilv_kernel: 4 waves (128 query rows)
// per work-group, 2 work-groups per CU (2 waves per SIMD, which is what lets
// plain VALU instructions of the two waves issue side by side).  Each wave
// software-pipelines its tiles: iteration t holds S(t), the packed P(t-1) and
// the LDS tiles K(t+1), V(t-1), and interleaves the QK MFMAs of tile t+1 and
// the PV MFMAs of tile t-1 with the softmax of tile t in fenced slots.  K and
// V tiles are copied from global memory straight into the swizzled LDS
// layout (global_load_lds), a full iteration ahead.  Wide heads (D = 256)
// run attn_wide_kernel, which keeps one tile of scores live to stay within
// the register file and stages tiles through registers.
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

// Segmented (split-KV) schedule, an opt-in mode outside the contract's
// exact order: the work-group of segment seg runs only the key tiles
// [seg nk / nseg, (seg + 1) nk / nseg), from the initial state, and keeps its
// FP32 partials instead of finalizing.  seg_tiles moves the tile bases to the
// segment's first tile; the segment's last tile is partial only if it is the
// sequence's last one.
__device__ __forceinline__ void seg_tiles(const AttnParams &p, int seg, int nseg, int kt_bytes, const uint8_t *&kbase,
                                          const uint8_t *&vbase, const float *&ksc, int &nk, int &tail_valid) {
    const int t0 = (int)((int64_t)seg * p.nk / nseg), t1 = (int)((int64_t)(seg + 1) * p.nk / nseg);
    kbase += (int64_t)t0 * kt_bytes;
    vbase += (int64_t)t0 * kt_bytes;
    ksc += t0;
    nk = t1 - t0;
    if (t1 < p.nk) tail_valid = 64;
}

// A segment's partial for query row n: the lane's RO values (channels
// 32 blk + 8 r4 + 4 hi + 0..3), and the row's m and d from the lanes of half 0.
template <int D>
__device__ __forceinline__ void store_seg_partial(const AttnParams &p, int b, int h, int seg, int nseg, int n, int hi,
                                                  const v16f (&acc)[D / 32], float m, float d) {
    const int64_t row = (((int64_t)b * p.Hq + h) * nseg + seg) * p.N + n;
    float *ro = p.seg_ro + row * D;
#pragma unroll
    for (int blk = 0; blk < D / 32; ++blk)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<float4 *>(ro + 32 * blk + 8 * r4 + 4 * hi) =
                make_float4(acc[blk][4 * r4], acc[blk][4 * r4 + 1], acc[blk][4 * r4 + 2], acc[blk][4 * r4 + 3]);
    if (hi == 0) *reinterpret_cast<float2 *>(p.seg_md + 2 * row) = make_float2(m, d);
}

template <int D, int WAVES, bool SEG>
__global__ __launch_bounds__(64 * WAVES, 1) void attn_wide_kernel(const AttnParams p) {
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
    const int nseg = SEG ? p.nseg : 1;
    const int qt = lid % nqt, seg = (lid / nqt) % nseg;
    const int h = (lid / (nqt * nseg)) % p.Hq, b = lid / (nqt * nseg * p.Hq);
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
    int nk = p.nk;
    int tail_valid = p.N - 64 * (nk - 1);            // valid keys of the last tile (1..64)
    if constexpr (SEG) seg_tiles(p, seg, nseg, KT, kbase, vbase, ksc, nk, tail_valid);

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
#undef SAGE_LOAD
#undef SAGE_STORE_K
#undef SAGE_STORE_V

    // ---- finalize: d over both lane halves, O = bf16((RO * (1/d)) * v_scale)
    const float dt = dsum + shfl_xor_f(dsum, 32);
    const int n = q0 + col;
    if constexpr (SEG) {
        if (n < p.N) store_seg_partial<D>(p, b, h, seg, nseg, n, hi, acc, m, dt);
        return;
    }
    const float rinv = 1.0f / dt;
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


// ---------------------------------------------------------------------------
// Interleaved schedule: 4 waves (128 query rows) per work-group, two
// work-groups per CU.  Iteration t of a wave holds the finished scores S(t),
// the packed probabilities P(t-1) and the LDS tiles K(t+1), V(t-1); it issues
// the PV MFMAs of tile t-1 and the QK MFMAs of tile t+1 between the softmax
// instructions of tile t, so the matrix pipe runs while the VALU computes.
// The accumulator sees the same operations in the same order as tile-by-tile
// processing: RO += P(t-1) V(t-1) happens before RO *= alpha(t).
// ---------------------------------------------------------------------------

// One wave-wide copy of 1 KiB from global memory straight into LDS: lane l
// reads 16 bytes at base + off and writes them to lds + 16 l.  Issued from
// inline assembly so that the compiler does not treat it as a store to every
// LDS buffer (it would then wait for the copy before the next LDS read of any
// buffer); the copy has no register results, and the kernel waits for it
// (vmcnt) before a barrier that precedes any read of its destination.  M0 is
// set here for every copy.
__device__ __forceinline__ void lds_dma16(const uint8_t *base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)p;
}

// Source offsets of the lane's 16-byte chunks of the first 1 KiB block
// (block `wave`) that a wave copies of every K and every V tile, chosen so
// that the LDS bytes land in the swizzled positions of k_lds / v_lds.  Its
// second block (wave + 4) is 32 K rows / 64 V^T rows further on, where both
// swizzles repeat: the same offsets from a base 4096 bytes higher.
struct DmaLane {
    uint32_t k, v;
};

__device__ __forceinline__ DmaLane dma_lane(int wave, int lane) {
    const int c = wave * 64 + lane;                   // LDS chunk written by this lane
    const int r = c >> 3, pos = c & 7;                // K: row r, chunk position pos
    const int hk = (r & 7) ^ ((r >> 3) & 1);
    const int d = c >> 2, vp = c & 3;                 // V^T: row d, chunk position vp
    const int hv = ((d >> 1) & 1) ^ (((d >> 2) & 1) << 1) ^ ((d >> 3) & 1);
    return DmaLane{(uint32_t)(r * 128 + 16 * (pos ^ hk)), (uint32_t)(d * 64 + 16 * (vp ^ hv))};
}

// The copies one iteration issues: a K tile and a V tile, each into the LDS
// buffer (address of this wave's first block) given.
struct DmaJob {
    const uint8_t *ksrc, *vsrc;
    uint32_t klds, vlds;
};

// Maximum of v over lane pairs (l, l ^ 32): one v_permlane32_swap exchanges
// the two halves of the wave.
__device__ __forceinline__ int max_xor32(int v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max((int)r[0], (int)r[1]);
}

// Maximum of the 16 biased scores of a key block and `x`.
__device__ __forceinline__ int block_max(const v16i &v, int x) {
    const int a = imax3(v[0], v[1], v[2]), b = imax3(v[3], v[4], v[5]), d = imax3(v[6], v[7], v[8]);
    const int e = imax3(v[9], v[10], v[11]), g = imax3(v[12], v[13], v[14]);
    return imax3(imax3(a, b, d), imax3(e, g, v[15]), x);
}

// Online-softmax statistics of a tile whose lane maximum (biased) is mx:
// m' = max(m, float(max S) * f - 8.807), alpha = 2^(m - m'), d *= alpha.
// `moved` tells whether any row of the wave changed its maximum (alpha is
// exactly 1 for the others).
__device__ __forceinline__ void row_stats(int mx, float f, float &m, float &alpha, bool &moved,
                                          float &dsum) {
    mx = max_xor32(mx);
    const float M = (__int_as_float(mx) - kBiasF) * f - 8.807f;
    const float mnew = __builtin_fmaxf(m, M);
    alpha = __builtin_amdgcn_exp2f(m - mnew);
    moved = __any(mnew != m);
    m = mnew;
    dsum = dsum * alpha;
}

// One iteration t.  On entry m, alpha, moved and dsum already account for
// the maximum of S(t) = (sc0, sc1) (scale fc), and RO holds the tiles before
// t - 1 at the previous maximum.  The iteration
//   - turns S(t) into probabilities (d += p, FP8 packing into pcur),
//   - when NEXT, computes S(t+1) = K(t+1) Q^T into (sn0, sn1) from the LDS
//     tile kt, and then its maximum (scale fn) into m, alpha, moved, dsum
//     for the next iteration,
//   - when PREV, adds P(t-1) V(t-1) (pprev, LDS tile vt) to RO, and then
//     rescales RO by alpha(t),
// which is the per-tile order RO = RO alpha(t) + P(t) V(t) with the PV of
// each tile deferred by one iteration.  Every key of these tiles is valid
// (the last tile, which may be partial, takes the one-tile path).
//
// The instructions are laid out in 13 slots separated by scheduling fences:
// slots 0-7 each compute one group of four exponentials with their FP8
// packing, slots 1-8 also issue one QK MFMA each, slots 9-12 each issue one
// PV MFMA beside the row maximum of S(t+1); the LDS fragment reads run one or
// two slots ahead of their MFMA and the four tile copies of the iteration
// (job) go out one per slot, so that the copies of all waves do not queue up
// at once.
template <bool PREV, bool NEXT>
__device__ __forceinline__ void ilv_step(const v16i &sc0, const v16i &sc1, v16i &sn0, v16i &sn1,
                                         const v8i &pprev, v8i &pcur, const uint8_t *kt,
                                         const uint8_t *vt, const v4i (&qf)[4], float fc, float fn,
                                         int col, int hi, float &m, float &alpha,
                                         bool &moved, float &dsum, v16f (&acc)[4], const DmaJob &job,
                                         const DmaLane &dl) {
    constexpr int D = 128;
#define SAGE_FENCE __builtin_amdgcn_sched_barrier(0)
    int a[32];
#pragma unroll
    for (int r = 0; r < 16; ++r) { a[r] = sc0[r]; a[16 + r] = sc1[r]; }
    v8i vf[4];
    v4i kf[8];
    auto rd_v = [&](int blk) {
        if constexpr (PREV) {
            const int d = 32 * blk + col;
            const v4i x0 = *reinterpret_cast<const v4i *>(vt + v_lds(d, 2 * hi));
            const v4i x1 = *reinterpret_cast<const v4i *>(vt + v_lds(d, 2 * hi + 1));
            vf[blk] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        }
    };
    auto mf_v = [&](int blk) {
        if constexpr (PREV)
            acc[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[blk], pprev, acc[blk], 0, 0, 0, 0, 0, 0);
    };
    // QK MFMA j: k-step j >> 1 of key block j & 1 (the two accumulation
    // chains alternate)
    auto rd_k = [&](int j) {
        if constexpr (NEXT)
            kf[j] = *reinterpret_cast<const v4i *>(kt + k_lds<D>(32 * (j & 1) + col, 2 * (j >> 1) + hi));
    };
    auto mf_k = [&](int j) {
        if constexpr (NEXT) {
            v16i &sn = (j & 1) ? sn1 : sn0;
            const v16i c = (j < 2) ? v16i{kBias, kBias, kBias, kBias, kBias, kBias, kBias, kBias, kBias,
                                          kBias, kBias, kBias, kBias, kBias, kBias, kBias}
                                   : sn;
            sn = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[j], qf[j >> 1], c, 0, 0, 0);
        }
    };
    const float nm = -m;
    int pk[8];
    auto grp = [&](int q) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = 4 * q + i;
            float e = __builtin_amdgcn_exp2f(__builtin_fmaf(__int_as_float(a[idx]) - kBiasF, fc, nm));
            pr[i] = e;
            dsum = dsum + e;
        }
        // bytes 2-3 of the first pack are overwritten by the second: the
        // first operand's own register (dead afterwards) serves as the old value
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(pr[0], pr[1], __float_as_int(pr[0]), false);
        pk[q] = __builtin_amdgcn_cvt_pk_fp8_f32(pr[2], pr[3], w, true);
        // keep the group in its slot (IR passes would otherwise sink it to
        // the first use, past the rescale branch)
        asm volatile("" ::"v"(pk[q]), "v"(dsum));
    };

    rd_k(0); rd_k(1); grp(0); SAGE_FENCE;
    mf_k(0); lds_dma16(job.ksrc, dl.k, job.klds); rd_k(2); grp(1); SAGE_FENCE;
    mf_k(1); lds_dma16(job.ksrc + 4096, dl.k, job.klds + 4096); rd_k(3); grp(2); SAGE_FENCE;
    mf_k(2); lds_dma16(job.vsrc, dl.v, job.vlds); rd_k(4); grp(3); SAGE_FENCE;
    mf_k(3); lds_dma16(job.vsrc + 4096, dl.v, job.vlds + 4096); rd_k(5); grp(4); SAGE_FENCE;
    mf_k(4); rd_k(6); grp(5); SAGE_FENCE;
    mf_k(5); rd_k(7); rd_v(0); grp(6); SAGE_FENCE;
    mf_k(6); rd_v(1); grp(7); SAGE_FENCE;
    mf_k(7); rd_v(2); SAGE_FENCE;
    const float alpha_c = alpha;
    const bool moved_c = moved;
    int x0 = 0;
    mf_v(0); rd_v(3);
    if constexpr (NEXT) x0 = block_max(sn0, -2147483647 - 1);
    SAGE_FENCE;
    mf_v(1);
    if constexpr (NEXT) x0 = block_max(sn1, x0);
    SAGE_FENCE;
    mf_v(2);
    if constexpr (NEXT) {
        row_stats(x0, fn, m, alpha, moved, dsum);
        asm volatile("" ::"v"(m), "v"(alpha), "v"(dsum), "s"((int)moved));
    }
    SAGE_FENCE;
    mf_v(3); SAGE_FENCE;
#undef SAGE_FENCE
    pcur = v8i{pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]};
    if (PREV && moved_c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = acc[i] * alpha_c;
    }
}

template <int D, bool SEG>
__global__ __launch_bounds__(256, 2) void attn_ilv_kernel(const AttnParams p) {
    constexpr int QTILE = 128;
    constexpr int KS = D / 32;
    constexpr int KT = 64 * D;
    __shared__ __attribute__((aligned(1024))) uint8_t kbuf[2][KT];
    __shared__ __attribute__((aligned(1024))) uint8_t vbuf[2][KT];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5, col = lane & 31;

    const int total = gridDim.x, nxcd = 8;
    const int xq = total / nxcd, xr = total % nxcd;
    const int x = blockIdx.x % nxcd, k = blockIdx.x / nxcd;
    const int lid = x * xq + min(x, xr) + k;
    const int nqt = (p.N + QTILE - 1) / QTILE;
    const int nseg = SEG ? p.nseg : 1;
    const int qt = lid % nqt, seg = (lid / nqt) % nseg;
    const int h = (lid / (nqt * nseg)) % p.Hq, b = lid / (nqt * nseg * p.Hq);
    const int hk = h / p.grp;
    const int q0 = qt * QTILE + 32 * wave;
    const int g = q0 >> 5;

    const int8_t *qrow = p.q8 + (((int64_t)b * p.Hq + h) * p.q_rows + q0 + col) * D + 16 * hi;
    v4i qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const v4i *>(qrow + 32 * s);
    const float qs = (g < p.nq) ? p.q_scale[((int64_t)b * p.Hq + h) * p.nq + g] : 1.0f;
    const float qc = qs * p.c;

    const uint8_t *kbase = reinterpret_cast<const uint8_t *>(p.k8) + ((int64_t)b * p.Hkv + hk) * p.k_rows * D;
    const uint8_t *vbase = p.v8 + ((int64_t)b * p.Hkv + hk) * (int64_t)p.nk * D * 64;
    const float *ksc = p.k_scale + ((int64_t)b * p.Hkv + hk) * p.nk;
    int nk = p.nk;
    int tail_valid = p.N - 64 * (nk - 1);           // valid keys of the last tile (1..64)
    if constexpr (SEG) seg_tiles(p, seg, nseg, KT, kbase, vbase, ksc, nk, tail_valid);

    v16f acc[KS];
#pragma unroll
    for (int i = 0; i < KS; ++i) acc[i] = v16f{};
    float m = -5000000.0f, alpha = 1.0f;
    bool moved = false;
    float dsum = hi ? 0.0f : 1.0f;
    // k_scale of tiles t and t+1 while iteration t runs; the one of tile t+2
    // is loaded at its start (ahead of the tile copies, so that waiting for
    // it never waits for them) and used an iteration later
    float ks0 = ksc[0], ks1 = ksc[min(1, nk - 1)], ks2;

    const DmaLane dl = dma_lane(wave, lane);
    const uint32_t kl0 = lds_addr(kbuf[0]) + 1024 * wave, kl1 = lds_addr(kbuf[1]) + 1024 * wave;
    const uint32_t vl0 = lds_addr(vbuf[0]) + 1024 * wave, vl1 = lds_addr(vbuf[1]) + 1024 * wave;

    // Tiles 0 .. nk-2 run software-pipelined (all their keys are valid);
    // the last tile, which may be partial, runs the one-tile path after the
    // pipeline drains.  A single tile goes straight to that path.
    v16i sa0, sa1, sb0, sb1;
    v8i pa = {}, pb = {};
    DmaJob job;
    if (nk > 1) {
        // prologue: K(0), K(1) resident, S(0) and its maximum
        lds_dma16(kbase, dl.k, kl0);
        lds_dma16(kbase + 4096, dl.k, kl0 + 4096);
        lds_dma16(kbase + KT, dl.k, kl1);
        lds_dma16(kbase + KT + 4096, dl.k, kl1 + 4096);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        qk_tile<D>(kbuf[0], qf, col, hi, sa0, sa1);
        row_stats(block_max(sa1, block_max(sa0, -2147483647 - 1)), qc * ks0, m, alpha, moved, dsum);

        // iteration t: wait for K(t+1) / V(t-1), barrier (K(t), V(t-2)
        // consumed); the iteration then copies K(t+2) and V(t) into the
        // buffers those occupied (K(nk-1) again, unread, once t + 2 runs
        // past the last tile)
#define SAGE_ILV_SYNC(T)                                                                       \
    do {                                                                                       \
        __builtin_amdgcn_s_waitcnt(0x0F70);                                                    \
        __syncthreads();                                                                       \
        ks2 = ksc[min((T) + 2, nk - 1)];                                                       \
        job.ksrc = kbase + (int64_t)min((T) + 2, nk - 1) * KT;                                 \
        job.vsrc = vbase + (int64_t)(T) * KT;                                                  \
        job.klds = ((T) & 1) ? kl1 : kl0;                                                      \
        job.vlds = ((T) & 1) ? vl1 : vl0;                                                      \
    } while (0)
#define SAGE_ILV_ARGS qf, qc * ks0, qc * ks1, col, hi, m, alpha, moved, dsum, acc, job, dl
        // iteration t reads S(t) and P(t-1) and writes S(t+1) and P(t) in the
        // register sets of its parity: even t (sa -> sb, pb -> pa), odd t
        // (sb -> sa, pa -> pb), so no set is ever copied
#define SAGE_STEP_EVEN(P, N, T)                                                                \
    ilv_step<P, N>(sa0, sa1, sb0, sb1, pb, pa, kbuf[((T) + 1) & 1], vbuf[((T) + 1) & 1], SAGE_ILV_ARGS)
#define SAGE_STEP_ODD(P, N, T)                                                                 \
    ilv_step<P, N>(sb0, sb1, sa0, sa1, pa, pb, kbuf[((T) + 1) & 1], vbuf[((T) + 1) & 1], SAGE_ILV_ARGS)
#define SAGE_NEXT_SCALE do { ks0 = ks1; ks1 = ks2; } while (0)
        const int tp = nk - 2;                       // the last pipelined iteration
        SAGE_ILV_SYNC(0);
        if (tp == 0) SAGE_STEP_EVEN(false, false, 0);
        else SAGE_STEP_EVEN(false, true, 0);
        SAGE_NEXT_SCALE;
        int t = 1;
        for (; t + 1 < tp; t += 2) {                 // pairs (odd t, even t + 1) before tp
            SAGE_ILV_SYNC(t);
            SAGE_STEP_ODD(true, true, t);
            SAGE_NEXT_SCALE;
            SAGE_ILV_SYNC(t + 1);
            SAGE_STEP_EVEN(true, true, t + 1);
            SAGE_NEXT_SCALE;
        }
        if (t < tp) {                                // one odd iteration before tp
            SAGE_ILV_SYNC(t);
            SAGE_STEP_ODD(true, true, t);
            SAGE_NEXT_SCALE;
            ++t;
        }
        if (tp > 0) {                                // iteration tp: no next tile to score
            SAGE_ILV_SYNC(tp);
            if (tp & 1) SAGE_STEP_ODD(true, false, tp);
            else SAGE_STEP_EVEN(true, false, tp);
            SAGE_NEXT_SCALE;
        }
#undef SAGE_ILV_SYNC
#undef SAGE_ILV_ARGS
#undef SAGE_STEP_EVEN
#undef SAGE_STEP_ODD
#undef SAGE_NEXT_SCALE
        // drain: PV of tile tp (V(tp) was copied in iteration tp; P(tp) is in
        // pa for an even tp, pb for an odd one), and the copy of V(nk-1) into
        // the buffer of V(tp-1)
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        lds_dma16(vbase + (int64_t)(nk - 1) * KT, dl.v, (nk - 1) & 1 ? vl1 : vl0);
        lds_dma16(vbase + (int64_t)(nk - 1) * KT + 4096, dl.v, ((nk - 1) & 1 ? vl1 : vl0) + 4096);
        {
            const uint8_t *vt = vbuf[tp & 1];
            const v8i pl = (tp & 1) ? pb : pa;
#pragma unroll
            for (int blk = 0; blk < KS; ++blk) {
                const int d = 32 * blk + col;
                const v4i va0 = *reinterpret_cast<const v4i *>(vt + v_lds(d, 2 * hi));
                const v4i va1 = *reinterpret_cast<const v4i *>(vt + v_lds(d, 2 * hi + 1));
                const v8i va = {va0[0], va0[1], va0[2], va0[3], va1[0], va1[1], va1[2], va1[3]};
                acc[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pl, acc[blk], 0, 0, 0, 0, 0, 0);
            }
        }
    } else {
        lds_dma16(kbase, dl.k, kl0);
        lds_dma16(kbase + 4096, dl.k, kl0 + 4096);
        lds_dma16(vbase, dl.v, vl0);
        lds_dma16(vbase + 4096, dl.v, vl0 + 4096);
    }
    // the last tile (K(nk-1) was copied two iterations ahead, V(nk-1) above)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    {
        const int tl = nk - 1;
        v16i s0, s1;
        qk_tile<D>(kbuf[tl & 1], qf, col, hi, s0, s1);
        softmax_pv<D, true>(s0, s1, vbuf[tl & 1], qc * ksc[tl], col, hi, tail_valid, m, dsum, acc);
    }

    const float dt = dsum + shfl_xor_f(dsum, 32);
    const int n = q0 + col;
    if constexpr (SEG) {
        if (n < p.N) store_seg_partial<D>(p, b, h, seg, nseg, n, hi, acc, m, dt);
        return;
    }
    const float rinv = 1.0f / dt;
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

// Combines the segment partials of one output row (segmented schedule):
// M = max_s m_s, a_s = exp2(m_s - M), d = sum_s d_s a_s and RO = sum_s RO_s a_s
// (from 0, in increasing s), then O = bf16((RO * (1/d)) * v_scale) as in the
// exact epilogue; with one segment a_0 = 1 and the result is the exact one.
// Thread: 4 channels of one row.  Grid (ceil(N / rows per block), Hq, B).
template <int D>
__global__ __launch_bounds__(256) void attn_seg_combine_kernel(const AttnParams p) {
    constexpr int TPR = D / 4, RPB = 256 / TPR;      // threads per row, rows per block
    const int tid = threadIdx.x;
    const int n = blockIdx.x * RPB + tid / TPR, d0 = 4 * (tid % TPR);
    const int h = blockIdx.y, b = blockIdx.z;
    if (n >= p.N) return;
    const int hk = h / p.grp;
    const int64_t row0 = ((int64_t)b * p.Hq + h) * p.nseg * p.N + n;   // segment s: row0 + s * N
    float M = -INFINITY;
    for (int s = 0; s < p.nseg; ++s) M = __builtin_fmaxf(M, p.seg_md[2 * (row0 + (int64_t)s * p.N)]);
    float d = 0.0f, r0 = 0.0f, r1 = 0.0f, r2 = 0.0f, r3 = 0.0f;
    for (int s = 0; s < p.nseg; ++s) {
        const int64_t row = row0 + (int64_t)s * p.N;
        const float2 md = *reinterpret_cast<const float2 *>(p.seg_md + 2 * row);
        const float4 ro = *reinterpret_cast<const float4 *>(p.seg_ro + row * D + d0);
        const float a = __builtin_amdgcn_exp2f(md.x - M);
        d = d + md.y * a;
        r0 = r0 + ro.x * a;
        r1 = r1 + ro.y * a;
        r2 = r2 + ro.z * a;
        r3 = r3 + ro.w * a;
    }
    const float rinv = 1.0f / d;
    const float4 sc = *reinterpret_cast<const float4 *>(p.v_scale + ((int64_t)b * p.Hkv + hk) * D + d0);
    uint16_t *orow = p.o + (int64_t)b * p.osb + (int64_t)n * p.osn + (int64_t)h * p.osh;
    *reinterpret_cast<uint2 *>(orow + d0) =
        make_uint2(pack_bf16x2((r0 * rinv) * sc.x, (r1 * rinv) * sc.y), pack_bf16x2((r2 * rinv) * sc.z, (r3 * rinv) * sc.w));
}

}  // namespace
}  // namespace sage

hipError_t sage_launch_attn(const sage::AttnParams &p, int D, hipStream_t s) {
    if (D == 128) {
        const unsigned nqt = (unsigned)((p.N + 127) / 128);
        sage::attn_ilv_kernel<128, false><<<dim3(nqt * p.Hq * p.B), 256, 0, s>>>(p);
    } else {
        constexpr int W = 4;
        const unsigned nqt = (unsigned)((p.N + 32 * W - 1) / (32 * W));
        sage::attn_wide_kernel<256, W, false><<<dim3(nqt * p.Hq * p.B), 64 * W, 0, s>>>(p);
    }
    return hipGetLastError();
}

hipError_t sage_launch_attn_segmented(const sage::AttnParams &p, int D, hipStream_t s) {
    if (D == 128) {
        const unsigned nqt = (unsigned)((p.N + 127) / 128);
        sage::attn_ilv_kernel<128, true><<<dim3(nqt * p.nseg * p.Hq * p.B), 256, 0, s>>>(p);
    } else {
        constexpr int W = 4;
        const unsigned nqt = (unsigned)((p.N + 32 * W - 1) / (32 * W));
        sage::attn_wide_kernel<256, W, true><<<dim3(nqt * p.nseg * p.Hq * p.B), 64 * W, 0, s>>>(p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned rpb = 256 / (D / 4);
    if (D == 128) sage::attn_seg_combine_kernel<128><<<dim3((p.N + rpb - 1) / rpb, p.Hq, p.B), 256, 0, s>>>(p);
    else sage::attn_seg_combine_kernel<256><<<dim3((p.N + rpb - 1) / rpb, p.Hq, p.B), 256, 0, s>>>(p);
    return hipGetLastError();
}
