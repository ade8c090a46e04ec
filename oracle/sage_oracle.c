/*
 * sage_oracle.c -- plain, slow CPU oracle of the quantized attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, import or
 * call this file: only tests/, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or table with the HIP library.
 *
 * Authority: the page "Exact Numerical Contract",
 * sections "Preparation", "Q And K Quantization", "INT8 QK And Score Domain",
 * "Online Softmax", "V And PV", "Finalization And Tails".  Where that page is
 * silent the reading used is stated next to the step.  The Walsh-Hadamard
 * variant follows the NPU issue page on INT8 KV with per-head Hadamard
 * rotation (the rotation costs nothing on the K side; its place in the
 * order of steps is the page's stated risk).
 *
 * Arithmetic conventions: every + - * / sqrt is IEEE binary32 with
 * round-to-nearest-even; the file is compiled with -ffp-contract=off, so no
 * multiply-add is fused unless fmaf() is written.  FP32 subnormals are kept.
 *
 * Parity status of each exported function is recorded in its comment:
 * "pinned by" names the kind of independent check in tests/ that fixes it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static float f32_of_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* BF16 storage -> FP32 value (exact widening).  Pinned by: torch bf16 decode. */
float oracle_bf16_to_f32(uint16_t h) { return f32_of_bits((uint32_t)h << 16); }

/* FP32 -> BF16, round to nearest, ties to even (the rounding the page fixes
 * for BF16, section "Preparation").  Adding 0x7FFF plus the kept LSB to the 32-bit pattern and
 * truncating is the usual exact RNE on the binary encoding (a carry into the
 * exponent gives the next binade or infinity, as rounding requires).
 * NaN keeps its sign and becomes quiet.  Pinned by: torch's conversion. */
uint16_t oracle_f32_to_bf16(float x)
{
    uint32_t u = bits_of_f32(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* OCP E4M3 decode: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
 * is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities.
 * Pinned by: torch.float8_e4m3fn decode of all 256 codes. */
float oracle_e4m3_to_f32(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/* FP32 -> OCP E4M3, round to nearest even, saturate finite overflow to +-448
 * (the page converts probabilities and V this way, sections "Online
 * Softmax" and "V And PV").  NaN -> 0x7F/0xFF.
 * The value is scaled by a power of two so that the code's last mantissa step
 * is 1, rounded with rint() in double (exact, default mode is to-nearest-even)
 * and re-encoded.  Pinned by: torch float8_e4m3fn below 448, format facts. */
uint8_t oracle_f32_to_e4m3(float x)
{
    uint8_t sign = (bits_of_f32(x) >> 31) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (x != x) return (uint8_t)(sign | 0x7f);
    if (a >= 448.0) return (uint8_t)(sign | 0x7e);          /* satfinite */
    if (a < ldexp(1.0, -6)) {                                /* subnormal range */
        double q = rint(a * 512.0);                          /* units of 2^-9 */
        return (uint8_t)(sign | (uint8_t)q);                 /* q == 8 is 2^-6 */
    }
    int e2;
    double fr = frexp(a, &e2);                               /* a = fr * 2^e2, fr in [0.5,1) */
    int e = e2 - 1;                                          /* a = (2 fr) * 2^e */
    double q = rint((2.0 * fr - 1.0) * 8.0);                 /* mantissa in eighths */
    if (q == 8.0) { q = 0.0; e += 1; }
    int code = ((e + 7) << 3) | (int)q;
    if (code > 0x7e) code = 0x7e;
    return (uint8_t)(sign | code);
}

/* FP32 -> INT8 like cvt.rni.sat.s8.f32 ("Q And K Quantization"): round to
 * nearest integer, ties to even, clamp to [-128, 127]; NaN -> 0.
 * Pinned by: numpy rint + clip. */
int8_t oracle_f32_to_i8(float x)
{
    if (x != x) return 0;
    double r = rint((double)x);
    if (r > 127.0) r = 127.0;
    if (r < -128.0) r = -128.0;
    return (int8_t)r;
}

/* 2^x for the softmax (an approximate, flush-to-zero instruction on the
 * page's hardware).  The oracle does not imitate an approximate instruction:
 * it takes exp2 in FP64, rounds once to FP32, and flushes results below the
 * smallest normal to zero (the page's flush to zero).  Pinned by: numpy exp2
 * in FP64. */
float oracle_exp2(float x)
{
    float r = (float)exp2((double)x);
    if (r < 0x1p-126f) r = 0.0f;
    return r;
}

/* Score-domain constant c = (1/sqrt(D)) * log2(e), evaluated in FP64 and
 * rounded once to FP32 (the page scales scores by 1/sqrt(D) in base 2,
 * section "INT8 QK And Score Domain").  Pinned by: the closed form in tests. */
float oracle_score_scale(int D)
{
    return (float)((1.0 / sqrt((double)D)) * 1.4426950408889634073599246810019);
}

/* ------------------------------------------------------------------------ */
/* Preparation                                                               */
/* ------------------------------------------------------------------------ */

/*
 * RNE rounding of a real (held exactly in a double) to IEEE binary16: 10
 * fraction bits, exponent range [-14, 15], subnormal quantum 2^-24, values
 * at or above 65520 become infinity.  Returned as the float of that binary16
 * value (every binary16 value is a float).
 * Pinned by: numpy's float64 -> float16 conversion over random, tie and
 * subnormal inputs.
 */
float oracle_f64_to_f16(double x)
{
    if (x == 0.0 || x != x) return (float)x;
    double ax = fabs(x);
    if (ax >= 65520.0) return x > 0 ? INFINITY : -INFINITY;
    int e2;
    frexp(ax, &e2);                      /* ax = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;                      /* ax in [2^E, 2^(E+1)) */
    double quantum = (E < -14) ? ldexp(1.0, -24) : ldexp(1.0, E - 10);
    double r = rint(ax / quantum) * quantum;   /* exact division by a power of two */
    return (float)(x < 0 ? -r : r);
}

/* In-place balanced pairwise sum over n (a power of two) in natural order:
 * each level adds neighbours (t[2i], t[2i+1]). */
static float pairwise_sum(float *t, int n)
{
    for (int w = n; w > 1; w /= 2)
        for (int i = 0; i < w / 2; i++) t[i] = t[2 * i] + t[2 * i + 1];
    return t[0];
}

/*
 * Per-head RMSNorm then split-half RoPE of one BF16 tensor ("Preparation",
 * steps 1-3).
 *
 *   x        BF16 logical [B, N, H, D] at element strides (sb, sn, sh), unit d stride
 *   w        BF16 [D] RMSNorm weight, shared by all heads
 *   cosr/sinr BF16 [N, R/2] rotation coefficients (row stride R/2)
 *   z        out: BF16 [B, H, N, D] contiguous
 *
 * Readings (the page leaves the reduction order and rsqrt form open):
 *   ss   = pairwise tree over d of x_d * x_d  (each square is exact in FP32)
 *   inv  = 1.0f / sqrtf(ss / D + eps)
 *   y_d  = bf16((x_d * inv) * w_d)
 *   for i < R/2, with a = y_i, b = y_{i+R/2}, c = cos[n,i], s = sin[n,i]:
 *       z_i = bf16(a*c - b*s),  z_{i+R/2} = bf16(b*c + a*s)
 *   z_d = y_d for d >= R.
 * Pinned by: constant-row closed form, FP64 RMSNorm within 1 BF16 ulp,
 * position-0 identity, untouched tail dims, rotation norms, relative position.
 */
void oracle_rmsnorm_rope(int B, int N, int H, int D, int R, float eps,
                         const uint16_t *x, int64_t sb, int64_t sn, int64_t sh,
                         const uint16_t *w, const uint16_t *cosr, const uint16_t *sinr,
                         uint16_t *z)
{
    const int half = R / 2;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++) {
            float *t = (float *)malloc(sizeof(float) * D);
            float *y = (float *)malloc(sizeof(float) * D);
            for (int n = 0; n < N; n++) {
                const uint16_t *row = x + b * sb + n * sn + h * sh;
                for (int d = 0; d < D; d++) {
                    float v = oracle_bf16_to_f32(row[d]);
                    t[d] = v * v;
                }
                float ss = pairwise_sum(t, D);
                float inv = 1.0f / sqrtf(ss / (float)D + eps);
                for (int d = 0; d < D; d++) {
                    float v = oracle_bf16_to_f32(row[d]);
                    float n1 = v * inv;
                    float n2 = n1 * oracle_bf16_to_f32(w[d]);
                    y[d] = oracle_bf16_to_f32(oracle_f32_to_bf16(n2));
                }
                uint16_t *out = z + (((int64_t)b * H + h) * N + n) * D;
                for (int d = 0; d < D; d++) out[d] = oracle_f32_to_bf16(y[d]);
                for (int i = 0; i < half; i++) {
                    float a = y[i], bb = y[i + half];
                    float c = oracle_bf16_to_f32(cosr[(int64_t)n * half + i]);
                    float s = oracle_bf16_to_f32(sinr[(int64_t)n * half + i]);
                    float r0 = a * c - bb * s;
                    float r1 = bb * c + a * s;
                    out[i] = oracle_f32_to_bf16(r0);
                    out[i + half] = oracle_f32_to_bf16(r1);
                }
            }
            free(t);
            free(y);
        }
}

/*
 * Exact global K sequence mean per (b, h, d) ("Preparation", step 4:
 * computed over the whole sequence and subtracted before K quantization).
 *
 *   zk    BF16 [B, H, N, D] prepared K
 *   mean  out: FP32 [B, H, D]
 *
 * Reading (the production tree is not frozen on the page): S is the balanced
 * pairwise tree, in natural order, over P = 2^ceil(log2 N) leaves (P = 1 for
 * N = 1), leaf n being zk[n] for n < N and +0.0f for n >= N;
 * mean = S / (float)N.  For N >= 64 the same tree is a pairwise tree inside
 * every aligned 64-row block followed by a pairwise tree over the blocks,
 * padded to a power of two with +0.0f.
 * Pinned by: constant column gives the constant exactly; FP64 mean within
 * FP32 rounding; sum of (z - mean) near zero; a column of negative zeros over
 * a power-of-two N has no padding leaf and sums to -0.0 (IEEE 754: the sum of
 * two zeros of one sign keeps that sign), one more row brings in a +0.0f leaf.
 */
void oracle_k_mean(int B, int H, int N, int D, const uint16_t *zk, float *mean)
{
    int64_t P = 1;
    while (P < N) P *= 2;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++) {
            float *t = (float *)malloc(sizeof(float) * P);
            for (int d = 0; d < D; d++) {
                for (int64_t n = 0; n < P; n++)
                    t[n] = (n < N) ? oracle_bf16_to_f32(zk[(((int64_t)b * H + h) * N + n) * D + d])
                                   : 0.0f;
                float S = pairwise_sum(t, (int)P);
                mean[((int64_t)b * H + h) * D + d] = S / (float)N;
            }
            free(t);
        }
}

/*
 * Normalized Walsh-Hadamard transform of one row, in place, FP32 (the NPU
 * issue's per-head rotation, which leaves QK^T unchanged).  Sylvester (natural)
 * order; butterfly stages with span 1, 2, ..., D/2, each pair (a, b) at
 * (j, j+span) becoming (a + b, a - b); then every element times 1/sqrt(D),
 * which is a power of two for the supported D (= 4^k), so the scaling is exact.
 * Pinned by: H H = I, agreement with scipy.linalg.hadamard, score invariance.
 */
void oracle_wht(float *u, int D)
{
    for (int span = 1; span < D; span *= 2)
        for (int i = 0; i < D; i += 2 * span)
            for (int j = i; j < i + span; j++) {
                float a = u[j], b = u[j + span];
                u[j] = a + b;
                u[j + span] = a - b;
            }
    float s = (float)(1.0 / sqrt((double)D));
    for (int d = 0; d < D; d++) u[d] = u[d] * s;
}

/* One quantization group: rows [r0, r1) of u (row length D, FP32) ->
 * amax = max(1e-7f, max|u|), scale = amax/127, q8 = i8(u * (127/amax))
 * ("Q And K Quantization"; the multiplier is its own division, as printed). */
static float quant_group(const float *u, int rows, int D, int8_t *q8)
{
    float m = 0.0f;
    for (int64_t e = 0; e < (int64_t)rows * D; e++) {
        float a = fabsf(u[e]);
        if (a > m) m = a;
    }
    float amax = (m > 1e-7f) ? m : 1e-7f;
    float scale = amax / 127.0f;
    float mul = 127.0f / amax;
    for (int64_t e = 0; e < (int64_t)rows * D; e++) q8[e] = oracle_f32_to_i8(u[e] * mul);
    return scale;
}

/*
 * Q quantization: one scale per 32 query rows ("Q And K Quantization").
 *   zq       BF16 [B, H, N, D] prepared Q
 *   q8       out: INT8 [B, H, N, D] (valid rows only)
 *   q_scale  out: FP32 [B, H, ceil(N/128)*4]; groups with no valid row get
 *            1e-7f/127 (the page's shape [1,56,1184] counts four groups per
 *            128-row tile; the reading is that every group is defined).
 * hadamard != 0 rotates each row (oracle_wht) before the group maximum.
 * Pinned by: |q8*scale - u| <= scale/2, the maximum maps to +-127, zero group.
 */
void oracle_quant_q(int B, int H, int N, int D, int hadamard, const uint16_t *zq,
                    int8_t *q8, float *q_scale)
{
    const int nq = ((N + 127) / 128) * 4;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++) {
            float *u = (float *)malloc(sizeof(float) * 32 * D);
            for (int g = 0; g < nq; g++) {
                int r0 = g * 32, r1 = r0 + 32 < N ? r0 + 32 : N;
                int rows = r1 > r0 ? r1 - r0 : 0;
                for (int r = 0; r < rows; r++) {
                    const uint16_t *src = zq + (((int64_t)b * H + h) * N + r0 + r) * D;
                    for (int d = 0; d < D; d++) u[(int64_t)r * D + d] = oracle_bf16_to_f32(src[d]);
                    if (hadamard) oracle_wht(u + (int64_t)r * D, D);
                }
                int8_t *dst = q8 + (((int64_t)b * H + h) * N + (rows ? r0 : 0)) * D;
                q_scale[((int64_t)b * H + h) * nq + g] = quant_group(u, rows, D, dst);
            }
            free(u);
        }
}

/*
 * K smoothing and quantization: u = zk - mean (FP32, one rounding), optional
 * rotation, one scale per 64 key rows ("Preparation" step 4 and "Q And K
 * Quantization").
 *   k8       out: INT8 [B, H, N, D]
 *   k_scale  out: FP32 [B, H, ceil(N/64)]
 * Pinned by: quantization bounds, constant column smoothed to exactly zero.
 */
void oracle_quant_k(int B, int H, int N, int D, int hadamard, const uint16_t *zk,
                    const float *mean, int8_t *k8, float *k_scale)
{
    const int nk = (N + 63) / 64;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++) {
            float *u = (float *)malloc(sizeof(float) * 64 * D);
            const float *mu = mean + ((int64_t)b * H + h) * D;
            for (int t = 0; t < nk; t++) {
                int r0 = t * 64, r1 = r0 + 64 < N ? r0 + 64 : N;
                int rows = r1 - r0;
                for (int r = 0; r < rows; r++) {
                    const uint16_t *src = zk + (((int64_t)b * H + h) * N + r0 + r) * D;
                    for (int d = 0; d < D; d++)
                        u[(int64_t)r * D + d] = oracle_bf16_to_f32(src[d]) - mu[d];
                    if (hadamard) oracle_wht(u + (int64_t)r * D, D);
                }
                int8_t *dst = k8 + (((int64_t)b * H + h) * N + r0) * D;
                k_scale[((int64_t)b * H + h) * nk + t] = quant_group(u, rows, D, dst);
            }
            free(u);
        }
}

/*
 * V to FP8 with one scale per (b, h, d) over the whole sequence ("V And PV"):
 *   amax = max_n |v|, floored at 1e-7f (reading: the page gives no floor,
 *          and an all-zero channel would otherwise divide by zero),
 *   v_scale = amax / 2.25f,  v8 = e4m3(v * (2.25f / amax)).
 *   v        BF16 logical [B, N, H, D] at strides (sb, sn, sh)
 *   v8       out: E4M3 [B, H, N, D] in logical key order
 *   v_scale  out: FP32 [B, H, D]
 * Pinned by: decoded v8 * v_scale within half an E4M3 step of v; amax -> 448/... .
 */
void oracle_quant_v(int B, int N, int H, int D, const uint16_t *v, int64_t sb, int64_t sn,
                    int64_t sh, uint8_t *v8, float *v_scale)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++)
            for (int d = 0; d < D; d++) {
                float m = 0.0f;
                for (int n = 0; n < N; n++) {
                    float a = fabsf(oracle_bf16_to_f32(v[b * sb + n * sn + h * sh + d]));
                    if (a > m) m = a;
                }
                float amax = (m > 1e-7f) ? m : 1e-7f;
                v_scale[((int64_t)b * H + h) * D + d] = amax / 2.25f;
                float mul = 2.25f / amax;
                for (int n = 0; n < N; n++) {
                    float x = oracle_bf16_to_f32(v[b * sb + n * sn + h * sh + d]);
                    v8[(((int64_t)b * H + h) * N + n) * D + d] = oracle_f32_to_e4m3(x * mul);
                }
            }
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

/* Operands of query row (b, h, i): its INT8 row and Q-group scale, and the
 * K, V, K-scale and V-scale arrays of its KV head h / (Hq / Hkv). */
struct row_operands {
    const int8_t *qi, *kb;
    const uint8_t *vb;
    const float *ks, *vs;
    float qs;
};

static struct row_operands row_operands_of(int N, int Hq, int Hkv, int D, const int8_t *q8,
                                           const float *q_scale, const int8_t *k8, const float *k_scale,
                                           const uint8_t *v8, const float *v_scale, int b, int h, int i)
{
    const int nq = ((N + 127) / 128) * 4;
    const int nk = (N + 63) / 64;
    const int grp = Hq / Hkv;
    struct row_operands r;
    int hk = h / grp;
    r.qi = q8 + (((int64_t)b * Hq + h) * N + i) * D;
    r.qs = q_scale[((int64_t)b * Hq + h) * nq + i / 32];
    r.kb = k8 + ((int64_t)b * Hkv + hk) * N * D;
    r.vb = v8 + ((int64_t)b * Hkv + hk) * N * D;
    r.ks = k_scale + ((int64_t)b * Hkv + hk) * nk;
    r.vs = v_scale + ((int64_t)b * Hkv + hk) * D;
    return r;
}

/* The per-tile steps for key tiles t0 .. t1-1 in increasing order, from the
 * state (RO, m, d); T is scratch of D floats.  The steps are listed with
 * oracle_attn_rows_mode below. */
static void attn_tiles(const struct row_operands *r, int N, int D, float c, const float *dec, int t0, int t1,
                       int pv_fp16, float *RO, float *T, float *m_io, float *d_io)
{
    const int8_t *qi = r->qi, *kb = r->kb;
    const uint8_t *vb = r->vb;
    const float *ks = r->ks;
    const float qs = r->qs;
    int32_t S[64];
    float sv[64];
    uint8_t p8[64];
    float m = *m_io, d = *d_io;
    for (int t = t0; t < t1; t++) {
        float f = (qs * c) * ks[t];
        float mx = -INFINITY;
        for (int j = 0; j < 64; j++) {
            int key = t * 64 + j;
            if (key < N) {
                int32_t acc = 0;
                for (int e = 0; e < D; e++)
                    acc += (int32_t)qi[e] * (int32_t)kb[(int64_t)key * D + e];
                S[j] = acc;
                sv[j] = (float)acc * f;
            } else {
                S[j] = 0;
                sv[j] = -5000000.0f;
            }
            if (sv[j] > mx) mx = sv[j];
        }
        float M = mx - 8.807f;
        float mn = (m > M) ? m : M;
        float alpha = oracle_exp2(m - mn);
        d = d * alpha;
        for (int e = 0; e < D; e++) RO[e] = RO[e] * alpha;
        for (int j = 0; j < 64; j++) {
            int key = t * 64 + j;
            float p = (key < N) ? oracle_exp2(fmaf((float)S[j], f, -mn)) : 0.0f;
            d = d + p;
            p8[j] = oracle_f32_to_e4m3(p);
        }
        if (!pv_fp16) {
            for (int e = 0; e < D; e++) T[e] = 0.0f;
            for (int j = 0; j < 64; j++) {
                int key = t * 64 + j;
                if (key >= N) continue;           /* invalid V rows are zero */
                float pj = dec[p8[j]];
                const uint8_t *vr = vb + (int64_t)key * D;
                for (int e = 0; e < D; e++) T[e] = T[e] + pj * dec[vr[e]];
            }
        } else {
            /* two ordered K=32 steps into an FP16 fragment: each step adds
             * its 32 exact products (exact in double) to the fragment and
             * rounds once to FP16 */
            for (int e = 0; e < D; e++) {
                double frag = 0.0;
                for (int half = 0; half < 2; half++) {
                    double acc = frag;
                    for (int j = 32 * half; j < 32 * half + 32; j++) {
                        int key = t * 64 + j;
                        if (key >= N) continue;
                        acc += (double)dec[p8[j]] * (double)dec[vb[(int64_t)key * D + e]];
                    }
                    frag = (double)oracle_f64_to_f16(acc);
                }
                T[e] = (float)frag;
            }
        }
        for (int e = 0; e < D; e++) RO[e] = RO[e] + T[e];
        m = mn;
    }
    *m_io = m;
    *d_io = d;
}

/* O = bf16((RO * (1/d)) * v_scale) ("Finalization And Tails"). */
static void finalize_row(const float *RO, float d, const float *vs, int D, uint16_t *o)
{
    float rcp = 1.0f / d;
    for (int e = 0; e < D; e++) o[e] = oracle_f32_to_bf16((RO[e] * rcp) * vs[e]);
}

/*
 * Quantized attention for a list of query rows ("INT8 QK And Score Domain",
 * "Online Softmax", "V And PV", "Finalization And Tails").
 *
 *   q8 [B,Hq,N,D], q_scale [B,Hq,ceil(N/128)*4], k8 [B,Hkv,N,D],
 *   k_scale [B,Hkv,ceil(N/64)], v8 [B,Hkv,N,D] (logical order), v_scale [B,Hkv,D]
 *   rows: nrows triples (b, h, i);  o: out BF16 [nrows, D]
 *   GQA: query head h reads KV head h / (Hq/Hkv).
 *
 * Per query row i (its Q group g = i/32), with c = oracle_score_scale(D),
 * starting from RO = 0, m = -5e6, d = 1, for tiles t = 0, 1, ... in order:
 *   f   = (q_scale[g] * c) * k_scale[t]            (reading of the dequant placement)
 *   S_j = sum_d q8[i,d] * k8[j,d]  (exact integer)
 *   s_j = float(S_j) * f for valid keys j < N, -5e6 for the tile's invalid keys
 *   M   = (max_j s_j) - 8.807f;   m' = max(m, M);   alpha = exp2(m - m')
 *   d  *= alpha;  RO *= alpha
 *   p_j = exp2(fma(float(S_j), f, -m')) for valid j, else 0;  d += p_j (ascending j)
 *   T[e] = sum_j dec(e4m3(p_j)) * dec(v8[j,e])   (FP32, ascending j; exact products)
 *   RO[e] += T[e];  m = m'
 * then O[e] = bf16((RO[e] * (1.0f / d)) * v_scale[e]).
 *
 * The per-tile FP32 sum T stands for the page's per-tile PV partial, which it
 * accumulates in FP16 on its hardware; the oracle keeps FP32 (reading), and
 * oracle_attn_rows_mode(..., pv_fp16 = 1) emulates the FP16 two-level
 * accumulation instead.
 * Pinned by: N=1 and zero-query closed forms, one-hot rows, FP64 softmax
 * attention (cosine), brute-force integer dot products.
 */
void oracle_attn_rows_mode(int B, int N, int Hq, int Hkv, int D,
                           const int8_t *q8, const float *q_scale,
                           const int8_t *k8, const float *k_scale,
                           const uint8_t *v8, const float *v_scale,
                           int64_t nrows, const int32_t *rows, uint16_t *o, int pv_fp16)
{
    const int nk = (N + 63) / 64;
    const float c = oracle_score_scale(D);
    float dec[256];
    for (int i = 0; i < 256; i++) dec[i] = oracle_e4m3_to_f32((uint8_t)i);

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; r++) {
        struct row_operands ro = row_operands_of(N, Hq, Hkv, D, q8, q_scale, k8, k_scale, v8, v_scale,
                                                 rows[3 * r], rows[3 * r + 1], rows[3 * r + 2]);
        float *RO = (float *)calloc(D, sizeof(float));
        float *T = (float *)malloc(sizeof(float) * D);
        float m = -5000000.0f, d = 1.0f;
        attn_tiles(&ro, N, D, c, dec, 0, nk, pv_fp16, RO, T, &m, &d);
        finalize_row(RO, d, ro.vs, D, o + r * D);
        free(RO);
        free(T);
    }
}

/*
 * Segmented (split-KV) schedule: an opt-in mode that is NOT the contract's
 * exact order (the contract forbids combining KV partials; the FP8-PV
 * page's segmented schedule is the model).  The nseg segments split the key
 * tiles [0, nk) into contiguous runs, segment s covering tiles
 * [s nk / nseg, (s + 1) nk / nseg) (integer division; 1 <= nseg <= nk, so no
 * run is empty).  Each segment runs the per-tile steps above from the
 * initial state (RO = 0, m = -5e6, d = 1) over its tiles, giving
 * (RO_s, m_s, d_s).  The segments are then combined in increasing s:
 *   M = max_s m_s,  a_s = exp2(m_s - M)  (the softmax's exp2),
 *   d = sum_s d_s * a_s,  RO[e] = sum_s RO_s[e] * a_s  (FP32, from 0, in order),
 * and O is finalized as in the exact path.  With nseg = 1 the combine is the
 * identity (a_0 = 1), so the result is the exact path's.
 * Pinned by: nseg = 1 against the exact oracle, the zero-query and one-hot
 * closed forms at every segmentation, FP64 attention on the dequantized
 * tensors.
 */
void oracle_attn_rows_segmented(int B, int N, int Hq, int Hkv, int D,
                                const int8_t *q8, const float *q_scale,
                                const int8_t *k8, const float *k_scale,
                                const uint8_t *v8, const float *v_scale,
                                int64_t nrows, const int32_t *rows, int nseg, uint16_t *o)
{
    const int nk = (N + 63) / 64;
    const float c = oracle_score_scale(D);
    float dec[256];
    for (int i = 0; i < 256; i++) dec[i] = oracle_e4m3_to_f32((uint8_t)i);

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; r++) {
        struct row_operands ro = row_operands_of(N, Hq, Hkv, D, q8, q_scale, k8, k_scale, v8, v_scale,
                                                 rows[3 * r], rows[3 * r + 1], rows[3 * r + 2]);
        float *ROs = (float *)calloc((size_t)nseg * D, sizeof(float));
        float *ms = (float *)malloc(sizeof(float) * nseg);
        float *ds = (float *)malloc(sizeof(float) * nseg);
        float *T = (float *)malloc(sizeof(float) * D);
        for (int s = 0; s < nseg; s++) {
            int t0 = (int)((int64_t)s * nk / nseg), t1 = (int)((int64_t)(s + 1) * nk / nseg);
            ms[s] = -5000000.0f;
            ds[s] = 1.0f;
            attn_tiles(&ro, N, D, c, dec, t0, t1, 0, ROs + (int64_t)s * D, T, &ms[s], &ds[s]);
        }
        float M = ms[0];
        for (int s = 1; s < nseg; s++) M = (ms[s] > M) ? ms[s] : M;
        float *RO = T;
        float d = 0.0f;
        for (int e = 0; e < D; e++) RO[e] = 0.0f;
        for (int s = 0; s < nseg; s++) {
            float a = oracle_exp2(ms[s] - M);
            d = d + ds[s] * a;
            for (int e = 0; e < D; e++) RO[e] = RO[e] + ROs[(int64_t)s * D + e] * a;
        }
        finalize_row(RO, d, ro.vs, D, o + r * D);
        free(ROs);
        free(ms);
        free(ds);
        free(T);
    }
}

/* The FP32 per-tile partial (pv_fp16 = 0) is the oracle's reading and the
 * parity target; pv_fp16 = 1 emulates the page's two-level PV (each 64-key
 * partial accumulated in FP16 by two ordered K=32 steps, then added to the
 * FP32 RO) to measure how far an FP32-accumulating path sits from it. */
void oracle_attn_rows(int B, int N, int Hq, int Hkv, int D,
                      const int8_t *q8, const float *q_scale,
                      const int8_t *k8, const float *k_scale,
                      const uint8_t *v8, const float *v_scale,
                      int64_t nrows, const int32_t *rows, uint16_t *o)
{
    oracle_attn_rows_mode(B, N, Hq, Hkv, D, q8, q_scale, k8, k_scale, v8, v_scale, nrows, rows, o, 0);
}

/* ------------------------------------------------------------------------ */
/* Decode-time INT8 K cache with per-head Hadamard rotation                  */
/* (the NPU issue page on INT8 KV with per-head Hadamard rotation, part A:   */
/* INT8 K with one FP32 scale per (head, token) taken after the rotation;    */
/* the rotation is free on the K side because (QH)(KH)^T = QK^T; V stays in  */
/* 16-bit floating point)                                                    */
/* ------------------------------------------------------------------------ */

/*
 * Cache entry of K row (b, t, h) of a BF16 view with element strides
 * (sb, sn, sh) and unit d stride:
 *   u     = oracle_wht(float(k))             (normalized, FP32 stages)
 *   amax  = max(1e-7, max_d |u|);  scale = amax / 127
 *   k8    = i8(u * (127 / amax))             (own division, RNE, saturating)
 * Writes k8 [B, H, T, D] and kscale [B, H, T].  The quantization formula is
 * the one the contract page gives for Q and K blocks, applied to one row.
 * Pinned by: |u - k8 * scale| <= scale / 2 and max |k8| = 127 per row, and the
 * rotated scores against scipy's Hadamard matrix.
 */
void oracle_kv_quant(int B, int T, int H, int D, const uint16_t *k, int64_t sb, int64_t sn,
                     int64_t sh, int8_t *k8, float *kscale)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++) {
            float *u = (float *)malloc(sizeof(float) * D);
            for (int t = 0; t < T; t++) {
                const uint16_t *row = k + (int64_t)b * sb + (int64_t)t * sn + (int64_t)h * sh;
                for (int d = 0; d < D; d++) u[d] = oracle_bf16_to_f32(row[d]);
                oracle_wht(u, D);
                int64_t r = ((int64_t)b * H + h) * T + t;
                kscale[r] = quant_group(u, 1, D, k8 + r * D);
            }
            free(u);
        }
}

/*
 * Single-query attention of query row (b, h) over the first T cached tokens
 * of KV head h / (Hq / Hkv), in FP64 (the page fixes the cache formats, not
 * the arithmetic of the decode step; FP64 is the plain reading):
 *   qr   = oracle_wht(float(q))                        (FP32, as the cache)
 *   s_t  = (sum_d qr[d] * k8[t, d]) * kscale[t] / sqrt(D)
 *   w    = softmax(s) over t < T
 *   o[d] = sum_t w_t * float(v[t, d]);  O = bf16(float(o))
 * q: BF16 [B, Hq, D]; k8 [B, Hkv, Tc, D], kscale [B, Hkv, Tc], v: BF16
 * [B, Hkv, Tc, D] (cache capacity Tc >= T); o: BF16 [B, Hq, D]; w (optional):
 * FP64 [B, Hq, T] attention weights.
 * Pinned by: numpy attention on the dequantized cache rotated back with
 * scipy's Hadamard matrix, T = 1 closed form, uniform weights for a zero query.
 */
void oracle_decode_attn(int B, int Hq, int Hkv, int D, int T, int Tc, const uint16_t *q,
                        const int8_t *k8, const float *kscale, const uint16_t *v, uint16_t *o,
                        double *w)
{
    const int grp = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < Hq; h++) {
            const int hk = h / grp;
            float *qr = (float *)malloc(sizeof(float) * D);
            double *s = (double *)malloc(sizeof(double) * (T > 0 ? T : 1));
            double *acc = (double *)calloc(D, sizeof(double));
            const uint16_t *qrow = q + ((int64_t)b * Hq + h) * D;
            for (int d = 0; d < D; d++) qr[d] = oracle_bf16_to_f32(qrow[d]);
            oracle_wht(qr, D);
            const int64_t base = ((int64_t)b * Hkv + hk) * Tc;
            double mx = -INFINITY;
            for (int t = 0; t < T; t++) {
                double dot = 0.0;
                const int8_t *kr = k8 + (base + t) * D;
                for (int d = 0; d < D; d++) dot += (double)qr[d] * (double)kr[d];
                s[t] = dot * (double)kscale[base + t] / sqrt((double)D);
                if (s[t] > mx) mx = s[t];
            }
            double l = 0.0;
            for (int t = 0; t < T; t++) {
                s[t] = exp(s[t] - mx);
                l += s[t];
            }
            for (int t = 0; t < T; t++) {
                const double wt = s[t] / l;
                if (w) w[((int64_t)b * Hq + h) * T + t] = wt;
                const uint16_t *vr = v + (base + t) * D;
                for (int d = 0; d < D; d++) acc[d] += wt * (double)oracle_bf16_to_f32(vr[d]);
            }
            for (int d = 0; d < D; d++) o[((int64_t)b * Hq + h) * D + d] = oracle_f32_to_bf16((float)acc[d]);
            free(qr);
            free(s);
            free(acc);
        }
}

/*
 * The same decode over a cache whose V is stored like K (the NPU issue page
 * on INT8 KV with per-head Hadamard rotation, part A: a rotated INT8 V needs
 * the transform applied once more to the output).  Reading taken: V rows are
 * rotated and quantized exactly as oracle_kv_quant does for K (one FP32 scale
 * per (head, token)), and since the normalized transform is its own inverse,
 * the output is that transform of the weighted sum of dequantized rows:
 *   r[d] = sum_t w_t * vscale[t] * v8[t, d]               (FP64)
 *   o    = (1/sqrt(D)) H r  (FP64 butterflies);  O = bf16(float(o))
 * with w the weights of oracle_decode_attn.  v8 [B, Hkv, Tc, D], vscale
 * [B, Hkv, Tc]; the other arguments as for oracle_decode_attn.
 * Pinned by: one token gives back the stored row within the quantization
 * bound, constant V rows give that row for any weights, and the weights equal
 * those of oracle_decode_attn.
 */
void oracle_decode_attn_v8(int B, int Hq, int Hkv, int D, int T, int Tc, const uint16_t *q,
                           const int8_t *k8, const float *kscale, const int8_t *v8, const float *vscale,
                           uint16_t *o, double *w)
{
    const int grp = Hq / Hkv;
    double *wt = (double *)malloc(sizeof(double) * (size_t)B * Hq * (T > 0 ? T : 1));
    uint16_t *unused = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)B * Hq * D);
    uint16_t *vzero = (uint16_t *)calloc((size_t)B * Hkv * Tc * D, sizeof(uint16_t));
    oracle_decode_attn(B, Hq, Hkv, D, T, Tc, q, k8, kscale, vzero, unused, wt);
    free(vzero);
    free(unused);
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < Hq; h++) {
            const int64_t base = ((int64_t)b * Hkv + h / grp) * Tc;
            const double *wr = wt + ((int64_t)b * Hq + h) * T;
            double *r = (double *)calloc(D, sizeof(double));
            for (int t = 0; t < T; t++) {
                const int8_t *vr = v8 + (base + t) * D;
                for (int d = 0; d < D; d++) r[d] += wr[t] * (double)vscale[base + t] * (double)vr[d];
            }
            for (int span = 1; span < D; span *= 2)
                for (int i = 0; i < D; i += 2 * span)
                    for (int j = i; j < i + span; j++) {
                        const double a = r[j], c = r[j + span];
                        r[j] = a + c;
                        r[j + span] = a - c;
                    }
            for (int d = 0; d < D; d++)
                o[((int64_t)b * Hq + h) * D + d] = oracle_f32_to_bf16((float)(r[d] / sqrt((double)D)));
            free(r);
        }
    if (w) memcpy(w, wt, sizeof(double) * (size_t)B * Hq * T);
    free(wt);
}

/* Number of OpenMP threads the oracle runs with (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Bulk conversions over arrays, for the exhaustive format tables in tests. */
void oracle_f32_to_bf16_n(const float *x, uint16_t *y, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) y[i] = oracle_f32_to_bf16(x[i]);
}
void oracle_f32_to_e4m3_n(const float *x, uint8_t *y, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) y[i] = oracle_f32_to_e4m3(x[i]);
}
void oracle_f32_to_i8_n(const float *x, int8_t *y, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) y[i] = oracle_f32_to_i8(x[i]);
}
void oracle_exp2_n(const float *x, float *y, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) y[i] = oracle_exp2(x[i]);
}
void oracle_wht_n(float *u, int64_t rows, int D)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) oracle_wht(u + r * D, D);
}
