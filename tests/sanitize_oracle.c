/* Drives every entry point of oracle/sage_oracle.c on small and edge shapes so
 * that a build with AddressSanitizer and UndefinedBehaviorSanitizer can check
 * the oracle's indexing and arithmetic (test infrastructure; built and run by
 * tests/test_oracle_sanitized.py).  Every buffer is allocated with exactly the
 * size the oracle's Python wrapper gives it, so an access past its end lands
 * in the sanitizer's redzone.  Prints "sanitize_oracle ok" at the end. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_f32_to_bf16(float x);
void oracle_rmsnorm_rope(int B, int N, int H, int D, int R, float eps, const uint16_t *x, int64_t sb, int64_t sn,
                         int64_t sh, const uint16_t *w, const uint16_t *cosr, const uint16_t *sinr, uint16_t *z);
void oracle_k_mean(int B, int H, int N, int D, const uint16_t *zk, float *mean);
void oracle_quant_q(int B, int H, int N, int D, int hadamard, const uint16_t *zq, int8_t *q8, float *q_scale);
void oracle_quant_k(int B, int H, int N, int D, int hadamard, const uint16_t *zk, const float *mean, int8_t *k8,
                    float *k_scale);
void oracle_quant_v(int B, int N, int H, int D, const uint16_t *v, int64_t sb, int64_t sn, int64_t sh, uint8_t *v8,
                    float *v_scale);
void oracle_attn_rows_mode(int B, int N, int Hq, int Hkv, int D, const int8_t *q8, const float *q_scale,
                           const int8_t *k8, const float *k_scale, const uint8_t *v8, const float *v_scale,
                           int64_t nrows, const int32_t *rows, uint16_t *o, int pv_fp16);
void oracle_attn_rows_segmented(int B, int N, int Hq, int Hkv, int D, const int8_t *q8, const float *q_scale,
                                const int8_t *k8, const float *k_scale, const uint8_t *v8, const float *v_scale,
                                int64_t nrows, const int32_t *rows, int nseg, uint16_t *o);
void oracle_kv_quant(int B, int T, int H, int D, const uint16_t *k, int64_t sb, int64_t sn, int64_t sh, int8_t *k8,
                     float *kscale);
void oracle_decode_attn(int B, int Hq, int Hkv, int D, int T, int Tc, const uint16_t *q, const int8_t *k8,
                        const float *kscale, const uint16_t *v, uint16_t *o, double *w);
void oracle_decode_attn_v8(int B, int Hq, int Hkv, int D, int T, int Tc, const uint16_t *q, const int8_t *k8,
                           const float *kscale, const int8_t *v8, const float *vscale, uint16_t *o, double *w);

static uint64_t rng = 0x9E3779B97F4A7C15ull;

static float uniform(void)          /* [-2, 2) */
{
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((double)(rng >> 11) / 9007199254740992.0 * 4.0 - 2.0);
}

static uint16_t *bf16_array(size_t n)
{
    uint16_t *a = malloc(n * sizeof *a);
    for (size_t i = 0; i < n; i++) a[i] = oracle_f32_to_bf16(uniform());
    return a;
}

static void prefill(int B, int N, int Hq, int Hkv, int D, int R, int hadamard, int inf_q)
{
    const int half = R / 2, nq = ((N + 127) / 128) * 4, nk = (N + 63) / 64;
    uint16_t *q = bf16_array((size_t)B * N * Hq * D), *k = bf16_array((size_t)B * N * Hkv * D);
    uint16_t *v = bf16_array((size_t)B * N * Hkv * D), *w = bf16_array((size_t)D);
    uint16_t *cs = bf16_array((size_t)N * half), *sn = bf16_array((size_t)N * half);
    if (inf_q) q[(size_t)(N / 2) * Hq * D + 3] = 0x7f80;                 /* +Inf */
    uint16_t *zq = malloc((size_t)B * Hq * N * D * 2), *zk = malloc((size_t)B * Hkv * N * D * 2);
    float *mean = malloc((size_t)B * Hkv * D * 4);
    int8_t *q8 = calloc((size_t)B * Hq * N * D, 1), *k8 = calloc((size_t)B * Hkv * N * D, 1);
    float *qs = malloc((size_t)B * Hq * nq * 4), *ks = malloc((size_t)B * Hkv * nk * 4);
    uint8_t *v8 = malloc((size_t)B * Hkv * N * D);
    float *vs = malloc((size_t)B * Hkv * D * 4);
    oracle_rmsnorm_rope(B, N, Hq, D, R, 1e-5f, q, (int64_t)N * Hq * D, (int64_t)Hq * D, D, w, cs, sn, zq);
    oracle_rmsnorm_rope(B, N, Hkv, D, R, 1e-5f, k, (int64_t)N * Hkv * D, (int64_t)Hkv * D, D, w, cs, sn, zk);
    oracle_k_mean(B, Hkv, N, D, zk, mean);
    oracle_quant_q(B, Hq, N, D, hadamard, zq, q8, qs);
    oracle_quant_k(B, Hkv, N, D, hadamard, zk, mean, k8, ks);
    oracle_quant_v(B, N, Hkv, D, v, (int64_t)N * Hkv * D, (int64_t)Hkv * D, D, v8, vs);

    const int64_t nrows = (int64_t)B * Hq * N;
    int32_t *rows = malloc((size_t)nrows * 3 * 4);
    int64_t r = 0;
    for (int b = 0; b < B; b++)
        for (int h = 0; h < Hq; h++)
            for (int i = 0; i < N; i++, r++) {
                rows[3 * r] = b; rows[3 * r + 1] = h; rows[3 * r + 2] = i;
            }
    uint16_t *o = malloc((size_t)nrows * D * 2);
    oracle_attn_rows_mode(B, N, Hq, Hkv, D, q8, qs, k8, ks, v8, vs, nrows, rows, o, 0);
    oracle_attn_rows_mode(B, N, Hq, Hkv, D, q8, qs, k8, ks, v8, vs, nrows, rows, o, 1);
    const int segs[3] = {1, 2, nk};
    for (int s = 0; s < 3; s++)
        oracle_attn_rows_segmented(B, N, Hq, Hkv, D, q8, qs, k8, ks, v8, vs, nrows, rows, segs[s], o);
    free(q); free(k); free(v); free(w); free(cs); free(sn); free(zq); free(zk); free(mean);
    free(q8); free(k8); free(qs); free(ks); free(v8); free(vs); free(rows); free(o);
}

static void decode(int B, int Hq, int Hkv, int Tc)
{
    const int D = 256;
    uint16_t *k = bf16_array((size_t)B * Tc * Hkv * D), *vc = bf16_array((size_t)B * Hkv * Tc * D);
    uint16_t *q = bf16_array((size_t)B * Hq * D);
    int8_t *k8 = malloc((size_t)B * Hkv * Tc * D);
    float *ks = malloc((size_t)B * Hkv * Tc * 4);
    oracle_kv_quant(B, Tc, Hkv, D, k, (int64_t)Tc * Hkv * D, (int64_t)Hkv * D, D, k8, ks);
    int8_t *v8 = malloc((size_t)B * Hkv * Tc * D);
    float *vs = malloc((size_t)B * Hkv * Tc * 4);
    /* the V cache [B, Hkv, Tc, D] read as rows [B, T, H, D] with strides */
    oracle_kv_quant(B, Tc, Hkv, D, vc, (int64_t)Hkv * Tc * D, D, (int64_t)Tc * D, v8, vs);
    uint16_t *o = malloc((size_t)B * Hq * D * 2);
    const int Ts[3] = {1, Tc / 2 + 1, Tc};
    for (int i = 0; i < 3; i++) {
        double *w = malloc((size_t)B * Hq * Ts[i] * sizeof(double));
        oracle_decode_attn(B, Hq, Hkv, D, Ts[i], Tc, q, k8, ks, vc, o, w);
        oracle_decode_attn_v8(B, Hq, Hkv, D, Ts[i], Tc, q, k8, ks, v8, vs, o, w);
        free(w);
    }
    free(k); free(vc); free(q); free(k8); free(ks); free(v8); free(vs); free(o);
}

int main(void)
{
    prefill(1, 1, 1, 1, 128, 96, 0, 0);        /* one query, one key */
    prefill(1, 65, 2, 1, 128, 0, 0, 0);        /* ragged tile, no RoPE, grouped heads */
    prefill(2, 130, 4, 2, 256, 192, 1, 0);     /* D = 256 with the rotation, batch 2 */
    prefill(1, 200, 2, 2, 128, 40, 0, 1);      /* RoPE half-width not a multiple of 8; an Inf */
    prefill(1, 64, 2, 2, 256, 256, 0, 0);      /* RoPE over every dimension */
    decode(2, 4, 2, 40);
    decode(1, 16, 1, 9);
    printf("sanitize_oracle ok\n");
    return 0;
}
