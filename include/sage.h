/*
 * sage.h -- C ABI of the MI355X (gfx950) quantized attention forward.
 *
 * The path computes the SageAttention-style INT8-QK / FP8-PV attention fixed by
 * the page "Exact Numerical Contract":
 *   sage_prep      section "Preparation" steps 1-4 (RMSNorm, RoPE, global K
 *                  mean) and the V maximum of section "V And PV";
 *   sage_quant_qk  section "Q And K Quantization" (INT8 Q per 32 rows, INT8 K
 *                  per 64 rows after mean subtraction) and the FP8 V cast of
 *                  section "V And PV";
 *   sage_attn_fwd  sections "INT8 QK And Score Domain", "Online Softmax",
 *                  "V And PV" and "Finalization And Tails".
 * Inputs follow the page's section "Canonical Boundary": BF16 Q/K/V in NHD
 * order given as strided views (so the interleaved QKV row of width 21,504 at
 * offsets 0 / 7,168 / 14,336 is accepted as is); the output is BF16 NHD,
 * contiguous in (head, dim) so that [N, H*D] is a free reshape.
 *
 * Optional rotation: with hadamard = 1, Q and mean-subtracted K rows are
 * multiplied by the normalized Walsh-Hadamard matrix before INT8
 * quantization (the NPU issue page on INT8 KV with per-head Hadamard
 * rotation: the rotation cancels in Q K^T).
 *
 * Ownership and threading: the caller allocates every device buffer (sizes
 * from sage_buffer_sizes) and the workspace.  The library never allocates,
 * frees or synchronises; it enqueues kernels on the given HIP stream (NULL is
 * the default stream) and returns.  Calls are reentrant; calls that share
 * buffers must be ordered by the caller (same stream).  sage_quant_qk must run
 * after sage_prep on the same buffers and workspace; sage_attn_fwd after
 * sage_quant_qk.
 *
 * Errors: every argument is validated before any launch.  On a refusal the
 * named status is returned and nothing is written.  A failed launch returns
 * SAGE_E_HIP.  There is no fallback path.
 */
#ifndef SAGE_H_
#define SAGE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sage_status {
    SAGE_OK = 0,
    SAGE_E_NULL = 1,         /* a required pointer is NULL                              */
    SAGE_E_SHAPE = 2,        /* B, N, Hq, Hkv or D out of range                         */
    SAGE_E_STRIDE = 3,       /* unit d stride missing, or output not contiguous in (h,d) */
    SAGE_E_ALIGN = 4,        /* a row or buffer start is not 16-byte aligned            */
    SAGE_E_ROPE = 5,         /* rope_dim odd, negative or above D                       */
    SAGE_E_GQA = 6,          /* Hq is not a multiple of Hkv                             */
    SAGE_E_WORKSPACE = 7,    /* workspace missing or smaller than sage_buffer_sizes     */
    SAGE_E_UNSUPPORTED = 8,  /* e.g. hadamard with D = 128, eps not positive            */
    SAGE_E_HIP = 9           /* a kernel launch failed                                  */
} sage_status;

/* Problem shape.
 *   B, N      batch and sequence length (1 <= N <= 2^24)
 *   Hq, Hkv   query and key/value heads; query head h reads KV head h/(Hq/Hkv);
 *             every launch must fit one dispatch of at most 2^32 - 1
 *             work-items along its grid's x dimension, else SAGE_E_SHAPE:
 *             ceil(N/128) * Hq * B * 256 (512 for D = 256) and
 *             (ceil(N/128) * Hq + ceil(N/64) * Hkv) * 256
 *   D         head dimension, 128 or 256
 *   rope_dim  R: split-half RoPE rotates dims [0, R) in pairs (i, i + R/2);
 *             even, 0 <= R <= D (96 for D = 128 on the contract page)
 *   hadamard  0 or 1 (1 requires D = 256)
 *   eps       RMSNorm epsilon (1e-5 on the contract page), > 0              */
typedef struct sage_shape {
    int32_t B, N, Hq, Hkv, D;
    int32_t rope_dim;
    int32_t hadamard;
    float eps;
} sage_shape;

/* A read-only BF16 tensor view of logical shape [B, N, H, D].  Element
 * (b, n, h, d) lives at ptr + 2 * (b*sb + n*sn + h*sh + d*sd) bytes.  sd must
 * be 1; ptr must be 16-byte aligned and sb, sn, sh multiples of 8 elements. */
typedef struct sage_view_bf16 {
    const void *ptr;
    int64_t sb, sn, sh, sd;
} sage_view_bf16;

/* Device buffers written by sage_prep / sage_quant_qk and read by
 * sage_attn_fwd.  Layouts (row-major, sizes from sage_buffer_sizes):
 *   q8       INT8 [B, Hq, q_rows, D]; rows >= N are zero
 *   q_scale  FP32 [B, Hq, n_q_groups], n_q_groups = ceil(N/128)*4; scale of
 *            query rows [32g, 32g+32); groups without a valid row hold 1e-7/127
 *   k8       INT8 [B, Hkv, k_rows, D], k_rows = 64 * n_k_tiles; rows >= N zero
 *   k_scale  FP32 [B, Hkv, n_k_tiles], n_k_tiles = ceil(N/64)
 *   k_mean   FP32 [B, Hkv, D], the global K mean subtracted before quantization
 *   v8       OCP E4M3 [B, Hkv, n_k_tiles, D, 64]: tile t, channel d holds the
 *            64 keys of the tile in the order sage_v8_key_of_slot gives; keys
 *            >= N are zero
 *   v_scale  FP32 [B, Hkv, D]
 *   q_prep   optional (NULL = not written) BF16 [B, Hq, N, D]: Q after RMSNorm
 *            and RoPE ("Preparation" steps 1-3), before any rotation; written
 *            by sage_quant_qk
 *   k_prep   optional (NULL = not written) BF16 [B, Hkv, N, D]: K after
 *            RMSNorm and RoPE, before mean subtraction and rotation; written
 *            by sage_quant_qk                                                 */
typedef struct sage_bufs {
    int8_t *q8;
    float *q_scale;
    int8_t *k8;
    float *k_scale;
    float *k_mean;
    uint8_t *v8;
    float *v_scale;
    uint16_t *q_prep;
    uint16_t *k_prep;
} sage_bufs;

/* Byte sizes of each buffer of sage_bufs and of the workspace, plus the
 * padded extents of the layouts above. */
typedef struct sage_sizes {
    size_t q8, q_scale, k8, k_scale, k_mean, v8, v_scale, workspace;
    int64_t q_rows, n_q_groups, k_rows, n_k_tiles;
} sage_sizes;

/* Validates *shape and fills *out.  Returns SAGE_E_NULL / SAGE_E_SHAPE /
 * SAGE_E_ROPE / SAGE_E_GQA / SAGE_E_UNSUPPORTED on an invalid shape. */
sage_status sage_buffer_sizes(const sage_shape *shape, sage_sizes *out);

/* Pass 1 ("Preparation" steps 1-4; V maximum of "V And PV").
 *   q, k, v     BF16 views, Q [B,N,Hq,D], K and V [B,N,Hkv,D] (device memory)
 *   w_q, w_k    BF16 [D] RMSNorm weights shared by all heads, NULL = ones
 *   rope_cos/sin BF16 [N, rope_dim/2] (row stride rope_dim/2) coefficients for
 *               positions 0..N-1; may be NULL when rope_dim == 0
 *   bufs        k_mean and v_scale are written; q8..v8 untouched
 *   workspace   device memory of at least sizes.workspace bytes; holds per-tile
 *               partial sums and maxima that sage_quant_qk reads
 *   stream      hipStream_t, NULL = default stream
 * Q is validated but not read here. */
sage_status sage_prep(const sage_shape *shape, const sage_view_bf16 *q, const sage_view_bf16 *k,
                      const sage_view_bf16 *v, const uint16_t *w_q, const uint16_t *w_k,
                      const uint16_t *rope_cos, const uint16_t *rope_sin, const sage_bufs *bufs,
                      void *workspace, size_t ws_bytes, void *stream);

/* Pass 2 ("Q And K Quantization"; FP8 cast of "V And PV").  Same arguments as
 * sage_prep.  Recomputes RMSNorm + RoPE (+ rotation) bit-identically to pass 1,
 * subtracts k_mean from K, and writes q8, q_scale, k8, k_scale and v8
 * (including zero padding rows), and q_prep / k_prep when they are not NULL
 * (16-byte aligned, else SAGE_E_ALIGN). */
sage_status sage_quant_qk(const sage_shape *shape, const sage_view_bf16 *q, const sage_view_bf16 *k,
                          const sage_view_bf16 *v, const uint16_t *w_q, const uint16_t *w_k,
                          const uint16_t *rope_cos, const uint16_t *rope_sin, const sage_bufs *bufs,
                          void *workspace, size_t ws_bytes, void *stream);

/* Fused attention ("INT8 QK And Score Domain" through "Finalization And
 * Tails"): INT8 QK^T on MFMA, base-2 online softmax over the KV tiles in
 * increasing order, E4M3 P times E4M3 V on MFMA, 1/d normalisation, BF16 out.
 *   o            BF16 [B, N, Hq, D] output, element (b,n,h,d) at
 *                o + 2*(b*osb + n*osn + h*osh + d); osh must equal D and osn
 *                Hq*D (rows reshapeable to [N, Hq*D]); 16-byte aligned.
 * Only rows n < N are written. */
sage_status sage_attn_fwd(const sage_shape *shape, const sage_bufs *bufs, void *o, int64_t osb,
                          int64_t osn, int64_t osh, void *stream);

/* Measurement variant of sage_attn_fwd: the same launch and output, and in
 * addition the first wave of every work-group reads the shader-clock counter
 * (s_memtime) and the constant-rate counter (s_memrealtime) when it starts
 * and when it ends, and writes the four values (uint64: clock at start, wall
 * at start, clock at end, wall at end) to stamps + 4 * (work-group index).
 * Cycles over wall ticks, times the constant counter's rate
 * (sage_wall_clock_khz), is the shader clock the launch ran at.
 *   stamps       device memory, 16-byte aligned, of at least
 *                sage_attn_stamp_bytes bytes (32 for every 32 query rows
 *                of every head: B * Hq * ceil(N/32) records, at least one
 *                per work-group of any launch; records past the launch's
 *                work-groups are not written)
 * Refusals: those of sage_attn_fwd, SAGE_E_NULL, SAGE_E_WORKSPACE (stamps
 * too small), SAGE_E_ALIGN. */
sage_status sage_attn_stamp_bytes(const sage_shape *shape, size_t *bytes);
sage_status sage_attn_fwd_stamped(const sage_shape *shape, const sage_bufs *bufs, void *o, int64_t osb,
                                  int64_t osn, int64_t osh, uint64_t *stamps, size_t stamp_bytes, void *stream);

/* Rate of the constant-rate counter of the current device, in kHz
 * (hipDeviceAttributeWallClockRate).  SAGE_E_NULL, SAGE_E_HIP. */
sage_status sage_wall_clock_khz(int32_t *khz);

/* Segmented (split-KV) attention: an opt-in mode that is NOT the exact order
 * of sage_attn_fwd.  The contract page forbids combining KV partials; this
 * mode combines them, after the FP8-PV page's segmented schedules, to give
 * short sequences more work-groups.  The key tiles [0, nk) (nk = ceil(N/64))
 * are split into nseg contiguous runs, run s covering tiles
 * [s*nk/nseg, (s+1)*nk/nseg); each run performs the per-tile steps of
 * sage_attn_fwd from the initial state (RO = 0, m = -5e6, d = 1), and the
 * runs are combined in increasing s: M = max m_s, a_s = exp2(m_s - M),
 * d = sum d_s a_s, RO = sum RO_s a_s, O = bf16((RO * (1/d)) * v_scale).
 * With nseg = 1 the result is bit-identical to sage_attn_fwd.
 *   nseg       1 <= nseg <= ceil(N/64)
 *   o, osb, osn, osh   as for sage_attn_fwd
 *   workspace  device memory of at least sage_attn_segmented_workspace bytes,
 *              16-byte aligned: the runs' FP32 partials (RO, m, d)
 * Refusals: those of sage_attn_fwd, SAGE_E_SHAPE (nseg out of range, or
 * ceil(N/128) * nseg * Hq * B * 256 (512 for D = 256) >= 2^32 work-items),
 * SAGE_E_WORKSPACE,
 * SAGE_E_ALIGN (workspace). */
sage_status sage_attn_segmented_workspace(const sage_shape *shape, int32_t nseg, size_t *bytes);
sage_status sage_attn_fwd_segmented(const sage_shape *shape, const sage_bufs *bufs, int32_t nseg, void *o,
                                    int64_t osb, int64_t osn, int64_t osh, void *workspace, size_t ws_bytes,
                                    void *stream);

/* ------------------------------------------------------------------------
 * Decode-time INT8 K cache (the NPU issue page on INT8 KV with per-head
 * Hadamard rotation, part A, the variant with INT8 K and 16-bit V): every K
 * row is multiplied by the normalized Walsh-Hadamard matrix and stored as
 * INT8 with one FP32 scale per (head, token); the query is rotated by the
 * same matrix, which leaves every score unchanged because the matrix is
 * orthogonal.  V is kept in BF16.  Head width D = 256 only.
 * ------------------------------------------------------------------------ */

/* The cache, owned by the caller (device memory, 16-byte aligned, capacity a
 * multiple of 8):
 *   k8       INT8 [B, Hkv, capacity, D]          rotated K rows
 *   k_scale  FP32 [B, Hkv, capacity]             amax / 127 of each rotated row
 *   v        BF16 [B, Hkv, capacity / 8, D, 8]   V in blocks of 8 tokens per
 *            channel: token t, channel d of a (batch, KV head) at
 *            ((t / 8) * D + d) * 8 + t % 8
 * or, for a cache with INT8 V (v NULL; the same page: a rotated INT8 V needs
 * the transform once more on the output, which the decode applies):
 *   v8       INT8 [B, Hkv, capacity / 8, D, 8]   rotated V rows, quantized as
 *            the K rows are, in the same 8-token blocks per channel
 *   v_scale  FP32 [B, Hkv, capacity]             amax / 127 of each rotated
 *            V row
 * Exactly one of v and v8 is set; v_scale goes with v8.                      */
typedef struct sage_kv_cache {
    int8_t *k8;
    float *k_scale;
    uint16_t *v;
    int32_t B, Hkv, D, capacity;
    int8_t *v8;
    float *v_scale;
} sage_kv_cache;

/* Writes n new tokens at cache positions [t0, t0 + n): per row (b, t, h) of
 * the BF16 views k and v ([B, n, Hkv, D], unit d stride, 16-byte aligned
 * rows), u = H k / 16, k_scale = max(1e-7, max|u|) / 127,
 * k8 = round-half-even-saturate(u * (127 / max(1e-7, max|u|))), v copied
 * into its blocks, or with INT8 V rotated and quantized by the same formulas
 * into v8 and v_scale (the other tokens of a partly written block keep their
 * values).
 * Refusals: SAGE_E_NULL (also: both or neither of v and v8 set, or v8
 * without v_scale), SAGE_E_UNSUPPORTED (D != 256), SAGE_E_SHAPE
 * (B, Hkv, capacity not a multiple of 8, n < 1, t0 < 0,
 * t0 + n > capacity, or more than 2^26 - 1 blocks of 8 tokens times Hkv,
 * the work-items one dispatch holds), SAGE_E_STRIDE,
 * SAGE_E_ALIGN, SAGE_E_HIP. */
sage_status sage_kv_append(const sage_kv_cache *cache, const sage_view_bf16 *k, const sage_view_bf16 *v,
                           int32_t t0, int32_t n, void *stream);

/* Workspace bytes of sage_decode_attn for Hq query heads over T tokens. */
sage_status sage_decode_workspace(const sage_kv_cache *cache, int32_t Hq, int32_t T, size_t *bytes);

/* Single-query attention of each of the Hq query heads (view q [B, 1, Hq, D])
 * over cache positions [0, T) of KV head h / (Hq / Hkv):
 *   s_t = ((H q / 16) . k8_t) * k_scale_t / 16,  w = softmax(s),
 *   o = bf16(sum_t w_t v_t)
 * or with INT8 V:  o = bf16((H / 16) sum_t w_t v_scale_t v8_t)
 * o: BF16 [B, Hq, D] contiguous.  The cache is read once: the work-group of
 * one KV head and a chunk of 128 * ns tokens (ns in 1..16, set from the cache
 * size so that the step has about 512 work-groups) serves its Hq / Hkv query
 * heads on the matrix cores (exact INT32 dot products of K with a three-part
 * INT8 expansion of the rotated query; BF16 V times a two-part BF16 split of
 * the weights, FP32 accumulation), and the chunk partials are combined in a
 * fixed order (deterministic).
 * Refusals: SAGE_E_NULL, SAGE_E_UNSUPPORTED (D != 256, Hq / Hkv > 16),
 * SAGE_E_GQA, SAGE_E_SHAPE (T < 1 or T > capacity),
 * SAGE_E_STRIDE, SAGE_E_ALIGN, SAGE_E_WORKSPACE, SAGE_E_HIP. */
sage_status sage_decode_attn(const sage_kv_cache *cache, int32_t Hq, const sage_view_bf16 *q, int32_t T,
                             void *o, void *workspace, size_t ws_bytes, void *stream);

/* Allocation-free variant of sage_decode_attn, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and output, with the
 * chunk partials kept in a fixed array that the library holds on each GPU it
 * runs on (sage_decode_noalloc_max_bytes() bytes, 16 MiB, kept until the
 * process ends) instead of a caller workspace.  The call itself allocates
 * nothing.  Every call on a GPU shares that GPU's array: calls that overlap
 * on one GPU (different streams, no ordering between them) race and may
 * return wrong outputs; calls ordered on one stream are safe, since each call
 * writes every partial it reads.
 * Refusals: those of sage_decode_attn, and SAGE_E_WORKSPACE when the call's
 * partials (sage_decode_workspace bytes) exceed the array. */
sage_status sage_decode_attn_noalloc(const sage_kv_cache *cache, int32_t Hq, const sage_view_bf16 *q, int32_t T,
                                     void *o, void *stream);

/* Size in bytes of the fixed per-GPU array of sage_decode_attn_noalloc. */
size_t sage_decode_noalloc_max_bytes(void);

/* Test hook: applies one device number-format primitive of the preparation
 * kernels, in the exact form they use, to the FP32 values whose bit patterns
 * are first, first + 1, ..., first + count - 1, and writes the results to out
 * (device memory, 16-byte aligned), element i for pattern first + i:
 *   kind 0  BF16, round to nearest even                 uint16 [count]
 *   kind 1  INT8, round to nearest even, saturate,      int8   [count]
 *           NaN -> 0
 *   kind 2  OCP E4M3, round to nearest even, saturate   uint8  [count]
 *           to +-448, NaN -> 0x7F / 0xFF
 *   kind 3  RMSNorm reciprocal 1.0f / sqrtf(x)          float  [count]
 *   kind 4  x / 127.0f (quantization scale)             float  [count]
 *   kind 5  127.0f / x (quantization multiplier)        float  [count]
 *   kind 6  x / 2.25f (V scale)                         float  [count]
 *   kind 7  2.25f / x (V multiplier)                    float  [count]
 *   kind 8  2^x as the attention kernel's softmax       float  [count]
 *           computes it (v_exp_f32)
 *   kind 9  OCP E4M3 as the V cast converts (hardware  uint8  [count]
 *           conversion; equal to kind 2 for |x| < 448
 *           and NaN; the V cast's values stay below 2.25)
 *   kind 10..15  the lane exchange of the preparation   float  [count]
 *           and decode reductions and butterflies at
 *           xor distance M = 2^(kind - 10): element i
 *           gets the input of element i ^ M (i within
 *           its wave of 64; count a multiple of 64)
 * For tests that compare these roundings with an independent implementation
 * over every FP32 pattern (Preparation; Q And K Quantization; V And PV), and
 * that measure the accuracy of the softmax exponential (Online Softmax).
 * Refusals: SAGE_E_NULL, SAGE_E_ALIGN, SAGE_E_UNSUPPORTED (kind outside
 * 0..15), SAGE_E_SHAPE (count < 1, count > 2^26, first + count > 2^32, or
 * for kinds 10..15 a count that is not a multiple of 64), SAGE_E_HIP. */
sage_status sage_selftest_primitive(int32_t kind, uint32_t first, uint32_t count, void *out, void *stream);

/* Key (0..63, within its tile) stored at position `slot` (0..63) of every
 * channel row of a v8 tile; -1 if slot is out of range. */
int32_t sage_v8_key_of_slot(int32_t slot);

/* Human-readable name of a status code (static string). */
const char *sage_status_str(sage_status status);

/* Library version, major*10000 + minor*100 + patch. */
int32_t sage_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H_ */
