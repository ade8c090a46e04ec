// api.hip -- host side of the C ABI declared in include/sage.h: argument
// validation, buffer sizing and kernel launches.  Never allocates, frees or
// synchronises; every refusal happens before the first launch.

#include "sage.h"
#include "device.h"
#include "decode.h"

#include <cmath>
#include <cstring>

// Defined in selftest.hip (the number-format test hook).
hipError_t sage_launch_primitive(int kind, uint32_t first, uint32_t count, void *out, hipStream_t s);

namespace {

constexpr int64_t kMaxN = int64_t(1) << 24;
// A dispatch holds its grid size in work-items as 32 bits per dimension.
constexpr int64_t kMaxItems = 4294967295LL;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

sage_status check_shape(const sage_shape *s) {
    if (!s) return SAGE_E_NULL;
    if (s->B < 1 || s->N < 1 || s->N > kMaxN || s->Hq < 1 || s->Hkv < 1) return SAGE_E_SHAPE;
    if (s->D != 128 && s->D != 256) return SAGE_E_SHAPE;
    if ((int64_t)s->B * s->Hq > 65535 * 64 || s->B > 65535 || s->Hq > 65535) return SAGE_E_SHAPE;
    // every launch fits one dispatch: the attention grid (ceil(N/128) * Hq * B
    // work-groups of 256 threads, 512 for D = 256) and the quantization grid
    // (ceil(N/128) * Hq + ceil(N/64) * Hkv work-groups of 256 threads per
    // batch row) hold at most kMaxItems work-items; the other preparation
    // grids are smaller
    const int64_t nqt = (s->N + 127) / 128, nkt = (s->N + 63) / 64;
    if (nqt * s->Hq * s->B * (s->D == 256 ? 512 : 256) > kMaxItems) return SAGE_E_SHAPE;
    if ((nqt * s->Hq + nkt * s->Hkv) * 256 > kMaxItems) return SAGE_E_SHAPE;
    if (s->Hq % s->Hkv != 0) return SAGE_E_GQA;
    if (s->rope_dim < 0 || s->rope_dim > s->D || (s->rope_dim & 1)) return SAGE_E_ROPE;
    if (s->hadamard != 0 && s->hadamard != 1) return SAGE_E_UNSUPPORTED;
    if (s->hadamard && s->D != 256) return SAGE_E_UNSUPPORTED;   // exact 1/sqrt(D) needs D = 4^k
    if (!(s->eps > 0.0f) || !std::isfinite(s->eps)) return SAGE_E_UNSUPPORTED;
    return SAGE_OK;
}

void fill_sizes(const sage_shape *s, sage_sizes *z) {
    const int64_t B = s->B, N = s->N, Hq = s->Hq, Hkv = s->Hkv, D = s->D;
    z->q_rows = ceil_div(N, 256) * 256;
    z->n_q_groups = ceil_div(N, 128) * 4;
    z->n_k_tiles = ceil_div(N, 64);
    z->k_rows = 64 * z->n_k_tiles;
    z->q8 = (size_t)(B * Hq * z->q_rows * D);
    z->q_scale = (size_t)(B * Hq * z->n_q_groups) * 4;
    z->k8 = (size_t)(B * Hkv * z->k_rows * D);
    z->k_scale = (size_t)(B * Hkv * z->n_k_tiles) * 4;
    z->k_mean = (size_t)(B * Hkv * D) * 4;
    z->v8 = (size_t)(B * Hkv * z->n_k_tiles * D * 64);
    z->v_scale = (size_t)(B * Hkv * D) * 4;
    const size_t part = round256((size_t)(B * Hkv * z->n_k_tiles * D) * 4);
    z->workspace = 2 * part + round256((size_t)(B * Hkv * D) * 4);
}

// A BF16 view: unit d stride, non-negative strides, 16-byte aligned rows.
// Its extent cannot be checked here; the caller owns that.
sage_status check_view(const sage_view_bf16 *v) {
    if (!v || !v->ptr) return SAGE_E_NULL;
    if (v->sd != 1) return SAGE_E_STRIDE;
    if (v->sb < 0 || v->sn < 0 || v->sh < 0) return SAGE_E_STRIDE;
    if (!aligned16(v->ptr) || (v->sb & 7) || (v->sn & 7) || (v->sh & 7)) return SAGE_E_ALIGN;
    return SAGE_OK;
}

sage_status check_bufs(const sage_bufs *b) {
    if (!b) return SAGE_E_NULL;
    if (!b->q8 || !b->q_scale || !b->k8 || !b->k_scale || !b->k_mean || !b->v8 || !b->v_scale)
        return SAGE_E_NULL;
    const void *all[] = {b->q8, b->q_scale, b->k8, b->k_scale, b->k_mean, b->v8, b->v_scale};
    for (const void *p : all)
        if (!aligned16(p)) return SAGE_E_ALIGN;
    return SAGE_OK;
}

sage_status build_prep(const sage_shape *shape, const sage_view_bf16 *q, const sage_view_bf16 *k,
                       const sage_view_bf16 *v, const uint16_t *w_q, const uint16_t *w_k,
                       const uint16_t *rope_cos, const uint16_t *rope_sin, const sage_bufs *bufs,
                       void *workspace, size_t ws_bytes, sage::PrepParams *p) {
    sage_status st = check_shape(shape);
    if (st != SAGE_OK) return st;
    if ((st = check_view(q)) != SAGE_OK) return st;
    if ((st = check_view(k)) != SAGE_OK) return st;
    if ((st = check_view(v)) != SAGE_OK) return st;
    if ((st = check_bufs(bufs)) != SAGE_OK) return st;
    if ((bufs->q_prep && !aligned16(bufs->q_prep)) || (bufs->k_prep && !aligned16(bufs->k_prep))) return SAGE_E_ALIGN;
    if (shape->rope_dim > 0 && (!rope_cos || !rope_sin)) return SAGE_E_NULL;
    if (shape->rope_dim > 0 && (shape->rope_dim / 2) % 8 == 0 && (!aligned16(rope_cos) || !aligned16(rope_sin)))
        return SAGE_E_ALIGN;
    if ((w_q && !aligned16(w_q)) || (w_k && !aligned16(w_k))) return SAGE_E_ALIGN;
    sage_sizes z;
    fill_sizes(shape, &z);
    if (!workspace) return SAGE_E_WORKSPACE;
    if (ws_bytes < z.workspace) return SAGE_E_WORKSPACE;
    if (!aligned16(workspace)) return SAGE_E_ALIGN;

    std::memset(p, 0, sizeof(*p));
    p->B = shape->B; p->N = shape->N; p->Hq = shape->Hq; p->Hkv = shape->Hkv; p->D = shape->D;
    p->R = shape->rope_dim; p->hadamard = shape->hadamard; p->eps = shape->eps;
    p->q = {static_cast<const uint16_t *>(q->ptr), q->sb, q->sn, q->sh};
    p->k = {static_cast<const uint16_t *>(k->ptr), k->sb, k->sn, k->sh};
    p->v = {static_cast<const uint16_t *>(v->ptr), v->sb, v->sn, v->sh};
    p->w_q = w_q; p->w_k = w_k; p->cos_t = rope_cos; p->sin_t = rope_sin;
    p->q8 = bufs->q8; p->q_scale = bufs->q_scale; p->k8 = bufs->k8; p->k_scale = bufs->k_scale;
    p->k_mean = bufs->k_mean; p->v8 = bufs->v8; p->v_scale = bufs->v_scale;
    p->q_prep = bufs->q_prep; p->k_prep = bufs->k_prep;
    const size_t part = round256((size_t)((int64_t)shape->B * shape->Hkv * z.n_k_tiles * shape->D) * 4);
    char *ws = static_cast<char *>(workspace);
    p->ws_ksum = reinterpret_cast<float *>(ws);
    p->ws_vmax = reinterpret_cast<float *>(ws + part);
    p->ws_vamax = reinterpret_cast<float *>(ws + 2 * part);
    p->q_rows = z.q_rows; p->k_rows = z.k_rows;
    p->nq = (int)z.n_q_groups; p->nk = (int)z.n_k_tiles;
    return SAGE_OK;
}

}  // namespace

extern "C" {

sage_status sage_buffer_sizes(const sage_shape *shape, sage_sizes *out) {
    if (!out) return SAGE_E_NULL;
    sage_status st = check_shape(shape);
    if (st != SAGE_OK) return st;
    fill_sizes(shape, out);
    return SAGE_OK;
}

sage_status sage_prep(const sage_shape *shape, const sage_view_bf16 *q, const sage_view_bf16 *k,
                      const sage_view_bf16 *v, const uint16_t *w_q, const uint16_t *w_k,
                      const uint16_t *rope_cos, const uint16_t *rope_sin, const sage_bufs *bufs,
                      void *workspace, size_t ws_bytes, void *stream) {
    sage::PrepParams p;
    sage_status st = build_prep(shape, q, k, v, w_q, w_k, rope_cos, rope_sin, bufs, workspace, ws_bytes, &p);
    if (st != SAGE_OK) return st;
    return sage_launch_prep_stats(p, static_cast<hipStream_t>(stream)) == hipSuccess ? SAGE_OK : SAGE_E_HIP;
}

sage_status sage_quant_qk(const sage_shape *shape, const sage_view_bf16 *q, const sage_view_bf16 *k,
                          const sage_view_bf16 *v, const uint16_t *w_q, const uint16_t *w_k,
                          const uint16_t *rope_cos, const uint16_t *rope_sin, const sage_bufs *bufs,
                          void *workspace, size_t ws_bytes, void *stream) {
    sage::PrepParams p;
    sage_status st = build_prep(shape, q, k, v, w_q, w_k, rope_cos, rope_sin, bufs, workspace, ws_bytes, &p);
    if (st != SAGE_OK) return st;
    return sage_launch_quant(p, static_cast<hipStream_t>(stream)) == hipSuccess ? SAGE_OK : SAGE_E_HIP;
}

namespace {

// Validates the arguments shared by the attention entry points and fills
// the kernel parameters (nseg = 1, no partials).
sage_status build_attn(const sage_shape *shape, const sage_bufs *bufs, void *o, int64_t osb, int64_t osn,
                       int64_t osh, sage::AttnParams *p) {
    sage_status st = check_shape(shape);
    if (st != SAGE_OK) return st;
    if ((st = check_bufs(bufs)) != SAGE_OK) return st;
    if (!o) return SAGE_E_NULL;
    if (osh != shape->D || osn != (int64_t)shape->Hq * shape->D || osb < 0) return SAGE_E_STRIDE;
    if (!aligned16(o) || (osb & 7)) return SAGE_E_ALIGN;
    sage_sizes z;
    fill_sizes(shape, &z);
    std::memset(p, 0, sizeof(*p));
    p->B = shape->B; p->N = shape->N; p->Hq = shape->Hq; p->Hkv = shape->Hkv;
    p->grp = shape->Hq / shape->Hkv;
    p->nq = (int)z.n_q_groups; p->nk = (int)z.n_k_tiles;
    p->q_rows = z.q_rows; p->k_rows = z.k_rows;
    p->c = (float)((1.0 / std::sqrt((double)shape->D)) * 1.4426950408889634073599246810019);
    p->q8 = bufs->q8; p->q_scale = bufs->q_scale; p->k8 = bufs->k8; p->k_scale = bufs->k_scale;
    p->v8 = bufs->v8; p->v_scale = bufs->v_scale;
    p->o = static_cast<uint16_t *>(o);
    p->osb = osb; p->osn = osn; p->osh = osh;
    p->nseg = 1;
    return SAGE_OK;
}

// Bytes of the segment partials: RO [B, Hq, nseg, N, D] FP32, then (m, d)
// [B, Hq, nseg, N, 2] FP32 at a 256-byte boundary; 0 if it overflows.
size_t seg_ro_bytes(const sage_shape *s, int32_t nseg) {
    const double rows = (double)s->B * s->Hq * nseg * s->N;
    if (rows * s->D * 4 > 9.0e18) return 0;
    return round256((size_t)s->B * s->Hq * nseg * s->N * s->D * 4);
}

sage_status check_nseg(const sage_shape *shape, int32_t nseg) {
    sage_sizes z;
    fill_sizes(shape, &z);
    if (nseg < 1 || nseg > z.n_k_tiles) return SAGE_E_SHAPE;
    // the two-launch form: 128 query rows per work-group and segment (the
    // one-work-group form checks its own grid and otherwise takes this one)
    const int64_t nqt = (shape->N + 127) / 128;
    if (nqt * nseg * shape->Hq * shape->B * (shape->D == 256 ? 512 : 256) > kMaxItems) return SAGE_E_SHAPE;
    if (seg_ro_bytes(shape, nseg) == 0) return SAGE_E_SHAPE;
    return SAGE_OK;
}

}  // namespace

sage_status sage_attn_fwd(const sage_shape *shape, const sage_bufs *bufs, void *o, int64_t osb,
                          int64_t osn, int64_t osh, void *stream) {
    sage::AttnParams p;
    sage_status st = build_attn(shape, bufs, o, osb, osn, osh, &p);
    if (st != SAGE_OK) return st;
    return sage_launch_attn(p, shape->D, static_cast<hipStream_t>(stream)) == hipSuccess ? SAGE_OK : SAGE_E_HIP;
}

sage_status sage_attn_stamp_bytes(const sage_shape *shape, size_t *bytes) {
    sage_status st = check_shape(shape);
    if (st != SAGE_OK) return st;
    if (!bytes) return SAGE_E_NULL;
    // one record per work-group; no launch has more than one work-group per
    // 32 query rows of a head
    *bytes = (size_t)shape->B * shape->Hq * (size_t)((shape->N + 31) / 32) * 4 * sizeof(uint64_t);
    return SAGE_OK;
}

sage_status sage_attn_fwd_stamped(const sage_shape *shape, const sage_bufs *bufs, void *o, int64_t osb,
                                  int64_t osn, int64_t osh, uint64_t *stamps, size_t stamp_bytes, void *stream) {
    sage::AttnParams p;
    sage_status st = build_attn(shape, bufs, o, osb, osn, osh, &p);
    if (st != SAGE_OK) return st;
    size_t need = 0;
    if ((st = sage_attn_stamp_bytes(shape, &need)) != SAGE_OK) return st;
    if (!stamps) return SAGE_E_NULL;
    if (stamp_bytes < need) return SAGE_E_WORKSPACE;
    if (!aligned16(stamps)) return SAGE_E_ALIGN;
    p.stamps = stamps;
    return sage_launch_attn(p, shape->D, static_cast<hipStream_t>(stream)) == hipSuccess ? SAGE_OK : SAGE_E_HIP;
}

sage_status sage_wall_clock_khz(int32_t *khz) {
    if (!khz) return SAGE_E_NULL;
    int dev = 0, rate = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SAGE_E_HIP;
    if (hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return SAGE_E_HIP;
    *khz = rate;
    return SAGE_OK;
}

sage_status sage_attn_segmented_workspace(const sage_shape *shape, int32_t nseg, size_t *bytes) {
    sage_status st = check_shape(shape);
    if (st != SAGE_OK) return st;
    if (!bytes) return SAGE_E_NULL;
    if ((st = check_nseg(shape, nseg)) != SAGE_OK) return st;
    *bytes = seg_ro_bytes(shape, nseg) + round256((size_t)shape->B * shape->Hq * nseg * shape->N * 2 * 4);
    return SAGE_OK;
}

sage_status sage_attn_fwd_segmented(const sage_shape *shape, const sage_bufs *bufs, int32_t nseg, void *o,
                                    int64_t osb, int64_t osn, int64_t osh, void *workspace, size_t ws_bytes,
                                    void *stream) {
    sage::AttnParams p;
    sage_status st = build_attn(shape, bufs, o, osb, osn, osh, &p);
    if (st != SAGE_OK) return st;
    size_t need = 0;
    if ((st = sage_attn_segmented_workspace(shape, nseg, &need)) != SAGE_OK) return st;
    if (!workspace || ws_bytes < need) return SAGE_E_WORKSPACE;
    if (!aligned16(workspace)) return SAGE_E_ALIGN;
    p.nseg = nseg;
    p.seg_ro = static_cast<float *>(workspace);
    p.seg_md = reinterpret_cast<float *>(static_cast<char *>(workspace) + seg_ro_bytes(shape, nseg));
    return sage_launch_attn_segmented(p, shape->D, static_cast<hipStream_t>(stream)) == hipSuccess ? SAGE_OK
                                                                                                  : SAGE_E_HIP;
}

namespace {

sage_status check_cache(const sage_kv_cache *c) {
    if (!c || !c->k8 || !c->k_scale) return SAGE_E_NULL;
    if ((c->v != nullptr) == (c->v8 != nullptr) || (c->v8 && !c->v_scale)) return SAGE_E_NULL;
    if (c->D != 256) return SAGE_E_UNSUPPORTED;
    if (c->B < 1 || c->B > 65535 || c->Hkv < 1 || c->capacity < 1) return SAGE_E_SHAPE;
    if (c->capacity % sage::kVBlock != 0) return SAGE_E_SHAPE;
    if ((int64_t)c->B * c->Hkv * c->capacity > (int64_t(1) << 34)) return SAGE_E_SHAPE;
    if (!aligned16(c->k8) || !aligned16(c->k_scale)) return SAGE_E_ALIGN;
    if (c->v ? !aligned16(c->v) : (!aligned16(c->v8) || !aligned16(c->v_scale))) return SAGE_E_ALIGN;
    return SAGE_OK;
}

}  // namespace

sage_status sage_kv_append(const sage_kv_cache *cache, const sage_view_bf16 *k, const sage_view_bf16 *v,
                           int32_t t0, int32_t n, void *stream) {
    sage_status st = check_cache(cache);
    if (st != SAGE_OK) return st;
    if ((st = check_view(k)) != SAGE_OK) return st;
    if ((st = check_view(v)) != SAGE_OK) return st;
    if (n < 1 || t0 < 0 || (int64_t)t0 + n > cache->capacity) return SAGE_E_SHAPE;
    const int64_t nblk = ((int64_t)t0 + n - 1) / sage::kVBlock - t0 / sage::kVBlock + 1;
    // (nblk * Hkv + 3) / 4 work-groups of 256 threads
    if ((nblk * cache->Hkv + 3) / 4 * 256 > kMaxItems) return SAGE_E_SHAPE;
    sage::KvAppendParams p;
    std::memset(&p, 0, sizeof(p));
    p.B = cache->B; p.Hkv = cache->Hkv; p.D = cache->D; p.n = n; p.t0 = t0; p.cap = cache->capacity;
    p.nblk = (int)nblk;
    p.k = sage::View{static_cast<const uint16_t *>(k->ptr), k->sb, k->sn, k->sh};
    p.v = sage::View{static_cast<const uint16_t *>(v->ptr), v->sb, v->sn, v->sh};
    p.k8 = cache->k8; p.k_scale = cache->k_scale; p.vc = cache->v;
    if (!cache->v) { p.v8c = cache->v8; p.v_scale = cache->v_scale; }
    return sage_launch_kv_append(p, static_cast<hipStream_t>(stream)) == hipSuccess ? SAGE_OK : SAGE_E_HIP;
}

sage_status sage_decode_workspace(const sage_kv_cache *cache, int32_t Hq, int32_t T, size_t *bytes) {
    sage_status st = check_cache(cache);
    if (st != SAGE_OK) return st;
    if (!bytes) return SAGE_E_NULL;
    if (Hq < 1 || T < 1 || T > cache->capacity) return SAGE_E_SHAPE;
    *bytes = round256((size_t)sage::decode_ws_bytes(cache->B, Hq, cache->Hkv, T));
    return SAGE_OK;
}

namespace {

// Validates the arguments shared by the decode entry points and fills the
// kernel parameters (all but the partials buffer); *need gets the bytes of
// chunk partials the call writes.
sage_status build_decode(const sage_kv_cache *cache, int32_t Hq, const sage_view_bf16 *q, int32_t T, void *o,
                         sage::DecodeParams *p, size_t *need) {
    sage_status st = check_cache(cache);
    if (st != SAGE_OK) return st;
    if ((st = check_view(q)) != SAGE_OK) return st;
    if (!o) return SAGE_E_NULL;
    if (!aligned16(o)) return SAGE_E_ALIGN;
    if (Hq < 1 || T < 1 || T > cache->capacity) return SAGE_E_SHAPE;
    if (Hq % cache->Hkv != 0) return SAGE_E_GQA;
    const int grp = Hq / cache->Hkv;
    if (grp > sage::kDecodeMaxGroup) return SAGE_E_UNSUPPORTED;
    if ((st = sage_decode_workspace(cache, Hq, T, need)) != SAGE_OK) return st;
    const int64_t nchunk = sage::decode_nchunk(cache->B, cache->Hkv, T);
    if (nchunk * cache->Hkv * 256 > kMaxItems) return SAGE_E_SHAPE;
    std::memset(p, 0, sizeof(*p));
    p->B = cache->B; p->Hq = Hq; p->Hkv = cache->Hkv; p->grp = grp; p->D = cache->D; p->T = T;
    p->cap = cache->capacity;
    p->ns = sage::decode_steps(cache->B, cache->Hkv, T);
    p->nchunk = (int)nchunk;
    p->q = sage::View{static_cast<const uint16_t *>(q->ptr), q->sb, q->sn, q->sh};
    p->k8 = cache->k8; p->k_scale = cache->k_scale; p->vc = cache->v;
    if (!cache->v) { p->v8c = cache->v8; p->v_scale = cache->v_scale; }
    p->o = static_cast<uint16_t *>(o);
    return SAGE_OK;
}

}  // namespace

sage_status sage_decode_attn(const sage_kv_cache *cache, int32_t Hq, const sage_view_bf16 *q, int32_t T,
                             void *o, void *workspace, size_t ws_bytes, void *stream) {
    sage::DecodeParams p;
    size_t need = 0;
    sage_status st = build_decode(cache, Hq, q, T, o, &p, &need);
    if (st != SAGE_OK) return st;
    if (!workspace || ws_bytes < need) return SAGE_E_WORKSPACE;
    if (!aligned16(workspace)) return SAGE_E_ALIGN;
    p.part = static_cast<float *>(workspace);
    return sage_launch_decode(p, static_cast<hipStream_t>(stream)) == hipSuccess ? SAGE_OK : SAGE_E_HIP;
}

sage_status sage_decode_attn_noalloc(const sage_kv_cache *cache, int32_t Hq, const sage_view_bf16 *q, int32_t T,
                                     void *o, void *stream) {
    sage::DecodeParams p;
    size_t need = 0;
    sage_status st = build_decode(cache, Hq, q, T, o, &p, &need);
    if (st != SAGE_OK) return st;
    if (need > sage::kDecodeScratchBytes) return SAGE_E_WORKSPACE;
    void *scratch_ptr = nullptr;
    if (sage_decode_scratch(&scratch_ptr) != hipSuccess) return SAGE_E_HIP;
    p.part = static_cast<float *>(scratch_ptr);
    return sage_launch_decode(p, static_cast<hipStream_t>(stream)) == hipSuccess ? SAGE_OK : SAGE_E_HIP;
}

size_t sage_decode_noalloc_max_bytes(void) { return sage::kDecodeScratchBytes; }

sage_status sage_selftest_primitive(int32_t kind, uint32_t first, uint32_t count, void *out, void *stream) {
    if (!out) return SAGE_E_NULL;
    if (!aligned16(out)) return SAGE_E_ALIGN;
    if (kind < 0 || kind > 15) return SAGE_E_UNSUPPORTED;
    if (count < 1 || count > (1u << 26) || (uint64_t)first + count > (uint64_t(1) << 32)) return SAGE_E_SHAPE;
    if (kind >= 10 && count % 64 != 0) return SAGE_E_SHAPE;            // lane exchanges: whole waves
    return sage_launch_primitive(kind, first, count, out, static_cast<hipStream_t>(stream)) == hipSuccess ? SAGE_OK
                                                                                                        : SAGE_E_HIP;
}

int32_t sage_v8_key_of_slot(int32_t slot) {
    if (slot < 0 || slot >= 64) return -1;
    return sage_v8_slot_key(slot);
}

const char *sage_status_str(sage_status s) {
    switch (s) {
    case SAGE_OK: return "SAGE_OK";
    case SAGE_E_NULL: return "SAGE_E_NULL: a required pointer is NULL";
    case SAGE_E_SHAPE: return "SAGE_E_SHAPE: B, N, heads or head dim out of range";
    case SAGE_E_STRIDE: return "SAGE_E_STRIDE: d stride must be 1 and the output contiguous in (head, dim)";
    case SAGE_E_ALIGN: return "SAGE_E_ALIGN: buffers and rows must be 16-byte aligned";
    case SAGE_E_ROPE: return "SAGE_E_ROPE: rope_dim must be even and within [0, D]";
    case SAGE_E_GQA: return "SAGE_E_GQA: query heads must be a multiple of KV heads";
    case SAGE_E_WORKSPACE: return "SAGE_E_WORKSPACE: workspace missing or too small";
    case SAGE_E_UNSUPPORTED: return "SAGE_E_UNSUPPORTED: option not supported for this shape";
    case SAGE_E_HIP: return "SAGE_E_HIP: a kernel launch failed";
    }
    return "unknown sage_status";
}

int32_t sage_version(void) { return 100; }

}  // extern "C"
