"""Decode-time INT8 K cache on the GPU against the oracle: the cache (rotated
INT8 K, per-(head, token) scales, BF16 V) byte-identical, the single-query
attention within the rounding of an FP32 evaluation (at most one or two BF16
steps of the output, cosine 0.99999), and the KL-divergence gate of the NPU
issue page on the GPU-written cache."""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from gpu_util import banner

pytestmark = pytest.mark.gpu

D = 256
HM = scipy.linalg.hadamard(D).astype(np.float64) / math.sqrt(D)


def _kv(rng, B, n, Hkv, scale=1.0):
    """K and V as strided views of one interleaved buffer [B, n, (2 Hkv + 1) D]."""
    buf = torch.from_numpy((rng.standard_normal((B, n, (2 * Hkv + 1) * D)) * scale).astype(np.float32))
    buf = buf.to(torch.bfloat16)
    k = buf[:, :, D:(Hkv + 1) * D].view(B, n, Hkv, D)
    v = buf[:, :, (Hkv + 1) * D:].view(B, n, Hkv, D)
    return buf, k, v


def _cache_k_host(cache, T):
    return cache.k8[:, :, :T].cpu().numpy(), cache.k_scale[:, :, :T].cpu().numpy()


def _v_bits(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def test_append_matches_oracle_byte_for_byte():
    import quantized_exact_order_amd as sage
    rng = np.random.default_rng(20)
    B, n, Hkv, t0, cap = 2, 300, 3, 17, 400
    banner(f"kv_append B={B} n={n} Hkv={Hkv} t0={t0}")
    buf, k, v = _kv(rng, B, n, Hkv, scale=3.0)
    dbuf = buf.cuda()
    dk = dbuf[:, :, D:(Hkv + 1) * D].view(B, n, Hkv, D)
    dv = dbuf[:, :, (Hkv + 1) * D:].view(B, n, Hkv, D)
    cache = sage.KvCache.allocate(B, Hkv, cap, "cuda")
    cache.k8.fill_(0x55)
    cache.v.view(torch.int16).fill_(0x3f80)            # BF16 1.0 in every slot before the append
    sage.kv_append(cache, dk, dv, t0)
    torch.cuda.synchronize()
    k8, ks = oracle.kv_quant(k)
    assert np.array_equal(cache.k8[:, :, t0:t0 + n].cpu().numpy(), k8)
    assert np.array_equal(cache.k_scale[:, :, t0:t0 + n].cpu().numpy().view(np.uint32), ks.view(np.uint32))
    vr = _v_bits(cache.v_rows())
    assert np.array_equal(vr[:, :, t0:t0 + n], _v_bits(v.permute(0, 2, 1, 3)))
    # the other tokens of the partly written 8-token blocks (and all others) keep their values
    assert (vr[:, :, :t0] == 0x3f80).all() and (vr[:, :, t0 + n:] == 0x3f80).all()
    assert (cache.k8[:, :, :t0] == 0x55).all() and (cache.k8[:, :, t0 + n:] == 0x55).all()


def test_append_in_pieces_equals_one_append():
    import quantized_exact_order_amd as sage
    rng = np.random.default_rng(21)
    B, n, Hkv = 1, 200, 2
    banner("kv_append in pieces")
    _, k, v = _kv(rng, B, n, Hkv)
    k, v = k.cuda(), v.cuda()
    a = sage.KvCache.allocate(B, Hkv, n, "cuda")
    b = sage.KvCache.allocate(B, Hkv, n, "cuda")
    sage.kv_append(a, k, v, 0)
    for s, e in ((0, 1), (1, 64), (64, 130), (130, 200)):
        sage.kv_append(b, k[:, s:e], v[:, s:e], s)
    torch.cuda.synchronize()
    assert torch.equal(a.k8, b.k8) and torch.equal(a.k_scale.view(torch.int32), b.k_scale.view(torch.int32))
    assert torch.equal(a.v.view(torch.int16), b.v.view(torch.int16))


def _check_decode(B, Hq, Hkv, T, cap, seed, q_scale=1.0, label="", poison=False, int8_v=False):
    import quantized_exact_order_amd as sage
    rng = np.random.default_rng(seed)
    label = label + (" int8 V" if int8_v else "")
    banner(f"decode {label} B={B} Hq={Hq} Hkv={Hkv} T={T} cap={cap}")
    _, k, v = _kv(rng, B, T, Hkv)
    q = torch.from_numpy((rng.standard_normal((B, Hq, D)) * q_scale).astype(np.float32)).to(torch.bfloat16)
    cache = sage.KvCache.allocate(B, Hkv, cap, "cuda", int8_v=int8_v)
    if poison:          # NaN in every V slot, K and V scale and K byte pattern that the append does not write
        if int8_v:
            cache.v8.fill_(-128)
            cache.v_scale.view(torch.int32).fill_(0x7fc00000)
        else:
            cache.v.view(torch.int16).fill_(0x7fc0)
        cache.k_scale.view(torch.int32).fill_(0x7fc00000)
        cache.k8.fill_(-128)
    sage.kv_append(cache, k.cuda(), v.cuda(), 0)
    o = sage.decode_attn(cache, q.cuda(), T)
    torch.cuda.synchronize()
    k8, ks = oracle.kv_quant(k)
    if int8_v:
        v8, vs = oracle.kv_quant(v)
        o_ref, _ = oracle.decode_attn_v8(q, k8, ks, v8, vs, T)
    else:
        o_ref, _ = oracle.decode_attn(q, k8, ks, _v_bits(v.permute(0, 2, 1, 3)), T)
    g = o.cpu().float().numpy().astype(np.float64)
    r = oracle.bf16_to_f32(o_ref).astype(np.float64)
    err = np.abs(g - r)
    print(f"[gpu] {label}: max-abs {err.max():.3g} (scale {np.abs(r).max():.3g}), "
          f"differing {np.mean(g != r):.4f}, cos {oracle.cosine(g, r):.7f}", flush=True)
    assert err.max() <= 2 ** -7 * np.abs(r).max()
    assert oracle.cosine(g, r) >= 0.99999


@pytest.mark.parametrize("Hq", [2, 4, 6, 8, 16, 26, 32])
def test_decode_group_sizes(Hq):
    _check_decode(2, Hq, 2, 300, 320, seed=30 + Hq, label=f"grp {Hq // 2}")


@pytest.mark.parametrize("T", [1, 2, 7, 9, 31, 33, 63, 64, 255, 256, 257, 511, 513, 1000])
def test_decode_token_counts(T):
    _check_decode(1, 8, 2, T, 1024, seed=40 + T, q_scale=2.0, label=f"T={T}")


@pytest.mark.parametrize("T,cap", [(1, 8), (13, 16), (300, 304), (296, 296), (777, 1024)])
def test_decode_ignores_unwritten_cache_slots(T, cap):
    # slots past T hold NaN; the last chunk reaches past the capacity when T = cap
    _check_decode(2, 16, 2, T, cap, seed=70 + T, q_scale=2.0, label="poisoned", poison=True)


@pytest.mark.parametrize("B,Hq,Hkv,T,poison", [(4, 8, 4, 8200, True), (4, 16, 4, 20000, False),
                                                (8, 16, 8, 5000, False)])
def test_decode_multi_step_chunks(B, Hq, Hkv, T, poison):
    # caches large enough for several 32-token steps per wave (the waves of a
    # work-group take interleaved steps), with a last chunk that leaves some
    # waves fewer steps or none: 8200 = 32 chunks of 256 + 8 tokens,
    # 20000 = 39 chunks of 512 + 32, 5000 = 9 chunks of 512 + 392
    _check_decode(B, Hq, Hkv, T, T, seed=80 + B + Hkv, q_scale=2.0, label="multi-step", poison=poison)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("int8_v", [False, True])
def test_decode_cache_past_2_31_elements(int8_v):
    # B = 16 sequences x 8 KV heads x 67,000 tokens x 256: the K cache holds
    # 2.2e9 bytes and V 2.2e9 values (BF16 or INT8), past 2^31.  The GPU
    # appends and decodes everything; the oracle quantizes and attends single
    # (b, KV head) slices, among them the last one at the far end of the cache
    import quantized_exact_order_amd as sage
    B, Hkv, grp, T = 16, 8, 4, 67000
    Hq = Hkv * grp
    banner(f"decode cache past 2^31 elements: B={B} Hkv={Hkv} T={T} int8_v={int8_v}")
    gen = torch.Generator(device="cuda").manual_seed(91)
    k, v = (torch.randn((B, T, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(2))
    q = (2.0 * torch.randn((B, Hq, D), generator=gen, device="cuda")).to(torch.bfloat16)
    cache = sage.KvCache.allocate(B, Hkv, T, "cuda", int8_v=int8_v)
    sage.kv_append(cache, k, v, 0)
    o = sage.decode_attn(cache, q, T)
    torch.cuda.synchronize()
    vblocks = cache.v8 if int8_v else cache.v
    assert cache.k8.numel() > 2 ** 31 and vblocks.numel() > 2 ** 31
    for b, hk in ((0, 0), (7, 3), (B - 1, Hkv - 1)):
        ks = k[b:b + 1, :, hk:hk + 1].cpu()
        k8, kscale = oracle.kv_quant(ks)
        assert np.array_equal(cache.k8[b, hk].cpu().numpy(), k8[0, 0]), (b, hk)
        assert np.array_equal(cache.k_scale[b, hk].cpu().numpy().view(np.uint32), kscale[0, 0].view(np.uint32))
        vblk = vblocks[b:b + 1, hk:hk + 1].permute(0, 1, 2, 4, 3).reshape(1, 1, T, D)   # [1, 1, T/8, D, 8] -> rows
        qs = q[b:b + 1, hk * grp:(hk + 1) * grp].cpu()
        if int8_v:
            v8, vscale = oracle.kv_quant(v[b:b + 1, :, hk:hk + 1].cpu())
            assert np.array_equal(vblk.cpu().numpy(), v8), (b, hk)
            assert np.array_equal(cache.v_scale[b, hk].cpu().numpy().view(np.uint32), vscale[0, 0].view(np.uint32))
            o_ref, _ = oracle.decode_attn_v8(qs, k8, kscale, v8, vscale, T)
        else:
            vs = _v_bits(v[b:b + 1, :, hk:hk + 1].permute(0, 2, 1, 3))
            assert np.array_equal(_v_bits(vblk), vs), (b, hk)
            o_ref, _ = oracle.decode_attn(qs, k8, kscale, vs, T)
        g = o[b:b + 1, hk * grp:(hk + 1) * grp].cpu().float().numpy().astype(np.float64)
        r = oracle.bf16_to_f32(o_ref).astype(np.float64)
        assert np.abs(g - r).max() <= 2 ** -7 * np.abs(r).max(), (b, hk)
        assert oracle.cosine(g, r) >= 0.99999, (b, hk)
    del cache, k, v
    torch.cuda.empty_cache()


@pytest.mark.timeout(300)
def test_decode_long_context():
    _check_decode(1, 16, 4, 32768, 32768, seed=50, q_scale=2.0, label="32k tokens")


@pytest.mark.parametrize("mult", [1, 8, 30])
def test_kld_gate_on_gpu_cache(mult):
    import quantized_exact_order_amd as sage
    rng = np.random.default_rng(60 + mult)
    banner(f"KLD gate, outlier x{mult}")
    klds = []
    for _ in range(8):
        kk = rng.standard_normal((512, D))
        if mult != 1:
            kk[:, rng.choice(D, 8, replace=False)] *= mult
        k = torch.from_numpy(kk.astype(np.float32)).to(torch.bfloat16).view(1, 512, 1, D)
        q = torch.from_numpy(rng.standard_normal(D).astype(np.float32)).to(torch.bfloat16)
        cache = sage.KvCache.allocate(1, 1, 512, "cuda")
        sage.kv_append(cache, k.cuda(), k.cuda(), 0)
        torch.cuda.synchronize()
        k8, ks = _cache_k_host(cache, 512)
        kd = k8[0, 0].astype(np.float64) * ks[0, 0, :, None].astype(np.float64)
        qr = HM @ q.float().numpy().astype(np.float64)
        s_q = kd @ qr / math.sqrt(D)
        s_f = k[0, :, 0].float().numpy().astype(np.float64) @ q.float().numpy().astype(np.float64) / math.sqrt(D)
        pq = np.exp(s_q - s_q.max()); pq /= pq.sum()
        pf = np.exp(s_f - s_f.max()); pf /= pf.sum()
        klds.append(float(np.sum(pf * (np.log(pf) - np.log(pq)))))
    print(f"[gpu] outlier x{mult}: KLD {np.mean(klds):.3g}", flush=True)
    assert np.mean(klds) <= 1e-3


@pytest.mark.parametrize("int8_v", [False, True])
def test_decode_step_hip_graph_replays_match_eager(int8_v):
    # one serving step (append one token, then decode over the cache) captured
    # in a HIP graph with caller-owned output and workspace, replayed three
    # times with unrelated eager work between replays that overwrites the
    # appended slot, the output and the workspace
    import quantized_exact_order_amd as sage
    rng = np.random.default_rng(95)
    B, Hq, Hkv, T0, cap = 2, 16, 2, 3000, 3072
    banner(f"decode step in a HIP graph B={B} Hq={Hq} Hkv={Hkv} T0={T0} int8_v={int8_v}")
    _, k, v = _kv(rng, B, T0 + 1, Hkv)
    k, v = k.cuda(), v.cuda()
    q = torch.from_numpy((rng.standard_normal((B, Hq, D)) * 2.0).astype(np.float32)).to(torch.bfloat16).cuda()
    q2 = q.flip(1).contiguous()
    cache = sage.KvCache.allocate(B, Hkv, cap, "cuda", int8_v=int8_v)
    sage.kv_append(cache, k[:, :T0], v[:, :T0], 0)
    k1, v1 = k[:, T0:], v[:, T0:]
    vt = (lambda: cache.v.view(torch.int16)) if not int8_v else (lambda: torch.cat(
        [cache.v8.flatten(), cache.v_scale.view(torch.int8).flatten()]))
    need = max(sage.decode_workspace(cache, Hq, T0 + 1), sage.decode_workspace(cache, Hq, T0))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")

    def step():
        sage.kv_append(cache, k1, v1, T0)
        sage.decode_attn(cache, q, T0 + 1, o=o, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = o.clone()
    k8_eager, ks_eager, v_eager = cache.k8.clone(), cache.k_scale.clone(), vt().clone()
    o_full = sage.decode_attn(cache, q, T0 + 1)            # library-allocated buffers: same bytes
    torch.cuda.synchronize()
    assert torch.equal(o_full.view(torch.int16), eager.view(torch.int16))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        cache.k8[:, :, T0].fill_(7)
        cache.k_scale[:, :, T0].fill_(3.0)
        if int8_v:
            cache.v_scale[:, :, T0].fill_(5.0)
        o.zero_()
        sage.decode_attn(cache, q2, T0, o=torch.empty_like(o), workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert torch.equal(cache.k8, k8_eager) and torch.equal(vt(), v_eager)
        assert torch.equal(cache.k_scale.view(torch.int32), ks_eager.view(torch.int32)), f"replay {rep}"


def test_int8_v_append_matches_oracle_byte_for_byte():
    # V rows rotated and quantized exactly as K rows, stored in 8-token blocks;
    # appended in pieces that start and end inside blocks, the other tokens of
    # a block keep their bytes
    import quantized_exact_order_amd as sage
    rng = np.random.default_rng(120)
    B, n, Hkv, t0, cap = 2, 300, 3, 17, 400
    banner(f"kv_append int8 V B={B} n={n} Hkv={Hkv} t0={t0}")
    _, k, v = _kv(rng, B, n, Hkv, scale=3.0)
    cache = sage.KvCache.allocate(B, Hkv, cap, "cuda", int8_v=True)
    cache.v8.fill_(0x55)
    cache.v_scale.fill_(2.0)
    for s, e in ((0, 1), (1, 70), (70, 131), (131, n)):
        sage.kv_append(cache, k[:, s:e].cuda(), v[:, s:e].cuda(), t0 + s)
    torch.cuda.synchronize()
    k8, ks = oracle.kv_quant(k)
    v8, vs = oracle.kv_quant(v)
    assert np.array_equal(cache.k8[:, :, t0:t0 + n].cpu().numpy(), k8)
    assert np.array_equal(cache.k_scale[:, :, t0:t0 + n].cpu().numpy().view(np.uint32), ks.view(np.uint32))
    vr = cache.v_rows().cpu().numpy()
    assert np.array_equal(vr[:, :, t0:t0 + n], v8)
    assert np.array_equal(cache.v_scale[:, :, t0:t0 + n].cpu().numpy().view(np.uint32), vs.view(np.uint32))
    assert (vr[:, :, :t0] == 0x55).all() and (vr[:, :, t0 + n:] == 0x55).all()
    assert (cache.v_scale[:, :, :t0] == 2.0).all() and (cache.v_scale[:, :, t0 + n:] == 2.0).all()


@pytest.mark.parametrize("B,Hq,Hkv,T,cap,poison", [
    (2, 2, 2, 300, 320, False), (2, 16, 2, 300, 320, False), (2, 26, 2, 300, 320, False),
    (1, 8, 2, 1, 8, True), (1, 8, 2, 9, 16, True), (1, 8, 2, 63, 64, False), (1, 8, 2, 257, 1024, True),
    (1, 8, 2, 1000, 1000, False), (4, 8, 4, 8200, 8200, True), (4, 16, 4, 20000, 20000, False),
    (1, 16, 4, 32768, 32768, False)])
def test_int8_v_decode(B, Hq, Hkv, T, cap, poison):
    _check_decode(B, Hq, Hkv, T, cap, seed=130 + T + Hq, q_scale=2.0, label="", poison=poison, int8_v=True)
