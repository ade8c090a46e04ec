"""Pins of the oracle's decode-time INT8 K cache (per-head Hadamard rotation,
one FP32 scale per (head, token)) and of its single-query attention, against
scipy's Hadamard matrix, numpy FP64 attention on the dequantized cache, closed
forms, and the KL-divergence gate of the NPU issue page (attention weights
against the unquantized cache, head width 256, 512 keys, 8 draws; uniform, 8x
and 30x outlier channels)."""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle

D = 256
HM = scipy.linalg.hadamard(D).astype(np.float64) / math.sqrt(D)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


def _f(t):
    return t.float().numpy().astype(np.float64)


def test_cache_rows_are_rotated_then_row_scaled():
    rng = np.random.default_rng(10)
    k = _bf16(rng.standard_normal((2, 37, 3, D)) * rng.uniform(0.1, 5, (2, 37, 3, 1)))
    k8, ks = oracle.kv_quant(k)
    u = np.einsum("bthd,ed->bhte", _f(k), HM)                # rotated rows, FP64
    err = np.abs(u - k8.astype(np.float64) * ks[..., None].astype(np.float64))
    assert (err <= ks[..., None] * (0.5 + 1e-4) + 1e-9).all()
    assert (np.abs(k8).max(axis=-1) == 127).all()
    # amax / 127 with amax the largest |u| (FP32 butterflies vs FP64 matrix)
    np.testing.assert_allclose(ks, np.abs(u).max(axis=-1) / 127, rtol=1e-5)


def test_strided_views_match_contiguous_rows():
    rng = np.random.default_rng(11)
    big = _bf16(rng.standard_normal((1, 20, 5 * D)))
    k = big[:, :, 2 * D:4 * D].view(1, 20, 2, D)              # interleaved-buffer view
    a8, a_s = oracle.kv_quant(k)
    b8, b_s = oracle.kv_quant(k.contiguous())
    assert np.array_equal(a8, b8) and np.array_equal(a_s.view(np.uint32), b_s.view(np.uint32))


def _numpy_decode(q, k8, ks, v, T, grp):
    """FP64 attention on the dequantized cache, query rotated with scipy."""
    B, Hq, _ = q.shape
    o = np.empty((B, Hq, D)); w = np.empty((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            hk = h // grp
            qr = HM @ _f(q[b, h])
            kd = k8[b, hk, :T].astype(np.float64) * ks[b, hk, :T, None].astype(np.float64)
            s = kd @ qr / math.sqrt(D)
            e = np.exp(s - s.max())
            w[b, h] = e / e.sum()
            o[b, h] = w[b, h] @ _f(v[b, hk, :T])
    return o, w


def test_decode_matches_numpy_on_dequantized_cache():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, T, Tc = 2, 6, 2, 50, 64
    k = _bf16(rng.standard_normal((B, Tc, Hkv, D)))
    v = _bf16(rng.standard_normal((B, Hkv, Tc, D)))
    q = _bf16(rng.standard_normal((B, Hq, D)) * 2)
    k8, ks = oracle.kv_quant(k)
    o, w = oracle.decode_attn(q, k8, ks, v.view(torch.int16).numpy().view(np.uint16), T)
    o_ref, w_ref = _numpy_decode(q, k8, ks, v, T, Hq // Hkv)
    np.testing.assert_allclose(w, w_ref, rtol=1e-5, atol=1e-12)
    got = oracle.bf16_to_f32(o).astype(np.float64)
    assert np.abs(got - o_ref).max() <= 2 ** -8 * np.abs(o_ref).max()


def test_decode_closed_forms():
    rng = np.random.default_rng(13)
    k = _bf16(rng.standard_normal((1, 8, 1, D)))
    v = _bf16(rng.standard_normal((1, 1, 8, D)))
    vb = v.view(torch.int16).numpy().view(np.uint16)
    k8, ks = oracle.kv_quant(k)
    q = _bf16(rng.standard_normal((1, 1, D)))
    o, w = oracle.decode_attn(q, k8, ks, vb, 1)              # one token: o = v[0]
    assert w[0, 0, 0] == 1.0 and np.array_equal(o[0, 0], vb[0, 0, 0])
    z = torch.zeros((1, 1, D), dtype=torch.bfloat16)        # zero query: uniform weights
    o, w = oracle.decode_attn(z, k8, ks, vb, 8)
    np.testing.assert_allclose(w, 1 / 8, rtol=0, atol=1e-15)
    mean = _f(v[0, 0]).mean(axis=0)
    assert np.abs(oracle.bf16_to_f32(o[0, 0]) - mean).max() <= 2 ** -8 * np.abs(mean).max()


def _draw(rng, mult, n_keys=512, n_out=8):
    """One draw of the gate: query and keys N(0,1); `n_out` channels of the keys
    scaled by `mult` (uniform control: mult = 1)."""
    k = rng.standard_normal((n_keys, D))
    if mult != 1:
        k[:, rng.choice(D, n_out, replace=False)] *= mult
    return _bf16(rng.standard_normal(D)), _bf16(k)


def _kld(p, q):
    return float(np.sum(p * (np.log(p) - np.log(q))))


def _weights_unquantized(q, k):
    s = _f(k) @ _f(q) / math.sqrt(D)
    e = np.exp(s - s.max())
    return e / e.sum()


def _weights_int8_unrotated(q, k):
    # the control row: the same per-(head, token) INT8 scale without rotation
    u = _f(k).astype(np.float32)
    amax = np.maximum(np.abs(u).max(axis=1, keepdims=True), np.float32(1e-7))
    k8 = np.clip(np.rint(u * (np.float32(127) / amax)), -128, 127)
    s = (k8 * (amax / np.float32(127))).astype(np.float64) @ _f(q) / math.sqrt(D)
    e = np.exp(s - s.max())
    return e / e.sum()


def _gate_row(mult, draws=8, seed=14):
    rng = np.random.default_rng(seed + int(mult))
    rot, unrot = [], []
    for _ in range(draws):
        q, k = _draw(rng, mult)
        p = _weights_unquantized(q, k)
        k8, ks = oracle.kv_quant(k.view(1, -1, 1, D))
        _, w = oracle.decode_attn(q.view(1, 1, D), k8, ks, np.zeros((1, 1, k.shape[0], D), np.uint16), k.shape[0])
        rot.append(_kld(p, w[0, 0]))
        unrot.append(_kld(p, _weights_int8_unrotated(q, k)))
    return float(np.mean(rot)), float(np.mean(unrot))


@pytest.mark.parametrize("mult", [1, 8, 30])
def test_kld_gate_rotated_int8_cache(mult):
    rot, unrot = _gate_row(mult)
    print(f"outlier x{mult}: KLD rotated {rot:.3g}, unrotated {unrot:.3g}")
    assert rot <= 1e-3
    if mult == 1:
        assert 0.3 < unrot / rot < 3.0                   # rotation is worth nothing on the control
    if mult == 30:
        assert unrot > 5 * rot and unrot > 1e-3           # and is what keeps x30 inside the gate


def _v8_case(rng, B, T, Hq, Hkv, vmul=1.0):
    q = _bf16(rng.standard_normal((B, Hq, D)) * 2.0)
    k = _bf16(rng.standard_normal((B, T, Hkv, D)))
    v = _bf16(rng.standard_normal((B, T, Hkv, D)) * vmul)
    k8, ks = oracle.kv_quant(k)
    v8, vs = oracle.kv_quant(v)
    return q, k8, ks, v, v8, vs


def test_int8_v_one_token_gives_back_the_row():
    # T = 1: weight 1, the output is the stored row rotated back, within the
    # row's quantization error (|e_i| <= s/2 per rotated element, so at most
    # sqrt(D) s / 2 = 8 s per output element) plus one BF16 rounding
    rng = np.random.default_rng(110)
    q, k8, ks, v, v8, vs = _v8_case(rng, 2, 1, 4, 2, vmul=3.0)
    o, w = oracle.decode_attn_v8(q, k8, ks, v8, vs, 1)
    assert (w == 1.0).all()
    got = oracle.bf16_to_f32(o).astype(np.float64)
    ref = np.repeat(_f(v)[:, 0], 2, axis=1)                   # heads 0,1 -> KV 0; 2,3 -> KV 1
    bound = 8 * np.repeat(vs[:, :, 0], 2, axis=1)[..., None] + 2 ** -8 * np.abs(ref)
    assert (np.abs(got - ref) <= bound).all()
    # and the whole-row error is far below that per-element bound
    assert np.sqrt(((got - ref) ** 2).sum(-1)).max() <= 8 * vs.max() * 1.01


def test_int8_v_matches_the_rotated_back_matrix_formula():
    # FP64 reference with scipy's Hadamard matrix: o = HM (sum_t w_t s_t v8_t)
    rng = np.random.default_rng(111)
    B, T, Hq, Hkv = 2, 45, 6, 3
    q, k8, ks, v, v8, vs = _v8_case(rng, B, T, Hq, Hkv)
    o, w = oracle.decode_attn_v8(q, k8, ks, v8, vs, T)
    _, w_bf16 = oracle.decode_attn(q, k8, ks, np.zeros((B, Hkv, T, D), np.uint16), T)
    assert np.array_equal(w, w_bf16)                           # the weights do not depend on V
    deq = v8.astype(np.float64) * vs[..., None].astype(np.float64)        # [B, Hkv, T, D]
    r = np.einsum("bht,bhtd->bhd", w, np.repeat(deq, Hq // Hkv, axis=1))
    ref = np.einsum("ed,bhd->bhe", HM, r)
    got = oracle.bf16_to_f32(o).astype(np.float64)
    assert np.abs(got - ref).max() <= 2 ** -8 * np.abs(ref).max()
    # and it stays within the quantization bound of the BF16-V result
    o16, _ = oracle.decode_attn(q, k8, ks, np.ascontiguousarray(
        v.permute(0, 2, 1, 3).contiguous().view(torch.int16).numpy().view(np.uint16)), T)
    g16 = oracle.bf16_to_f32(o16).astype(np.float64)
    assert np.abs(got - g16).max() <= 8 * vs.max() + 2 ** -7 * np.abs(g16).max()


def test_int8_v_constant_rows_ignore_the_weights():
    # every cached V row equal: any weights summing to 1 give that row back
    rng = np.random.default_rng(112)
    B, T, Hq, Hkv = 1, 33, 4, 1
    q = _bf16(rng.standard_normal((B, Hq, D)) * 4.0)
    k8, ks = oracle.kv_quant(_bf16(rng.standard_normal((B, T, Hkv, D))))
    row = rng.standard_normal(D)
    v8, vs = oracle.kv_quant(_bf16(np.broadcast_to(row, (B, T, Hkv, D))))
    o, w = oracle.decode_attn_v8(q, k8, ks, v8, vs, T)
    assert w.std(axis=-1).min() > 0                            # the weights are not uniform
    got = oracle.bf16_to_f32(o).astype(np.float64)
    one, _ = oracle.decode_attn_v8(q, k8[:, :, :1], ks[:, :, :1], v8[:, :, :1], vs[:, :, :1], 1)
    np.testing.assert_allclose(got, oracle.bf16_to_f32(one).astype(np.float64), rtol=2 ** -7, atol=1e-6)
