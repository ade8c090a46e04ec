"""Pins of the oracle's quantized attention (page "Exact Numerical Contract",
sections "INT8 QK And Score Domain", "Online Softmax", "V And PV",
"Finalization And Tails") against closed forms, one-hot cases built directly
from quantized tensors, FP64 attention on the dequantized tensors, and the
accuracy gate against FP64 unquantized attention.
"""
import math

import numpy as np
import pytest

import oracle
import workloads

P_PEAK = 2.0 ** 8.807          # probability of the row maximum (FP8 offset 8.807)


def _synthetic(B, N, Hq, Hkv, D, rng):
    """A Prepared bundle built directly from random quantized tensors."""
    nq = ((N + 127) // 128) * 4
    nk = (N + 63) // 64
    q8 = rng.integers(-127, 128, (B, Hq, N, D), dtype=np.int8)
    k8 = rng.integers(-127, 128, (B, Hkv, N, D), dtype=np.int8)
    codes = rng.integers(0, 0x7F, (B, Hkv, N, D)).astype(np.uint8)   # finite positives
    sign = rng.integers(0, 2, (B, Hkv, N, D)).astype(np.uint8) << 7
    v8 = codes | sign
    qs = rng.uniform(0.5, 2.0, (B, Hq, nq)).astype(np.float32) * np.float32(0.02)
    ks = rng.uniform(0.5, 2.0, (B, Hkv, nk)).astype(np.float32) * np.float32(0.02)
    vs = rng.uniform(0.1, 1.0, (B, Hkv, D)).astype(np.float32)
    z = np.zeros((1,), np.uint16)
    return oracle.Prepared(z, z, z, q8, qs, k8, ks, v8, vs)


def _dequant_attention_f64(p, rows):
    """FP64 softmax attention on the dequantized tensors (no FP8 P rounding)."""
    B, Hq, N, D = p.q8.shape
    Hkv = p.k8.shape[1]
    c = 1.0 / math.sqrt(D)
    out = np.empty((len(rows), D))
    for r, (b, h, i) in enumerate(rows):
        hk = h // (Hq // Hkv)
        q = p.q8[b, h, i].astype(np.float64) * p.q_scale[b, h, i // 32]
        k = p.k8[b, hk].astype(np.float64) * np.repeat(p.k_scale[b, hk], 64)[:N, None]
        v = oracle.e4m3_to_f32(p.v8[b, hk]).astype(np.float64) * p.v_scale[b, hk][None, :]
        s = (k @ q) * c
        e = np.exp(s - s.max())
        out[r] = (e / e.sum()) @ v
    return out


def test_single_key_closed_form(oracle_lib):
    # N = 1: p = exp2(8.807) -> e4m3 448 for the only key, d = exp2(8.807),
    # so O = bf16((448 * dec(v8)) / d * v_scale)
    rng = np.random.default_rng(30)
    p = _synthetic(1, 1, 2, 2, 128, rng)
    o = oracle_lib.bf16_to_f32(oracle_lib.attn_rows(p, oracle.all_rows(1, 2, 1)))
    for h in range(2):
        v = oracle_lib.e4m3_to_f32(p.v8[0, h, 0]).astype(np.float64) * p.v_scale[0, h]
        exact = 448.0 / P_PEAK * v
        assert np.all(np.abs(o[h] - exact) <= np.abs(exact) * 2.0**-8 + 1e-30)


@pytest.mark.parametrize("N", [5, 64, 130, 1000])
def test_zero_query_row_averages_v(oracle_lib, N):
    # q8 row == 0: every score is 0, every p = exp2(8.807) -> 448, so
    # O = (448 / exp2(8.807)) * mean_n dec(v8) * v_scale
    rng = np.random.default_rng(31)
    p = _synthetic(1, N, 1, 1, 128, rng)
    p.q8[0, 0, 3] = 0
    o = oracle_lib.bf16_to_f32(oracle_lib.attn_rows(p, np.array([[0, 0, 3]])))[0]
    v = oracle_lib.e4m3_to_f32(p.v8[0, 0]).astype(np.float64)
    exact = 448.0 / P_PEAK * v.mean(axis=0) * p.v_scale[0, 0]
    tol = np.abs(exact) * 2.0**-8 + 1e-6 * p.v_scale[0, 0] * np.abs(v).max()
    assert np.all(np.abs(o - exact) <= tol)


@pytest.mark.parametrize("N,jstar", [(70, 0), (70, 69), (300, 130), (1000, 999), (1000, 577)])
def test_one_hot_row_selects_key(oracle_lib, N, jstar):
    # q8 = 127 e_0; k8[:, 0] = 0 except k8[j*, 0] = 127: the score gap is
    # 16129 * f = 2057 (log2 units) -> every other probability underflows to 0
    # and O is the dequantized V row of key j* (in its tile, tail included).
    rng = np.random.default_rng(32)
    Hq, Hkv, D = 4, 2, 128
    p = _synthetic(1, N, Hq, Hkv, D, rng)
    p.q8[...] = 0
    p.q8[..., 0] = 127
    p.k8[...] = 0
    p.k8[:, :, jstar, 0] = 127
    p.q_scale[...] = 1.0
    p.k_scale[...] = 1.0
    rows = np.array([[0, h, i] for h in range(Hq) for i in (0, N - 1)])
    o = oracle_lib.bf16_to_f32(oracle_lib.attn_rows(p, rows))
    for r, (_, h, _) in enumerate(rows):
        hk = h // (Hq // Hkv)                      # GQA: consecutive query heads share a KV head
        v = oracle_lib.e4m3_to_f32(p.v8[0, hk, jstar]).astype(np.float64) * p.v_scale[0, hk]
        exact = 448.0 / P_PEAK * v
        assert np.all(np.abs(o[r] - exact) <= np.abs(exact) * 2.0**-8 + 1e-30)


@pytest.mark.parametrize("N,Hq,Hkv,D", [(200, 2, 2, 128), (1000, 4, 2, 128), (333, 2, 1, 256)])
def test_matches_fp64_on_dequantized_tensors(oracle_lib, N, Hq, Hkv, D):
    # The oracle differs from exact softmax attention over the dequantized
    # Q/K/V only by the E4M3 rounding of P (<= 2^-4 relative) and FP32 sums.
    rng = np.random.default_rng(33)
    p = _synthetic(1, N, Hq, Hkv, D, rng)
    p.q_scale[...] *= np.float32(1.5)
    rows = np.array([[0, h, i] for h in range(Hq) for i in range(0, N, max(1, N // 40))] +
                    [[0, Hq - 1, N - 1]])
    o = oracle_lib.bf16_to_f32(oracle_lib.attn_rows(p, rows)).astype(np.float64)
    ref = _dequant_attention_f64(p, rows)
    scale = np.abs(ref).max(axis=1, keepdims=True)
    assert np.max(np.abs(o - ref) / scale) < 0.04
    assert oracle.cosine(o, ref) > 0.999


@pytest.mark.parametrize("name", ["tiny", "tail"])
def test_accuracy_vs_fp64_unquantized(oracle_lib, name):
    # the quantized pipeline stays within cosine 0.99 of FP64 softmax attention
    # on the same prepared BF16 Q/K and BF16 V (the accuracy requirement)
    inp = workloads.make_inputs(workloads.CONFIGS[name])
    p = oracle.prepare(inp)
    o = oracle_lib.bf16_to_f32(oracle.attention(p))
    ref = oracle.reference_attention_f64(p.zq, p.zk, inp.v)
    assert oracle.cosine(o, ref) >= 0.99
    for h in range(inp.cfg.Hq):
        assert oracle.cosine(o[:, :, h], ref[:, :, h]) >= 0.99


def test_accuracy_gqa_hadamard_sampled_rows(oracle_lib):
    cfg = workloads.CONFIGS["gqa"]
    inp = workloads.make_inputs(cfg, N=1024)
    p = oracle.prepare(inp)
    rows = np.array([[0, h, i] for h in range(cfg.Hq) for i in (0, 1, 511, 1000, 1023)])
    o = oracle_lib.bf16_to_f32(oracle.attn_rows(p, rows))
    ref = oracle.reference_attention_f64(p.zq, p.zk, inp.v, rows=rows)
    assert oracle.cosine(o, ref) >= 0.99


def test_mean_smoothing_does_not_change_the_reference(oracle_lib):
    # subtracting the per-channel K mean shifts each query's scores uniformly:
    # FP64 softmax attention is unchanged (why the reference needs no smoothing)
    inp = workloads.make_inputs(workloads.CONFIGS["tiny"])
    p = oracle.prepare(inp)
    ref0 = oracle.reference_attention_f64(p.zq, p.zk, inp.v)
    zk_sm = oracle_lib.f32_to_bf16(oracle_lib.bf16_to_f32(p.zk) - p.k_mean[:, :, None, :])
    ref1 = oracle.reference_attention_f64(p.zq, zk_sm, inp.v)
    assert oracle.cosine(ref0, ref1) > 0.9999
