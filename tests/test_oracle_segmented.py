"""Pins of the oracle's segmented (split-KV) schedule, the opt-in non-exact
mode modelled on the FP8-PV page's segmented schedules: nseg contiguous runs
of key tiles, each run from the contract's initial state, combined in
increasing segment order with weights exp2(m_s - M).

With one segment the combine is the identity, so the exact oracle is the
reference; at every segmentation the zero-query and one-hot closed forms
hold, two keys in different segments with a known score gap weigh their V
rows 2^gap : 1, and the output stays close to FP64 softmax attention on the
dequantized tensors."""
import math

import numpy as np
import pytest

import oracle
import workloads
from test_oracle_attn import P_PEAK, _dequant_attention_f64, _synthetic


def _segments(nk, nseg):
    return [(s * nk // nseg, (s + 1) * nk // nseg) for s in range(nseg)]


@pytest.mark.parametrize("name", ["tiny", "tail"])
def test_one_segment_is_the_exact_schedule(oracle_lib, name):
    inp = workloads.make_inputs(workloads.CONFIGS[name])
    p = oracle.prepare(inp)
    assert np.array_equal(oracle.attention_segmented(p, 1), oracle.attention(p))


def test_one_segment_is_the_exact_schedule_gqa_d256(oracle_lib):
    rng = np.random.default_rng(40)
    p = _synthetic(1, 333, 4, 2, 256, rng)
    rows = oracle.all_rows(1, 4, 333)
    assert np.array_equal(oracle.attn_rows_segmented(p, rows, 1), oracle.attn_rows(p, rows))


def test_segments_cover_every_tile_once():
    for nk in (1, 2, 3, 7, 12, 591):
        for nseg in sorted({n for n in (1, 2, 3, nk // 2, nk) if 1 <= n <= nk}):
            seg = _segments(nk, nseg)
            assert seg[0][0] == 0 and seg[-1][1] == nk
            assert all(a < b for a, b in seg) and all(seg[i][1] == seg[i + 1][0] for i in range(nseg - 1))


@pytest.mark.parametrize("N,nseg", [(130, 2), (130, 3), (1000, 2), (1000, 5), (1000, 16)])
def test_zero_query_row_averages_v(oracle_lib, N, nseg):
    # every score 0 in every segment: p = exp2(8.807) -> 448, equal maxima,
    # unit weights, O = (448 / exp2(8.807)) * mean_n dec(v8) * v_scale
    rng = np.random.default_rng(41)
    p = _synthetic(1, N, 1, 1, 128, rng)
    p.q8[0, 0, 3] = 0
    o = oracle_lib.bf16_to_f32(oracle_lib.attn_rows_segmented(p, np.array([[0, 0, 3]]), nseg))[0]
    v = oracle_lib.e4m3_to_f32(p.v8[0, 0]).astype(np.float64)
    exact = 448.0 / P_PEAK * v.mean(axis=0) * p.v_scale[0, 0]
    tol = np.abs(exact) * 2.0**-8 + 1e-6 * p.v_scale[0, 0] * np.abs(v).max()
    assert np.all(np.abs(o - exact) <= tol)


def _one_hot(N, Hq, Hkv, D, keys, kvals, rng):
    """q8 = 127 e_0, k8[:, 0] = kvals at the given keys and 0 elsewhere, unit scales."""
    p = _synthetic(1, N, Hq, Hkv, D, rng)
    p.q8[...] = 0
    p.q8[..., 0] = 127
    p.k8[...] = 0
    for j, kv in zip(keys, kvals):
        p.k8[:, :, j, 0] = kv
    p.q_scale[...] = 1.0
    p.k_scale[...] = 1.0
    return p


@pytest.mark.parametrize("N,nseg,jstar", [(1000, 4, 0), (1000, 4, 256), (1000, 4, 255), (1000, 4, 999),
                                          (1000, 16, 577), (300, 5, 64), (300, 5, 63)])
def test_one_hot_row_selects_key(oracle_lib, N, nseg, jstar):
    # the dominant key's segment has the maximum; every other segment's weight
    # exp2(m_s - M) underflows to 0, so O is the key's dequantized V row
    # (keys 255/256 and 63/64 sit on segment boundaries)
    rng = np.random.default_rng(42)
    Hq, Hkv, D = 4, 2, 128
    p = _one_hot(N, Hq, Hkv, D, [jstar], [127], rng)
    rows = np.array([[0, h, i] for h in range(Hq) for i in (0, N - 1)])
    o = oracle_lib.bf16_to_f32(oracle_lib.attn_rows_segmented(p, rows, nseg))
    for r, (_, h, _) in enumerate(rows):
        hk = h // (Hq // Hkv)
        v = oracle_lib.e4m3_to_f32(p.v8[0, hk, jstar]).astype(np.float64) * p.v_scale[0, hk]
        exact = 448.0 / P_PEAK * v
        assert np.all(np.abs(o[r] - exact) <= np.abs(exact) * 2.0**-8 + 1e-30)


@pytest.mark.parametrize("j1,j2,k1,k2", [(10, 700, 100, 98), (700, 10, 98, 100), (30, 900, 80, 79)])
def test_two_keys_in_two_segments_weigh_by_score_gap(oracle_lib, j1, j2, k1, k2):
    # Two keys in different segments carry scores s1, s2 (about 80-100 in
    # log2 units, a unit of k8 worth about 1) far above every other key
    # (which scores 0).  Each segment's own p for its key is exp2(8.807) ->
    # 448, and the combine weighs the segments by exp2(m_s - M) =
    # 2^(s_s - max), so O is the softmax average of the two V rows:
    # (448 / exp2(8.807)) (w1 v1 + w2 v2) / (w1 + w2), w = 2^s.
    rng = np.random.default_rng(43)
    N, D = 1000, 128
    p = _one_hot(N, 1, 1, D, [j1, j2], [k1, k2], rng)
    p.q_scale[...] = 0.0625
    o = oracle_lib.bf16_to_f32(oracle_lib.attn_rows_segmented(p, np.array([[0, 0, 5]]), 2))[0]
    c = (1.0 / math.sqrt(D)) * math.log2(math.e)
    s1, s2 = 127 * k1 * 0.0625 * c, 127 * k2 * 0.0625 * c
    w1, w2 = 2.0 ** (s1 - max(s1, s2)), 2.0 ** (s2 - max(s1, s2))
    v1 = oracle_lib.e4m3_to_f32(p.v8[0, 0, j1]).astype(np.float64)
    v2 = oracle_lib.e4m3_to_f32(p.v8[0, 0, j2]).astype(np.float64)
    exact = 448.0 / P_PEAK * (w1 * v1 + w2 * v2) / (w1 + w2) * p.v_scale[0, 0]
    tol = np.abs(exact) * 2.0**-7 + 1e-3 * np.abs(exact).max()
    assert np.all(np.abs(o - exact) <= tol)
    # the two V rows really are mixed (neither weight is negligible)
    assert 0.01 < min(w1, w2) / (w1 + w2) < 0.5


@pytest.mark.parametrize("N,Hq,Hkv,D,nseg", [(1000, 4, 2, 128, 2), (1000, 4, 2, 128, 5), (1000, 2, 2, 128, 16),
                                             (333, 2, 1, 256, 3), (333, 2, 1, 256, 6)])
def test_matches_fp64_on_dequantized_tensors(oracle_lib, N, Hq, Hkv, D, nseg):
    # as for the exact schedule: only the E4M3 rounding of P (now relative to
    # each segment's own maximum) and FP32 sums separate it from FP64 softmax
    rng = np.random.default_rng(44)
    p = _synthetic(1, N, Hq, Hkv, D, rng)
    p.q_scale[...] *= np.float32(1.5)
    rows = np.array([[0, h, i] for h in range(Hq) for i in range(0, N, max(1, N // 40))] +
                    [[0, Hq - 1, N - 1]])
    o = oracle_lib.bf16_to_f32(oracle_lib.attn_rows_segmented(p, rows, nseg)).astype(np.float64)
    ref = _dequant_attention_f64(p, rows)
    scale = np.abs(ref).max(axis=1, keepdims=True)
    assert np.max(np.abs(o - ref) / scale) < 0.04
    assert oracle.cosine(o, ref) > 0.999


@pytest.mark.parametrize("name,nseg", [("tiny", 2), ("tiny", 4), ("tail", 3), ("tail", 16)])
def test_accuracy_vs_fp64_unquantized(oracle_lib, name, nseg):
    inp = workloads.make_inputs(workloads.CONFIGS[name])
    p = oracle.prepare(inp)
    o = oracle_lib.bf16_to_f32(oracle.attention_segmented(p, nseg))
    ref = oracle.reference_attention_f64(p.zq, p.zk, inp.v)
    assert oracle.cosine(o, ref) >= 0.99


def test_segmentation_changes_some_bits_but_not_the_result(oracle_lib):
    # non-exact: P is rounded to E4M3 against each segment's own maximum, so
    # some outputs differ from the exact schedule, within its tolerance
    inp = workloads.make_inputs(workloads.CONFIGS["tiny"])
    p = oracle.prepare(inp)
    a = oracle_lib.bf16_to_f32(oracle.attention(p)).astype(np.float64)
    b = oracle_lib.bf16_to_f32(oracle.attention_segmented(p, 4)).astype(np.float64)
    assert (a != b).mean() > 0.01
    assert np.abs(a - b).max() < 2e-2 and oracle.cosine(a, b) > 0.999


@pytest.mark.parametrize("nseg", [2, 8, 16])
def test_segmented_is_no_farther_from_fp64_than_exact(oracle_lib, nseg):
    # with outlier rows (x20) the quantization error dominates: a segment's
    # P keeps E4M3 precision against its own maximum, so the segmented
    # output is at least as close to FP64 softmax attention as the exact one
    inp = workloads.make_inputs(workloads.CONFIGS["tail"])
    p = oracle.prepare(inp)
    ref = oracle.reference_attention_f64(p.zq, p.zk, inp.v)
    a = oracle_lib.bf16_to_f32(oracle.attention(p)).astype(np.float64)
    b = oracle_lib.bf16_to_f32(oracle.attention_segmented(p, nseg)).astype(np.float64)
    assert np.abs(b - ref).max() <= np.abs(a - ref).max() * 1.05
    assert oracle.cosine(b, ref) >= oracle.cosine(a, ref) - 1e-5


def test_refuses_segment_counts_outside_the_tiles(oracle_lib):
    rng = np.random.default_rng(45)
    p = _synthetic(1, 130, 1, 1, 128, rng)        # 3 key tiles
    with pytest.raises(ValueError):
        oracle_lib.attn_rows_segmented(p, np.array([[0, 0, 0]]), 0)
    with pytest.raises(ValueError):
        oracle_lib.attn_rows_segmented(p, np.array([[0, 0, 0]]), 4)
