"""The canonical boundary printed on the contract page (tests/golden/
canonical_boundary.json) against the synthetic workload and the oracle's
shape conventions."""
import json
import os

import numpy as np

import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "canonical_boundary.json")))


def test_canonical_workload_matches_printed_boundary():
    cfg = workloads.CONFIGS["canonical"]
    assert (cfg.B, cfg.N, cfg.Hq, cfg.D) == (GOLD["batch"], GOLD["seq"], GOLD["heads"], GOLD["head_dim"])
    assert (cfg.Hq + 2 * cfg.Hkv) * cfg.D == GOLD["qkv_row_width"]
    assert [0, cfg.Hq * cfg.D, (cfg.Hq + cfg.Hkv) * cfg.D] == GOLD["qkv_offsets"]
    assert cfg.rope_dim == GOLD["rope_dims"][1] and cfg.eps == GOLD["rmsnorm_eps"]


def test_interleaved_views_have_printed_strides():
    # small N, same head geometry: strides of the B and N axes scale with N
    cfg = workloads.CONFIGS["canonical"]
    inp = workloads.make_inputs(cfg, N=8)
    W = GOLD["qkv_row_width"]
    for t, off in zip((inp.q, inp.k, inp.v), GOLD["qkv_offsets"]):
        assert t.stride() == (8 * W, W, 128, 1)
        assert t.storage_offset() == off
    assert GOLD["qkv_strides"][0] == GOLD["seq"] * W


def test_scale_and_tile_counts():
    N = GOLD["seq"]
    assert [1, GOLD["heads"], ((N + 127) // 128) * 4] == GOLD["q_scale_shape"]
    assert [1, GOLD["heads"], (N + 63) // 64] == GOLD["k_scale_shape"]
    assert (N + 63) // 64 - 1 == GOLD["last_kv_tile"]
    assert ((N + 63) // 64) * 64 == GOLD["v_padded_rows"]
    assert N - 128 * (N // 128) == GOLD["tail_valid_rows_q128"]
    assert N - 64 * (N // 64) == GOLD["tail_valid_rows_k64"]


def test_fp8_offset_keeps_peak_probability_finite(oracle_lib):
    # 2^8.807 rounds to the largest E4M3 value and never saturates past it
    peak = np.float32(2.0 ** GOLD["fp8_offset"])
    assert peak < 448.0 and oracle_lib.f32_to_e4m3(np.float32([peak]))[0] == 0x7E
    # the PV page's bound: 448 * 2.25 * 64 keys stays below the FP16 maximum
    assert 448 * GOLD["v_fp8_divisor"] * 64 < 65504


def test_oracle_shapes_on_ragged_length(oracle_lib):
    import oracle
    inp = workloads.make_custom(1, 50, 2, 2, 128, 96, seed=7)
    p = oracle.prepare(inp)
    assert p.q_scale.shape == (1, 2, 4) and p.k_scale.shape == (1, 2, 1)
    assert p.q8.shape == (1, 2, 50, 128) and p.v8.shape == (1, 2, 50, 128)
