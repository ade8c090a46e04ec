"""Pins of the oracle's number formats against independent definitions.

The oracle's BF16 / E4M3 / INT8 / exp2 routines are checked against library
routines that implement the same format (torch's float32->bfloat16 and
float8_e4m3fn conversions, numpy's rint), against format facts of OCP E4M3
(max 448, smallest subnormal 2^-9, no infinities) and against FP64 exp2.
"""
import math

import numpy as np
import pytest
import torch


def _patterns_with_ties():
    """Every upper-16-bit pattern combined with low halves that include the
    BF16 rounding ties and their neighbours."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF], np.uint32)
    return (hi[:, None] | lows[None, :]).ravel()


def test_bf16_matches_torch_on_all_exponents_and_ties(oracle_lib):
    bits = _patterns_with_ties()
    rng = np.random.default_rng(0)
    bits = np.concatenate([bits, rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)])
    x = bits.view(np.float32)
    mine = oracle_lib.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(mine[~nan], ref[~nan])
    # NaN stays NaN with its sign
    got = oracle_lib.bf16_to_f32(mine[nan])
    assert np.all(np.isnan(got))
    assert np.array_equal(mine[nan] >> 15, (bits[nan] >> 31).astype(np.uint16))


def test_bf16_round_half_even_spot_values(oracle_lib):
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert oracle_lib.f32_to_bf16(np.float32([1.0 + 2**-8]))[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> 1+2^-6
    assert oracle_lib.f32_to_bf16(np.float32([1.0 + 3 * 2**-8]))[0] == 0x3F82
    # largest finite float rounds to infinity
    assert oracle_lib.f32_to_bf16(np.float32([np.finfo(np.float32).max]))[0] == 0x7F80


def test_e4m3_decode_matches_torch_all_codes(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle_lib.e4m3_to_f32(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # format facts: max finite 448 at 0x7E, NaN at 0x7F, smallest subnormal 2^-9
    assert mine[0x7E] == 448.0 and np.isnan(mine[0x7F]) and mine[0x01] == 2.0**-9
    assert mine[0x08] == 2.0**-6 and mine[0xFE] == -448.0


def test_e4m3_encode_matches_torch_below_saturation(oracle_lib):
    rng = np.random.default_rng(1)
    # all values on a dense grid straddling every E4M3 binade, all midpoints
    # between neighbouring codes (ties), and random floats
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = oracle_lib.e4m3_to_f32(codes).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0
    grid = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    rnd = np.exp(rng.uniform(np.log(2.0**-12), np.log(448.0), size=1 << 20))
    x = np.concatenate([grid, rnd, [0.0, 2.0**-11, 2.0**-10, 3 * 2.0**-10]]).astype(np.float32)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) < 448.0]
    mine = oracle_lib.f32_to_e4m3(x)
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e4m3_saturates_finite(oracle_lib):
    x = np.float32([448.0, 449.0, 463.9, 464.0, 1e6, np.inf, -500.0, -np.inf])
    got = oracle_lib.f32_to_e4m3(x)
    assert list(got) == [0x7E] * 6 + [0xFE, 0xFE]
    assert oracle_lib.f32_to_e4m3(np.float32([np.nan]))[0] & 0x7F == 0x7F
    # the softmax peak 2^8.807 is just below 448 and rounds to 448
    assert oracle_lib.f32_to_e4m3(np.float32([2.0**8.807]))[0] == 0x7E


def test_i8_round_half_even_saturate(oracle_lib):
    rng = np.random.default_rng(2)
    halves = np.arange(-140, 140, dtype=np.float32) + np.float32(0.5)
    x = np.concatenate([halves, rng.uniform(-200, 200, 1 << 18).astype(np.float32),
                        np.float32([0.49999997, -0.49999997, 127.49999, 127.5, -128.5, -1e9, 1e9])])
    mine = oracle_lib.f32_to_i8(x)
    ref = np.clip(np.rint(x.astype(np.float64)), -128, 127).astype(np.int8)
    assert np.array_equal(mine, ref)
    assert oracle_lib.f32_to_i8(np.float32([np.nan]))[0] == 0


def test_exp2_fp64_rounded_with_flush(oracle_lib):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-140, 9, 1 << 18), [0.0, -126.0, -126.5, -149.0, -5e6, 8.807]]).astype(np.float32)
    got = oracle_lib.exp2(x)
    ref = np.exp2(x.astype(np.float64)).astype(np.float32)
    ref[ref < np.float32(2.0**-126)] = 0.0
    assert np.array_equal(got, ref)
    assert got[-2] == 0.0   # exp2(-5e6) vanishes: the first tile wipes d0 = 1


@pytest.mark.parametrize("D", [128, 256])
def test_score_scale_is_log2e_over_sqrt_d(oracle_lib, D):
    c = oracle_lib.score_scale(D)
    # c * sqrt(D) * ln 2 == 1 up to the single FP32 rounding of c
    assert abs(c * math.sqrt(D) * math.log(2.0) - 1.0) < 2.0**-23
    expected_bits = {128: 0x3E0293EE, 256: 0x3DB8AA3B}[D]
    assert np.float32(c).view(np.uint32) == expected_bits


def test_f16_rounding_matches_numpy():
    import oracle
    rng = np.random.default_rng(3)
    # every binary16 value, the midpoints between neighbours (ties) and their
    # neighbours in double, plus random doubles over the whole range
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2
    xs = np.concatenate([h, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                         rng.uniform(-70000, 70000, 4000), rng.standard_normal(4000) * 1e-5,
                         [65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25]])
    xs = np.concatenate([xs, -xs])
    mine = np.array([oracle.f64_to_f16(x) for x in xs], np.float64)
    with np.errstate(over="ignore"):              # values >= 65520 become inf, as in the oracle
        ref = xs.astype(np.float16).astype(np.float64)
    same = (mine == ref) | (np.isinf(mine) & np.isinf(ref) & (np.sign(mine) == np.sign(ref)))
    assert same.all(), xs[~same][:5]
