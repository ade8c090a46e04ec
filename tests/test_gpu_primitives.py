"""Exhaustive check of the device number-format primitives of the preparation
(sage_selftest_primitive) over FP32 bit patterns, element by element:

- BF16, INT8 and E4M3 rounding over all 2^32 patterns, against the oracle's
  own conversion routines (the page "Exact Numerical Contract", sections
  "Preparation", "Q And K Quantization" and "V And PV": round to nearest
  even; INT8 saturating with NaN -> 0; E4M3 saturating to +-448);
- the reciprocal square root of RMSNorm and the scale divisions and
  multipliers, over every non-negative pattern (their inputs are sums of
  squares and maxima), against numpy's correctly rounded float32 division
  and square root;
- the accuracy of the softmax exponential (not a bit-exact output) over every
  argument from -126 to 8.81, against FP64;
- the lane exchanges of the preparation and decode reductions (DPP, permlane
  moves): element i of every wave receives element i ^ M, bits unchanged.

Results must be bit-identical; where both sides give NaN the payloads are not
compared."""
import time

import numpy as np
import pytest
import torch

import oracle
from gpu_util import banner

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26
POS_END = 0x7F800001          # patterns [0, POS_END): +0 up to +inf


def _reference(kind, x):
    if kind == 0:
        return oracle.f32_to_bf16(x).view(np.int16)
    if kind == 1:
        return oracle.f32_to_i8(x)
    if kind in (2, 9):
        return oracle.f32_to_e4m3(x)
    with np.errstate(all="ignore"):
        if kind == 3:
            return np.float32(1.0) / np.sqrt(x)
        if kind == 4:
            return x / np.float32(127.0)
        if kind == 5:
            return np.float32(127.0) / x
        if kind == 6:
            return x / np.float32(2.25)
        return np.float32(2.25) / x


def _sweep(kind, end, keep=None):
    import quantized_exact_order_amd as sage
    banner(f"primitive {kind}: patterns [0, {end:#x})")
    t0 = time.time()
    out = None
    first = 0
    while first < end:
        n = min(CHUNK, end - first)
        out = sage.selftest_primitive(kind, first, n, out)
        torch.cuda.synchronize()
        got = out[:n].cpu().numpy()
        bits = np.arange(n, dtype=np.uint32) + np.uint32(first)
        ref = _reference(kind, bits.view(np.float32))
        if 3 <= kind <= 8:
            g, r = got.view(np.uint32), ref.view(np.uint32)
            bad = (g != r) & ~(np.isnan(got) & np.isnan(ref))
        else:
            bad = got != ref
        if keep is not None:
            bad &= keep(bits.view(np.float32))
        if bad.any():
            i = int(np.flatnonzero(bad)[0])
            pytest.fail(f"kind {kind}: pattern {int(bits[i]):#010x} gives {got[i]!r} on the GPU, "
                        f"{ref[i]!r} in the reference ({int(bad.sum())} of {n} in this chunk)")
        first += n
    print(f"[gpu] primitive {kind}: {end} patterns identical ({time.time() - t0:.1f} s)", flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kind", [0, 1, 2])
def test_format_conversions_over_all_patterns(kind):
    _sweep(kind, 1 << 32)


@pytest.mark.timeout(600)
def test_hardware_e4m3_conversion_below_448():
    # the V cast converts with the hardware instruction (and redoes NaN
    # words in software); its values are at most 2.25 in magnitude
    # (|v| <= amax times 2.25 / amax).  Every pattern of magnitude below 448,
    # and every NaN, converts as the oracle's OCP E4M3 does (round to nearest
    # even, subnormals down to 2^-9, NaN keeping its sign)
    def keep(x):
        with np.errstate(invalid="ignore"):
            return np.isnan(x) | (np.abs(x) < 448.0)
    _sweep(9, 1 << 32, keep)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kind", [3, 4, 5, 6, 7])
def test_scale_arithmetic_over_non_negative_patterns(kind):
    _sweep(kind, POS_END)


def _exp2_ulp_errors(first, end):
    import quantized_exact_order_amd as sage
    worst, worst_x, out = 0.0, None, None
    while first < end:
        n = min(CHUNK, end - first)
        out = sage.selftest_primitive(8, first, n, out)
        torch.cuda.synchronize()
        got = out[:n].cpu().numpy().astype(np.float64)
        x = (np.arange(n, dtype=np.uint32) + np.uint32(first)).view(np.float32)
        exact = np.exp2(x.astype(np.float64))
        ulp = np.spacing(exact.astype(np.float32)).astype(np.float64)
        err = np.abs(got - exact) / ulp
        i = int(np.argmax(err))
        if err[i] > worst:
            worst, worst_x = float(err[i]), float(x[i])
        first += n
    return worst, worst_x


@pytest.mark.timeout(600)
def test_softmax_exponential_accuracy():
    # every FP32 argument the softmax can pass down to -126 (below, the results
    # are subnormal and the oracle flushes them): 2^x from the attention kernel's
    # own instruction against FP64, in units of the FP32 ulp of the exact value.
    # The oracle rounds exp2 once (error <= 0.5 ulp); the device stays within
    # one ulp (measured maximum 0.78), which the tolerance reading of the
    # attention output rests on
    banner("softmax exponential: x in [-126, 8.81]")
    hi = int(np.float32(8.81).view(np.uint32))
    lo = int(np.float32(-126.0).view(np.uint32))
    w_pos, x_pos = _exp2_ulp_errors(0, hi + 1)
    w_neg, x_neg = _exp2_ulp_errors(0x80000000, lo + 1)
    worst = max(w_pos, w_neg)
    print(f"[gpu] v_exp_f32: max error {w_pos:.3f} ulp at x = {x_pos!r} (x >= 0), {w_neg:.3f} ulp at "
          f"x = {x_neg!r} (x < 0)", flush=True)
    assert worst <= 1.0


@pytest.mark.parametrize("kind", range(10, 16))
def test_lane_exchange_moves_the_partner_lanes_bits(kind):
    # patterns around 1.0, and a range of NaN payloads: a move keeps every bit
    import quantized_exact_order_amd as sage
    m = 1 << (kind - 10)
    banner(f"lane exchange xor {m}")
    for first in (0x3F800000, 0x7FC00000 - 2048, 0xFF800000 - 4096):
        n = 8192
        out = sage.selftest_primitive(kind, first, n).view(torch.int32).cpu().numpy().view(np.uint32)
        i = np.arange(n, dtype=np.uint64)
        want = (np.uint64(first) + (i ^ np.uint64(m))).astype(np.uint32)
        assert np.array_equal(out, want), (m, hex(first), int(np.count_nonzero(out != want)))
