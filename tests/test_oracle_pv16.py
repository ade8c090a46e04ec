"""The oracle's emulation of the page's two-level PV accumulation (each 64-key
partial accumulated in FP16 by two ordered K=32 steps, then added to the FP32
running output) against its FP32 per-tile reading.  The FP16 partial rounds
twice per tile with relative error at most 2^-11 of that tile's partial, so
the two modes agree to well within the output tolerance (measured: tiny, 10% of
outputs differ, max-abs 0.002; tail with x20 outliers, max-abs 0.016), while a
wrong step order or a lost term would move whole rows."""
import numpy as np

import oracle
import workloads


def _modes(name, rows=None):
    inp = workloads.make_inputs(workloads.CONFIGS[name])
    p = oracle.prepare(inp)
    if rows is None:
        a, b = oracle.attention(p), oracle.attention(p, pv_fp16=True)
    else:
        a, b = oracle.attn_rows(p, rows), oracle.attn_rows(p, rows, pv_fp16=True)
    return oracle.bf16_to_f32(a).astype(np.float64), oracle.bf16_to_f32(b).astype(np.float64)


def test_fp16_partials_stay_close_tiny():
    a, b = _modes("tiny")
    assert oracle.cosine(a, b) > 0.99999
    assert np.abs(a - b).max() < 4e-3
    assert 0.01 < (a != b).mean() < 0.5             # the emulation changes some bits, not all


def test_fp16_partials_stay_close_tail_outliers():
    a, b = _modes("tail")
    assert oracle.cosine(a, b) > 0.99999
    assert np.abs(a - b).max() < 2e-2
