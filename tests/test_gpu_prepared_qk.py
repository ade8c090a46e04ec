"""Steps 1-3 of the Contract's "Preparation" pinned on their own: the optional
BF16 outputs q_prep / k_prep of sage_quant_qk (Q and K after RMSNorm and RoPE,
before any rotation and before the K mean is subtracted) are byte-identical to
the oracle's prepared Q and K, on every config including the full canonical
interleaved problem.  A wrong rounding here could otherwise hide behind the
INT8 quantization that follows."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, shape_of, to_device

pytestmark = pytest.mark.gpu


def _check(inp, label):
    import quantized_exact_order_amd as sage
    banner(f"prepared Q/K {label}: N={inp.q.shape[1]} Hq={inp.cfg.Hq} Hkv={inp.cfg.Hkv} D={inp.cfg.D}")
    dev = to_device(inp)
    shape = shape_of(inp)
    bufs = sage.Buffers.allocate(shape, "cuda", prep_outputs=True)
    args = (dev["q"], dev["k"], dev["v"], dev["w_q"], dev["w_k"], dev["cos"], dev["sin"])
    sage.prep(shape, bufs, *args)
    sage.quant_qk(shape, bufs, *args)
    torch.cuda.synchronize()
    ref = oracle.prepare(inp)
    for name, want in (("q_prep", ref.zq), ("k_prep", ref.zk)):
        got = getattr(bufs, name).cpu().view(torch.int16).numpy().view(np.uint16)
        bad = got != want
        assert not bad.any(), (f"{label} {name}: {int(bad.sum())} of {bad.size} BF16 values differ, "
                               f"first at {np.argwhere(bad)[0].tolist()}")
    print(f"[gpu] prepared Q/K {label}: identical", flush=True)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["tiny", "tail", "gqa", "canonical"])
def test_prepared_q_and_k_match_the_oracle(name):
    _check(workloads.make_inputs(workloads.CONFIGS[name]), name)


def test_prepared_q_and_k_per_element_rope_and_inf():
    # R/2 = 20 is not a multiple of 8 (the per-element RoPE path); one +Inf in a
    # Q row makes that row NaN and zeros, as in the oracle
    inp = workloads.make_custom(2, 150, 4, 2, 128, 40, seed=810, weights=(0.5, 1.5))
    inp.q[1, 70, 3, 5] = float("inf")
    _check(inp, "rope_dim=40, Inf")
