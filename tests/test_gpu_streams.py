"""The library keeps no state between calls: independent problems issued on
separate HIP streams, with their calls interleaved on the host, give exactly
the bytes that the same problems give one after the other on one stream."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import banner, host_tensors, run_path, shape_of, to_device

pytestmark = pytest.mark.gpu


def test_independent_problems_on_separate_streams():
    import quantized_exact_order_amd as sage
    banner("three independent problems on three streams, calls interleaved")
    probs = [workloads.make_custom(1, 3000, 8, 8, 128, 96, seed=301),
             workloads.make_custom(2, 1500, 4, 2, 256, 192, seed=302, hadamard=True),
             workloads.make_custom(1, 700, 6, 3, 128, 0, seed=303, interleaved=True)]
    devs = [to_device(p) for p in probs]
    shapes = [shape_of(p) for p in probs]
    seq = [run_path(p, dev=d, shape=s) for p, d, s in zip(probs, devs, shapes)]
    ref = [(host_tensors(s, b), o.clone()) for s, b, o in seq]

    streams = [torch.cuda.Stream() for _ in probs]
    bufs = [sage.Buffers.allocate(s, "cuda") for s in shapes]
    outs = [torch.empty_like(o) for _, o in ref]
    for b in bufs:
        for t in (b.q8, b.k8, b.v8):
            t.fill_(0x5A)
    for o in outs:
        o.zero_()
    torch.cuda.synchronize()
    args = [(d["q"], d["k"], d["v"], d["w_q"], d["w_k"], d["cos"], d["sin"]) for d in devs]
    for i in range(3):
        sage.prep(shapes[i], bufs[i], *args[i], stream=streams[i])
    for i in range(3):
        sage.quant_qk(shapes[i], bufs[i], *args[i], stream=streams[i])
    for i in range(3):
        sage.attn_fwd(shapes[i], bufs[i], o=outs[i], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(3):
        got = host_tensors(shapes[i], bufs[i])
        for name, t in ref[i][0].items():
            assert np.array_equal(got[name].view(np.uint8), t.view(np.uint8)), (i, name)
        assert torch.equal(outs[i].view(torch.int16), ref[i][1].view(torch.int16)), i
