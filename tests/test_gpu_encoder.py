"""The short-encoder workload (27 independent layers, N=729, H=16, D=128) run
as one call with the layers stacked along the batch dimension, and as per-layer
calls captured in a HIP graph: both must give exactly the bytes of per-layer
eager calls, and a stacked layer must meet the oracle bar."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (assert_prep_bit_exact, banner, bf16_bits, compare_output, host_tensors)

pytestmark = pytest.mark.gpu

L = 27


def _stacked_inputs(n_layers, dev):
    cfg = workloads.CONFIGS["encoder"]
    layers = [workloads.make_inputs(cfg, layer=l) for l in range(n_layers)]
    q = torch.cat([x.q for x in layers]).to(dev)
    k = torch.cat([x.k for x in layers]).to(dev)
    v = torch.cat([x.v for x in layers]).to(dev)
    extra = (layers[0].w_q.to(dev), layers[0].w_k.to(dev), layers[0].cos.to(dev).contiguous(),
             layers[0].sin.to(dev).contiguous())
    return cfg, layers, q, k, v, extra


def _per_layer(sage, cfg, q, k, v, extra, n_layers, bufs=None, o=None):
    one = sage.Shape(1, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.rope_dim, cfg.hadamard, cfg.eps)
    if bufs is None:
        bufs = [sage.Buffers.allocate(one, q.device) for _ in range(n_layers)]
        o = torch.empty((n_layers, cfg.N, cfg.Hq, cfg.D), dtype=torch.bfloat16, device=q.device)
    for l in range(n_layers):
        a = (q[l:l + 1], k[l:l + 1], v[l:l + 1]) + extra
        sage.prep(one, bufs[l], *a)
        sage.quant_qk(one, bufs[l], *a)
        sage.attn_fwd(one, bufs[l], o[l:l + 1])
    return one, bufs, o


def test_stacked_layers_equal_per_layer_calls():
    import quantized_exact_order_amd as sage
    banner("encoder: 27 layers stacked as B=27 vs 27 single-layer calls")
    cfg, layers, q, k, v, extra = _stacked_inputs(L, "cuda")
    one, bufs1, o1 = _per_layer(sage, cfg, q, k, v, extra, L)
    stacked = sage.Shape(L, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.rope_dim, cfg.hadamard, cfg.eps)
    bufsL = sage.Buffers.allocate(stacked, q.device)
    sage.prep(stacked, bufsL, q, k, v, *extra)
    sage.quant_qk(stacked, bufsL, q, k, v, *extra)
    oL = sage.attn_fwd(stacked, bufsL)
    torch.cuda.synchronize()
    assert torch.equal(oL.view(torch.int16), o1.view(torch.int16))
    hs = host_tensors(stacked, bufsL)
    for l in (0, 13, 26):
        h1 = host_tensors(one, bufs1[l])
        for name, t in h1.items():
            assert np.array_equal(t.view(np.uint8), hs[name][l:l + 1].view(np.uint8)), f"layer {l} {name}"
    # one stacked layer against the oracle
    ref = oracle.prepare(layers[13])
    assert_prep_bit_exact(ref, {n: t[13:14] for n, t in hs.items()}, "stacked layer 13")
    o_ref = oracle.bf16_to_f32(oracle.attention(ref))
    compare_output(oracle.bf16_to_f32(bf16_bits(oL[13:14])), o_ref, "stacked layer 13")


def test_hip_graph_replays_match_eager():
    import quantized_exact_order_amd as sage
    n = 3
    banner(f"encoder: per-layer calls of {n} layers captured in a HIP graph, replayed 3 times")
    cfg, layers, q, k, v, extra = _stacked_inputs(n, "cuda")
    one, bufs, o = _per_layer(sage, cfg, q, k, v, extra, n)
    torch.cuda.synchronize()
    eager = o.clone()
    eager_tensors = [host_tensors(one, b) for b in bufs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _per_layer(sage, cfg, q, k, v, extra, n, bufs, o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _per_layer(sage, cfg, q, k, v, extra, n, bufs, o)
    for rep in range(3):
        # eager work between replays: clear the outputs and run an unrelated call
        o.zero_()
        for b in bufs:
            b.q8.zero_()
            b.k_mean.zero_()
        _per_layer(sage, cfg, q.flip(0).contiguous(), k, v, extra, 1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        for l, b in enumerate(bufs):
            for name, t in host_tensors(one, b).items():
                assert np.array_equal(t.view(np.uint8), eager_tensors[l][name].view(np.uint8)), \
                    f"replay {rep} layer {l} {name}"


@pytest.mark.parametrize("nseg", [2, 4, 12])
def test_stacked_segmented_equals_per_layer_segmented(nseg):
    # the segmented mode keeps every (batch, head, query block) on its own,
    # so stacking layers along the batch must not change a byte of any layer
    # (nseg 2 and 4 run in one work-group, 12 in two launches)
    import quantized_exact_order_amd as sage
    n = 3
    banner(f"encoder: {n} layers stacked vs single calls, segmented nseg={nseg}")
    cfg, layers, q, k, v, extra = _stacked_inputs(n, "cuda")
    one, bufs1, _ = _per_layer(sage, cfg, q, k, v, extra, n)
    o1 = torch.stack([sage.attn_fwd_segmented(one, bufs1[l], nseg)[0] for l in range(n)])
    stacked = sage.Shape(n, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.rope_dim, cfg.hadamard, cfg.eps)
    bufsL = sage.Buffers.allocate(stacked, q.device)
    sage.prep(stacked, bufsL, q, k, v, *extra)
    sage.quant_qk(stacked, bufsL, q, k, v, *extra)
    oL = sage.attn_fwd_segmented(stacked, bufsL, nseg)
    torch.cuda.synchronize()
    assert torch.equal(oL.view(torch.int16), o1.view(torch.int16))
