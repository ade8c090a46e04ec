"""The Python binding refuses, before any launch, arguments that the C ABI
cannot check: host or short side inputs (RMSNorm weights, RoPE tables),
views whose shape disagrees with the problem shape, buffers allocated for
another shape, and decode inputs that do not match the cache."""
import pytest
import torch

import workloads
from gpu_util import banner, shape_of, to_device

pytestmark = pytest.mark.gpu


def test_side_inputs_and_views_are_checked():
    import quantized_exact_order_amd as sage
    banner("binding argument checks")
    inp = workloads.make_inputs(workloads.CONFIGS["tiny"])
    dev = to_device(inp)
    shape = shape_of(inp)
    bufs = sage.Buffers.allocate(shape, "cuda")
    args = dict(q=dev["q"], k=dev["k"], v=dev["v"], w_q=dev["w_q"], w_k=dev["w_k"], cos=dev["cos"], sin=dev["sin"])

    def call(**over):
        a = {**args, **over}
        sage.prep(shape, bufs, a["q"], a["k"], a["v"], a["w_q"], a["w_k"], a["cos"], a["sin"])

    with pytest.raises(ValueError, match="w_q"):
        call(w_q=dev["w_q"].cpu())                             # a host pointer
    with pytest.raises(ValueError, match="cos"):
        call(cos=dev["cos"][:-1])                              # a short RoPE table
    with pytest.raises(ValueError, match="sin"):
        call(sin=dev["sin"].float())                           # wrong dtype
    with pytest.raises(ValueError, match="k must have shape"):
        call(k=dev["k"][:, :-1])                               # fewer rows than N
    other = sage.Buffers.allocate(shape_of(inp, N=shape.N - 64), "cuda")
    with pytest.raises(ValueError, match="buffer"):
        sage.attn_fwd(shape, other)
    call()                                                     # the valid call still runs
    torch.cuda.synchronize()


def test_decode_inputs_must_match_the_cache():
    import quantized_exact_order_amd as sage
    banner("binding decode checks")
    cache = sage.KvCache.allocate(1, 2, 64, "cuda")
    k = torch.zeros((1, 8, 2, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="k and v"):
        sage.kv_append(cache, k, k[:, :, :1], 0)
    with pytest.raises(ValueError, match="q must have shape"):
        sage.decode_attn(cache, torch.zeros((2, 4, 256), dtype=torch.bfloat16, device="cuda"), 8)
