"""The Python binding refuses, before any launch, arguments that the C ABI
cannot check: host or short side inputs (RMSNorm weights, RoPE tables),
views whose shape disagrees with the problem shape, buffers allocated for
another shape or of another dtype, host or short workspaces, and decode
inputs or cache tensors that do not agree."""
import pytest
import torch

import workloads
from gpu_util import banner, run_path, shape_of, to_device

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


def test_workspaces_and_buffer_dtypes_are_checked():
    import quantized_exact_order_amd as sage
    banner("binding workspace and dtype checks")
    inp = workloads.make_inputs(workloads.CONFIGS["tiny"])
    shape, bufs, _ = run_path(inp, attn=False)
    need = sage.attn_segmented_workspace(shape, 2)
    with pytest.raises(ValueError, match="workspace"):
        sage.attn_fwd_segmented(shape, bufs, 2, workspace=torch.empty(need, dtype=torch.uint8))   # host memory
    with pytest.raises(ValueError, match="workspace"):
        sage.attn_fwd_segmented(shape, bufs, 2, workspace=torch.empty(need - 1, dtype=torch.uint8, device="cuda"))
    good = bufs.q_scale
    bufs.q_scale = torch.empty(good.shape, dtype=torch.int8, device="cuda")       # right shape, 1/4 the bytes
    with pytest.raises(ValueError, match="q_scale"):
        sage.attn_fwd(shape, bufs)
    bufs.q_scale = good
    sage.attn_fwd(shape, bufs)                                                  # the valid call still runs
    torch.cuda.synchronize()


def test_cache_tensors_and_decode_outputs_are_checked():
    import quantized_exact_order_amd as sage
    banner("binding cache checks")
    cache = sage.KvCache.allocate(1, 2, 64, "cuda")
    q = torch.zeros((1, 4, 256), dtype=torch.bfloat16, device="cuda")
    need = sage.decode_workspace(cache, 4, 8)
    with pytest.raises(ValueError, match="workspace"):
        sage.decode_attn(cache, q, 8, workspace=torch.empty(need, dtype=torch.uint8))            # host memory
    with pytest.raises(ValueError, match="o must"):
        sage.decode_attn(cache, q, 8, o=torch.empty((1, 4, 256), dtype=torch.bfloat16))          # host output
    short = sage.KvCache(cache.k8, cache.k_scale[:, :, :32].contiguous(), cache.v)              # scales of 32 tokens
    with pytest.raises(ValueError, match="cache tensors"):
        sage.decode_attn(short, q, 8)
    host = sage.KvCache(cache.k8, cache.k_scale, cache.v.cpu())
    with pytest.raises(ValueError, match="cache tensors"):
        sage.kv_append(host, torch.zeros((1, 8, 2, 256), dtype=torch.bfloat16, device="cuda"),
                       torch.zeros((1, 8, 2, 256), dtype=torch.bfloat16, device="cuda"), 0)
    sage.decode_attn(cache, q, 8)                                               # the valid call still runs
    torch.cuda.synchronize()
