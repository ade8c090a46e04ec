"""The allocation-free decode entry point (sage_decode_attn_noalloc) against
sage_decode_attn with a caller workspace, through the C ABI: the same kernels,
so the outputs must be byte-identical, on two calls in a row (the second with
a smaller problem, over the partials the first left in the fixed array), for
the BF16-V and the INT8-V cache; and a problem whose partials exceed the
fixed array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import banner

pytestmark = pytest.mark.gpu

D = 256


def _filled_cache(sage, rng, B, Hkv, T, int8_v):
    kv = torch.from_numpy(rng.standard_normal((B, T, 2 * Hkv * D)).astype(np.float32)).to(torch.bfloat16).cuda()
    k = kv[:, :, :Hkv * D].view(B, T, Hkv, D)
    v = kv[:, :, Hkv * D:].view(B, T, Hkv, D)
    cache = sage.KvCache.allocate(B, Hkv, T, "cuda", int8_v=int8_v)
    sage.kv_append(cache, k, v, 0)
    return cache


def _c_noalloc(sage, cache, q, T, o):
    """sage_decode_attn_noalloc called through the C ABI directly."""
    B, Hq, _ = q.shape
    qv = sage._view(q.unsqueeze(1), "q")
    st = sage.lib.sage_decode_attn_noalloc(ctypes.byref(cache.c()), Hq, ctypes.byref(qv), T, o.data_ptr(),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("int8_v", [False, True])
def test_noalloc_decode_matches_workspace_decode(int8_v):
    import quantized_exact_order_amd as sage
    rng = np.random.default_rng(900 + int8_v)
    B, Hkv = 2, 4
    cache = _filled_cache(sage, rng, B, Hkv, 20000, int8_v)
    # first call: 16 query heads over 20,000 tokens; second: 8 heads over 3,001
    for Hq, T in ((16, 20000), (8, 3001)):
        banner(f"noalloc decode int8_v={int8_v} B={B} Hq={Hq} Hkv={Hkv} T={T}")
        need = sage.decode_workspace(cache, Hq, T)
        assert need <= sage.decode_noalloc_max_bytes()
        q = torch.from_numpy(rng.standard_normal((B, Hq, D)).astype(np.float32)).to(torch.bfloat16).cuda()
        o_ws = sage.decode_attn(cache, q, T)
        o_na = torch.full((B, Hq, D), 7.0, dtype=torch.bfloat16, device="cuda")
        assert _c_noalloc(sage, cache, q, T, o_na) == 0
        torch.cuda.synchronize()
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16))


def test_noalloc_decode_refuses_partials_beyond_the_array():
    import quantized_exact_order_amd as sage
    # B = 8 sequences of 16 query heads over 262,144 tokens: 128 chunks of
    # 2,048 tokens, 17.0 MB of partials, more than the 16 MiB array
    B, Hkv, Hq, T = 8, 1, 16, 262144
    banner(f"noalloc decode refusal B={B} Hq={Hq} T={T}")
    cache = sage.KvCache.allocate(B, Hkv, T, "cuda")
    assert sage.decode_workspace(cache, Hq, T) > sage.decode_noalloc_max_bytes()
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    o = torch.full((B, Hq, D), 7.0, dtype=torch.bfloat16, device="cuda")
    assert _c_noalloc(sage, cache, q, T, o) == 7            # SAGE_E_WORKSPACE, before any launch
    torch.cuda.synchronize()
    assert (o == 7.0).all()
