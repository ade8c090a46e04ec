"""The C-ABI library loads, exports every function include/sage.h declares,
sizes buffers, and refuses invalid arguments by name before any launch.
Host-only: no test here launches a kernel."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sage_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def sage():
    import quantized_exact_order_amd as sage
    return sage


def test_library_exports_every_declared_symbol(sage):
    names = _declared_functions()
    assert set(names) == set(sage.EXPORTS), names
    raw = ctypes.CDLL(sage.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_status_strings(sage):
    from quantized_exact_order_amd._lib import lib, STATUS_NAMES
    assert lib.sage_version() >= 100
    for code, name in STATUS_NAMES.items():
        assert lib.sage_status_str(code).decode().startswith(name)


def test_buffer_sizes_canonical(sage):
    import json
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "canonical_boundary.json")))
    z = sage.buffer_sizes(sage.Shape(1, 37810, 56, 56, 128, 96))
    assert z.n_q_groups == gold["q_scale_shape"][2]
    assert z.n_k_tiles == gold["k_scale_shape"][2]
    assert z.k_rows == gold["v_padded_rows"]
    assert z.q_scale == 56 * 1184 * 4 and z.k_scale == 56 * 591 * 4
    assert z.q8 >= 37810 * 56 * 128 and z.q_rows % 256 == 0
    assert z.v8 == 56 * 591 * 128 * 64 and z.k8 == 56 * 37824 * 128
    assert z.workspace >= 2 * 56 * 591 * 128 * 4


def test_v8_slot_order_is_a_permutation(sage):
    keys = sage.v8_slot_keys()
    assert sorted(keys) == list(range(64))
    from quantized_exact_order_amd._lib import lib
    assert lib.sage_v8_key_of_slot(64) == -1 and lib.sage_v8_key_of_slot(-1) == -1


@pytest.mark.parametrize("kw,err", [
    (dict(N=0), "SAGE_E_SHAPE"), (dict(B=0), "SAGE_E_SHAPE"), (dict(D=64), "SAGE_E_SHAPE"),
    (dict(N=(1 << 24) + 1), "SAGE_E_SHAPE"), (dict(Hkv=3), "SAGE_E_GQA"),
    (dict(rope_dim=95), "SAGE_E_ROPE"), (dict(rope_dim=130), "SAGE_E_ROPE"),
    (dict(rope_dim=-2), "SAGE_E_ROPE"), (dict(hadamard=True), "SAGE_E_UNSUPPORTED"),
    (dict(eps=0.0), "SAGE_E_UNSUPPORTED"), (dict(eps=float("nan")), "SAGE_E_UNSUPPORTED"),
    # 4096 * 64 heads * 8192 query tiles of 256 threads: 2^39 work-items in one launch
    (dict(B=4096, Hq=64, Hkv=64, N=1 << 20), "SAGE_E_SHAPE"),
    # the quantization grid, (86 + 171) * 65535 work-groups of 256 threads, past 2^32 - 1
    (dict(Hq=65535, Hkv=65535, N=64 * 171), "SAGE_E_SHAPE"),
])
def test_shape_refusals(sage, kw, err):
    base = dict(B=1, N=100, Hq=4, Hkv=2, D=128, rope_dim=96, hadamard=False, eps=1e-5)
    base.update(kw)
    with pytest.raises(sage.SageError) as ei:
        sage.buffer_sizes(sage.Shape(**base))
    assert ei.value.name == err


def _call_prep(fn, shape, q=None, k=None, v=None, bufs=None, ws=0x10000, ws_bytes=1 << 40,
               cos=0x2000, sin=0x3000, wq=None):
    from quantized_exact_order_amd._lib import SageView, SageBufs
    A = 0x100000
    good = SageView(A, 0, 3 * 4 * 128, 128, 1)
    q = q or good
    k = k or good
    v = v or good
    bufs = bufs or SageBufs(A, A, A, A, A, A, A)
    return fn(ctypes.byref(shape.c()), ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), wq, None,
              cos, sin, ctypes.byref(bufs), ws, ws_bytes, None)


@pytest.mark.parametrize("which", ["sage_prep", "sage_quant_qk"])
def test_pass_refusals_happen_before_launch(sage, which):
    from quantized_exact_order_amd._lib import lib, SageView, SageBufs, STATUS_NAMES
    fn = getattr(lib, which)
    shape = sage.Shape(1, 100, 4, 4, 128, 96)
    A = 0x100000
    name = lambda st: STATUS_NAMES[st]
    assert name(_call_prep(fn, shape, q=SageView(0, 0, 512, 128, 1))) == "SAGE_E_NULL"
    assert name(_call_prep(fn, shape, k=SageView(A, 0, 512, 128, 2))) == "SAGE_E_STRIDE"
    assert name(_call_prep(fn, shape, v=SageView(A + 2, 0, 512, 128, 1))) == "SAGE_E_ALIGN"
    assert name(_call_prep(fn, shape, q=SageView(A, 0, 513, 128, 1))) == "SAGE_E_ALIGN"
    assert name(_call_prep(fn, shape, bufs=SageBufs(A, A, 0, A, A, A, A))) == "SAGE_E_NULL"
    assert name(_call_prep(fn, shape, bufs=SageBufs(A, A, A + 4, A, A, A, A))) == "SAGE_E_ALIGN"
    assert name(_call_prep(fn, shape, ws=0)) == "SAGE_E_WORKSPACE"
    assert name(_call_prep(fn, shape, ws_bytes=16)) == "SAGE_E_WORKSPACE"
    assert name(_call_prep(fn, shape, cos=None)) == "SAGE_E_NULL"
    assert name(_call_prep(fn, shape, cos=0x2002)) == "SAGE_E_ALIGN"
    assert name(_call_prep(fn, shape, wq=0x4008)) == "SAGE_E_ALIGN"
    bad = sage.Shape(1, 100, 4, 4, 128, 97)
    assert name(_call_prep(fn, bad)) == "SAGE_E_ROPE"


def test_attn_refusals_happen_before_launch(sage):
    from quantized_exact_order_amd._lib import lib, SageBufs, STATUS_NAMES
    A = 0x100000
    shape = sage.Shape(1, 100, 4, 2, 128, 96)
    bufs = SageBufs(A, A, A, A, A, A, A)
    call = lambda o, sb, sn, sh, b=bufs: STATUS_NAMES[lib.sage_attn_fwd(
        ctypes.byref(shape.c()), ctypes.byref(b), o, sb, sn, sh, None)]
    assert call(None, 0, 512, 128) == "SAGE_E_NULL"
    assert call(A, 0, 1024, 128) == "SAGE_E_STRIDE"        # rows not contiguous in (h, d)
    assert call(A, 0, 512, 256) == "SAGE_E_STRIDE"
    assert call(A + 8, 0, 512, 128) == "SAGE_E_ALIGN"
    assert call(A, 0, 512, 128, SageBufs(A, 0, A, A, A, A, A)) == "SAGE_E_NULL"


def test_segmented_refusals_happen_before_launch(sage):
    from quantized_exact_order_amd._lib import lib, SageBufs, STATUS_NAMES
    A = 0x100000
    shape = sage.Shape(1, 100, 4, 2, 128, 96)                   # 2 key tiles
    bufs = SageBufs(A, A, A, A, A, A, A)
    n = ctypes.c_size_t()
    ws = lambda nseg, s=shape: STATUS_NAMES[lib.sage_attn_segmented_workspace(
        ctypes.byref(s.c()), nseg, ctypes.byref(n))]
    assert ws(0) == "SAGE_E_SHAPE" and ws(3) == "SAGE_E_SHAPE"
    assert ws(2) == "SAGE_OK"
    r256 = lambda x: x + (-x % 256)
    assert n.value == r256(1 * 4 * 2 * 100 * 128 * 4) + r256(1 * 4 * 2 * 100 * 2 * 4)   # RO, then (m, d)
    assert ws(1, sage.Shape(1, 100, 4, 3, 128, 96)) == "SAGE_E_GQA"
    call = lambda nseg, wsp=A, wsb=1 << 30, o=A: STATUS_NAMES[lib.sage_attn_fwd_segmented(
        ctypes.byref(shape.c()), ctypes.byref(bufs), nseg, o, 0, 512, 128, wsp, wsb, None)]
    assert call(2, o=None) == "SAGE_E_NULL"
    assert call(0) == "SAGE_E_SHAPE" and call(3) == "SAGE_E_SHAPE"
    assert call(2, wsb=16) == "SAGE_E_WORKSPACE"
    assert call(2, wsp=None) == "SAGE_E_WORKSPACE"
    assert call(2, wsp=A + 8) == "SAGE_E_ALIGN"
    # the grid limit counts the segments: ceil(N/128) * Hq * 256 = 131071 * 64 * 256 work-items
    # per segment, so 2 segments (4,294,934,528) fit under 2^32 - 1 and 3 do not
    big = sage.Shape(1, 128 * 131071, 64, 1, 128, 96)
    assert ws(2, big) == "SAGE_OK" and ws(3, big) == "SAGE_E_SHAPE"


def test_largest_grid_is_accepted(sage):
    # 2^32 - 1 work-items per dispatch is the limit; the quantization grid of
    # (85 + 170) * 65535 work-groups of 256 threads (4,278,190,080) is just under it
    z = sage.buffer_sizes(sage.Shape(1, 64 * 170, 65535, 65535, 128, 96))
    assert z.n_k_tiles == 170


def test_decode_cache_refusals_happen_before_launch(sage):
    from quantized_exact_order_amd._lib import lib, SageKvCache, SageView, STATUS_NAMES
    A = 0x100000
    name = lambda st: STATUS_NAMES[st]
    cache = lambda **kw: SageKvCache(**{**dict(k8=A, k_scale=A, v=A, B=1, Hkv=2, D=256, capacity=64), **kw})
    kv = SageView(A, 0, 2 * 256, 256, 1)
    append = lambda c, t0, n, k=kv: name(lib.sage_kv_append(ctypes.byref(c), ctypes.byref(k), ctypes.byref(kv),
                                                            t0, n, None))
    assert append(cache(k8=0), 0, 1) == "SAGE_E_NULL"
    assert append(cache(D=128), 0, 1) == "SAGE_E_UNSUPPORTED"
    assert append(cache(), 60, 5) == "SAGE_E_SHAPE"            # past the capacity
    assert append(cache(), -1, 1) == "SAGE_E_SHAPE"
    assert append(cache(), 0, 0) == "SAGE_E_SHAPE"
    assert append(cache(v=A + 4), 0, 1) == "SAGE_E_ALIGN"
    assert append(cache(capacity=60), 0, 1) == "SAGE_E_SHAPE"   # capacity not a multiple of 8
    # 2^20 blocks x 64 heads: 2^24 work-groups of 256 threads, one past the dispatch limit
    assert append(cache(Hkv=64, capacity=1 << 23), 0, 1 << 23) == "SAGE_E_SHAPE"
    assert append(cache(), 0, 1, SageView(A, 0, 512, 256, 2)) == "SAGE_E_STRIDE"
    # a cache holds BF16 V or INT8 V (v8 with its scales), never both or neither
    assert append(cache(v=0), 0, 1) == "SAGE_E_NULL"
    assert append(cache(v8=A), 0, 1) == "SAGE_E_NULL"
    assert append(cache(v8=A, v_scale=A), 0, 1) == "SAGE_E_NULL"
    assert append(cache(v=0, v8=A), 0, 1) == "SAGE_E_NULL"
    assert append(cache(v=0, v8=A + 4, v_scale=A), 0, 1) == "SAGE_E_ALIGN"
    assert append(cache(v=0, v8=A, v_scale=A + 4), 0, 1) == "SAGE_E_ALIGN"
    n = ctypes.c_size_t()
    assert name(lib.sage_decode_workspace(ctypes.byref(cache(v=0, v8=A, v_scale=A)), 8, 64, ctypes.byref(n))) \
        == "SAGE_OK"
    assert name(lib.sage_decode_workspace(ctypes.byref(cache(v8=A, v_scale=A)), 8, 64, ctypes.byref(n))) \
        == "SAGE_E_NULL"
    assert name(lib.sage_decode_workspace(ctypes.byref(cache()), 8, 64, ctypes.byref(n))) == "SAGE_OK"
    assert n.value == 1 * 8 * 1 * 260 * 4 + (-(1 * 8 * 260 * 4) % 256)     # one chunk of partials
    assert name(lib.sage_decode_workspace(ctypes.byref(cache()), 8, 65, ctypes.byref(n))) == "SAGE_E_SHAPE"
    q = SageView(A, 0, 8 * 256, 256, 1)
    attn = lambda c, Hq, T, ws=A, wsb=1 << 30, o=A: name(lib.sage_decode_attn(
        ctypes.byref(c), Hq, ctypes.byref(q), T, o, ws, wsb, None))
    assert attn(cache(), 8, 64, o=None) == "SAGE_E_NULL"
    assert attn(cache(), 7, 64) == "SAGE_E_GQA"
    assert attn(cache(), 34, 64) == "SAGE_E_UNSUPPORTED"      # 17 query heads per KV head
    assert attn(cache(), 8, 0) == "SAGE_E_SHAPE"
    assert attn(cache(), 8, 65) == "SAGE_E_SHAPE"
    assert attn(cache(), 8, 64, wsb=16) == "SAGE_E_WORKSPACE"
    assert attn(cache(), 8, 64, ws=0) == "SAGE_E_WORKSPACE"
    assert attn(cache(), 8, 64, o=A + 8) == "SAGE_E_ALIGN"


def test_primitive_hook_refusals_happen_before_launch(sage):
    from quantized_exact_order_amd._lib import lib, STATUS_NAMES
    A = 0x100000
    prim = lambda kind, first, count, out=A: STATUS_NAMES[lib.sage_selftest_primitive(kind, first, count, out, None)]
    assert prim(0, 0, 16, out=None) == "SAGE_E_NULL"
    assert prim(0, 0, 16, out=A + 4) == "SAGE_E_ALIGN"
    assert prim(-1, 0, 16) == "SAGE_E_UNSUPPORTED"
    assert prim(16, 0, 16) == "SAGE_E_UNSUPPORTED"
    assert prim(10, 0, 96) == "SAGE_E_SHAPE"                        # lane exchanges take whole waves
    assert prim(0, 0, 0) == "SAGE_E_SHAPE"
    assert prim(0, 0, (1 << 26) + 1) == "SAGE_E_SHAPE"             # more than one chunk
    assert prim(0, 0xFFFFFFF0, 17) == "SAGE_E_SHAPE"                # runs past pattern 2^32 - 1


def test_prepared_output_alignment_is_checked_before_launch(sage):
    from quantized_exact_order_amd._lib import lib, SageBufs, SageShape, SageView, STATUS_NAMES
    A = 0x100000
    shape = SageShape(1, 64, 2, 2, 128, 96, 0, 1e-5)
    view = SageView(A, 0, 2 * 128, 128, 1)
    bufs = SageBufs(A, A, A, A, A, A, A, A + 2, None)             # q_prep misaligned
    st = lib.sage_quant_qk(ctypes.byref(shape), ctypes.byref(view), ctypes.byref(view), ctypes.byref(view),
                           None, None, A, A, ctypes.byref(bufs), A, 1 << 30, None)
    assert STATUS_NAMES[st] == "SAGE_E_ALIGN"
