"""ctypes mirror of include/sage.h and loader of the in-tree libsage_amd.so.

Argument marshalling only: every step of the path runs in the HIP kernels of
the library.  If the library has not been built this module raises at import
time -- there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsage_amd.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python quantized_exact_order_amd/build.py` "
        "(hipcc, gfx950). There is no fallback implementation.")

_lib = ctypes.CDLL(LIB_PATH)

i32, i64, f32, sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

SAGE_OK = 0
STATUS_NAMES = {0: "SAGE_OK", 1: "SAGE_E_NULL", 2: "SAGE_E_SHAPE", 3: "SAGE_E_STRIDE",
                4: "SAGE_E_ALIGN", 5: "SAGE_E_ROPE", 6: "SAGE_E_GQA", 7: "SAGE_E_WORKSPACE",
                8: "SAGE_E_UNSUPPORTED", 9: "SAGE_E_HIP"}


class SageShape(ctypes.Structure):
    _fields_ = [("B", i32), ("N", i32), ("Hq", i32), ("Hkv", i32), ("D", i32),
                ("rope_dim", i32), ("hadamard", i32), ("eps", f32)]


class SageView(ctypes.Structure):
    _fields_ = [("ptr", vp), ("sb", i64), ("sn", i64), ("sh", i64), ("sd", i64)]


class SageBufs(ctypes.Structure):
    _fields_ = [("q8", vp), ("q_scale", vp), ("k8", vp), ("k_scale", vp), ("k_mean", vp),
                ("v8", vp), ("v_scale", vp), ("q_prep", vp), ("k_prep", vp)]


class SageSizes(ctypes.Structure):
    _fields_ = [("q8", sz), ("q_scale", sz), ("k8", sz), ("k_scale", sz), ("k_mean", sz),
                ("v8", sz), ("v_scale", sz), ("workspace", sz),
                ("q_rows", i64), ("n_q_groups", i64), ("k_rows", i64), ("n_k_tiles", i64)]


class SageKvCache(ctypes.Structure):
    _fields_ = [("k8", vp), ("k_scale", vp), ("v", vp), ("B", i32), ("Hkv", i32), ("D", i32),
                ("capacity", i32), ("v8", vp), ("v_scale", vp)]


P = ctypes.POINTER
_lib.sage_buffer_sizes.argtypes = [P(SageShape), P(SageSizes)]
_lib.sage_buffer_sizes.restype = i32
for _name in ("sage_prep", "sage_quant_qk"):
    fn = getattr(_lib, _name)
    fn.argtypes = [P(SageShape), P(SageView), P(SageView), P(SageView), vp, vp, vp, vp,
                   P(SageBufs), vp, sz, vp]
    fn.restype = i32
_lib.sage_attn_fwd.argtypes = [P(SageShape), P(SageBufs), vp, i64, i64, i64, vp]
_lib.sage_attn_fwd.restype = i32
_lib.sage_attn_segmented_workspace.argtypes = [P(SageShape), i32, P(sz)]
_lib.sage_attn_segmented_workspace.restype = i32
_lib.sage_attn_fwd_segmented.argtypes = [P(SageShape), P(SageBufs), i32, vp, i64, i64, i64, vp, sz, vp]
_lib.sage_attn_fwd_segmented.restype = i32
_lib.sage_attn_stamp_bytes.argtypes = [P(SageShape), P(sz)]
_lib.sage_attn_stamp_bytes.restype = i32
_lib.sage_attn_fwd_stamped.argtypes = [P(SageShape), P(SageBufs), vp, i64, i64, i64, vp, sz, vp]
_lib.sage_attn_fwd_stamped.restype = i32
_lib.sage_wall_clock_khz.argtypes = [P(i32)]
_lib.sage_wall_clock_khz.restype = i32
_lib.sage_kv_append.argtypes = [P(SageKvCache), P(SageView), P(SageView), i32, i32, vp]
_lib.sage_kv_append.restype = i32
_lib.sage_decode_workspace.argtypes = [P(SageKvCache), i32, i32, P(sz)]
_lib.sage_decode_workspace.restype = i32
_lib.sage_decode_attn.argtypes = [P(SageKvCache), i32, P(SageView), i32, vp, vp, sz, vp]
_lib.sage_decode_attn.restype = i32
_lib.sage_decode_attn_noalloc.argtypes = [P(SageKvCache), i32, P(SageView), i32, vp, vp]
_lib.sage_decode_attn_noalloc.restype = i32
_lib.sage_decode_noalloc_max_bytes.argtypes = []
_lib.sage_decode_noalloc_max_bytes.restype = sz
_lib.sage_selftest_primitive.argtypes = [i32, ctypes.c_uint32, ctypes.c_uint32, vp, vp]
_lib.sage_selftest_primitive.restype = i32
_lib.sage_v8_key_of_slot.argtypes = [i32]
_lib.sage_v8_key_of_slot.restype = i32
_lib.sage_status_str.argtypes = [i32]
_lib.sage_status_str.restype = ctypes.c_char_p
_lib.sage_version.restype = i32

EXPORTS = ("sage_buffer_sizes", "sage_prep", "sage_quant_qk", "sage_attn_fwd",
           "sage_attn_segmented_workspace", "sage_attn_fwd_segmented",
           "sage_attn_stamp_bytes", "sage_attn_fwd_stamped", "sage_wall_clock_khz",
           "sage_kv_append", "sage_decode_workspace", "sage_decode_attn",
           "sage_decode_attn_noalloc", "sage_decode_noalloc_max_bytes",
           "sage_selftest_primitive", "sage_v8_key_of_slot", "sage_status_str", "sage_version")


class SageError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{where}: {_lib.sage_status_str(status).decode()}")


def check(status: int, where: str) -> None:
    if status != SAGE_OK:
        raise SageError(status, where)


lib = _lib
