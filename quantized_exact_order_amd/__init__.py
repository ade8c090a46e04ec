"""MI355X (gfx950) quantized attention forward: Python binding of libsage_amd.

Thin marshalling layer over the C ABI of include/sage.h.  torch is used for
device memory and streams only; every step of the path (RMSNorm, RoPE, K mean,
quantization, attention) runs in the library's HIP kernels.

    shape = Shape(B, N, Hq, Hkv, D, rope_dim, hadamard, eps)
    bufs  = Buffers.allocate(shape, device)
    prep(shape, bufs, q, k, v, w_q, w_k, cos, sin)       # pass 1
    quant_qk(shape, bufs, q, k, v, w_q, w_k, cos, sin)   # pass 2
    o = attn_fwd(shape, bufs)                            # BF16 [B, N, Hq, D]

Decode-time INT8 K cache (per-head Hadamard rotation, one scale per token):

    cache = KvCache.allocate(B, Hkv, capacity, device)   # D = 256
    kv_append(cache, k, v, t0)                           # k, v BF16 [B, n, Hkv, D]
    o = decode_attn(cache, q, T)                         # q BF16 [B, Hq, D] -> [B, Hq, D]
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from ._lib import (EXPORTS, LIB_PATH, SageBufs, SageError, SageKvCache, SageShape, SageSizes,
                   SageView, check, lib)

__all__ = ["Shape", "Buffers", "buffer_sizes", "prep", "quant_qk", "attn_fwd", "forward",
           "attn_segmented_workspace", "attn_fwd_segmented", "attn_fwd_stamped", "wall_clock_hz",
           "v8_logical", "v8_slot_keys", "KvCache",
           "kv_append", "decode_workspace", "decode_attn", "decode_attn_noalloc", "decode_noalloc_max_bytes",
           "selftest_primitive", "SageError", "LIB_PATH",
           "EXPORTS"]


@dataclass(frozen=True)
class Shape:
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    rope_dim: int
    hadamard: bool = False
    eps: float = 1e-5

    def c(self) -> SageShape:
        return SageShape(self.B, self.N, self.Hq, self.Hkv, self.D, self.rope_dim,
                         int(self.hadamard), self.eps)


def buffer_sizes(shape: Shape) -> SageSizes:
    out = SageSizes()
    check(lib.sage_buffer_sizes(ctypes.byref(shape.c()), ctypes.byref(out)), "sage_buffer_sizes")
    return out


@dataclass
class Buffers:
    """Device tensors behind sage_bufs plus the pass-1 workspace."""
    q8: torch.Tensor         # int8  [B, Hq, q_rows, D]
    q_scale: torch.Tensor    # f32   [B, Hq, n_q_groups]
    k8: torch.Tensor         # int8  [B, Hkv, k_rows, D]
    k_scale: torch.Tensor    # f32   [B, Hkv, n_k_tiles]
    k_mean: torch.Tensor     # f32   [B, Hkv, D]
    v8: torch.Tensor         # uint8 [B, Hkv, n_k_tiles, D, 64] (E4M3, keys in slot order)
    v_scale: torch.Tensor    # f32   [B, Hkv, D]
    workspace: torch.Tensor  # uint8 [sizes.workspace]
    q_prep: Optional[torch.Tensor] = None   # bf16 [B, Hq, N, D] prepared Q (optional)
    k_prep: Optional[torch.Tensor] = None   # bf16 [B, Hkv, N, D] prepared K (optional)

    @classmethod
    def allocate(cls, shape: Shape, device, prep_outputs: bool = False) -> "Buffers":
        """Buffers for shape; prep_outputs also allocates q_prep / k_prep, the
        BF16 Q and K after RMSNorm and RoPE that sage_quant_qk then writes."""
        z = buffer_sizes(shape)
        B, N, Hq, Hkv, D = shape.B, shape.N, shape.Hq, shape.Hkv, shape.D
        e = lambda *s, dt: torch.empty(s, dtype=dt, device=device)
        return cls(e(B, Hq, z.q_rows, D, dt=torch.int8), e(B, Hq, z.n_q_groups, dt=torch.float32),
                   e(B, Hkv, z.k_rows, D, dt=torch.int8), e(B, Hkv, z.n_k_tiles, dt=torch.float32),
                   e(B, Hkv, D, dt=torch.float32),
                   e(B, Hkv, z.n_k_tiles, D, 64, dt=torch.uint8), e(B, Hkv, D, dt=torch.float32),
                   e(max(int(z.workspace), 1), dt=torch.uint8),
                   e(B, Hq, N, D, dt=torch.bfloat16) if prep_outputs else None,
                   e(B, Hkv, N, D, dt=torch.bfloat16) if prep_outputs else None)

    def c(self) -> SageBufs:
        ptr = lambda t: None if t is None else t.data_ptr()
        return SageBufs(self.q8.data_ptr(), self.q_scale.data_ptr(), self.k8.data_ptr(),
                        self.k_scale.data_ptr(), self.k_mean.data_ptr(), self.v8.data_ptr(),
                        self.v_scale.data_ptr(), ptr(self.q_prep), ptr(self.k_prep))

    def check(self, shape: Shape) -> None:
        """Raise unless these buffers have the sizes sage_buffer_sizes gives for shape."""
        z = buffer_sizes(shape)
        B, Hq, Hkv, D = shape.B, shape.Hq, shape.Hkv, shape.D
        i8, f32, u8 = torch.int8, torch.float32, torch.uint8
        want = {"q8": ((B, Hq, z.q_rows, D), i8), "q_scale": ((B, Hq, z.n_q_groups), f32),
                "k8": ((B, Hkv, z.k_rows, D), i8), "k_scale": ((B, Hkv, z.n_k_tiles), f32),
                "k_mean": ((B, Hkv, D), f32), "v8": ((B, Hkv, z.n_k_tiles, D, 64), u8),
                "v_scale": ((B, Hkv, D), f32)}
        for name, (shp, dt) in want.items():
            t = getattr(self, name)
            if tuple(t.shape) != shp or t.dtype != dt or not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError(f"buffer {name} must be a contiguous {dt} GPU tensor of shape {shp}")
        _workspace(self.workspace, z.workspace)
        for name, h in (("q_prep", Hq), ("k_prep", Hkv)):
            t = getattr(self, name)
            if t is not None and (tuple(t.shape) != (B, h, shape.N, D) or t.dtype != torch.bfloat16
                                  or not t.is_contiguous() or t.device.type != "cuda"):
                raise ValueError(f"{name} must be a contiguous BF16 GPU tensor of shape {(B, h, shape.N, D)}")


def _view(t: torch.Tensor, name: str) -> SageView:
    if t.dtype != torch.bfloat16 or t.dim() != 4 or t.device.type != "cuda":
        raise ValueError(f"{name} must be a BF16 [B, N, H, D] tensor on the GPU")
    sb, sn, sh, sd = t.stride()
    return SageView(t.data_ptr(), sb, sn, sh, sd)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _workspace(t: torch.Tensor, need: int) -> None:
    """A caller's workspace: contiguous GPU bytes, at least `need` of them (the
    C ABI checks the count it is told, not where the memory is)."""
    if t.device.type != "cuda" or not t.is_contiguous() or t.numel() * t.element_size() < need:
        raise ValueError(f"workspace must be a contiguous GPU tensor of at least {need} bytes")


def _aux(t: Optional[torch.Tensor], name: str, numel: int) -> Optional[int]:
    """Pointer of an optional BF16 side input (RMSNorm weight, RoPE table),
    checked here: the C ABI cannot tell a host pointer or a short buffer."""
    if t is None:
        return None
    if t.dtype != torch.bfloat16 or t.device.type != "cuda" or not t.is_contiguous() or t.numel() != numel:
        raise ValueError(f"{name} must be a contiguous BF16 GPU tensor of {numel} elements")
    return t.data_ptr()


def _pass(fn, where, shape, bufs, q, k, v, w_q, w_k, cos, sin, stream):
    qv, kv, vv = _view(q, "q"), _view(k, "k"), _view(v, "v")
    B, N, Hq, Hkv, D = shape.B, shape.N, shape.Hq, shape.Hkv, shape.D
    for t, name, h in ((q, "q", Hq), (k, "k", Hkv), (v, "v", Hkv)):
        if tuple(t.shape) != (B, N, h, D):
            raise ValueError(f"{name} must have shape {(B, N, h, D)}, got {tuple(t.shape)}")
    bufs.check(shape)
    half = shape.rope_dim // 2
    w_q, w_k = _aux(w_q, "w_q", D), _aux(w_k, "w_k", D)
    cos, sin = _aux(cos, "cos", N * half), _aux(sin, "sin", N * half)
    check(fn(ctypes.byref(shape.c()), ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv),
             w_q, w_k, cos, sin, ctypes.byref(bufs.c()),
             bufs.workspace.data_ptr(), bufs.workspace.numel() * bufs.workspace.element_size(),
             _stream(stream)), where)


def prep(shape: Shape, bufs: Buffers, q, k, v, w_q=None, w_k=None, cos=None, sin=None, stream=None):
    """Pass 1: k_mean, v_scale and the workspace partials (sage_prep)."""
    _pass(lib.sage_prep, "sage_prep", shape, bufs, q, k, v, w_q, w_k, cos, sin, stream)


def quant_qk(shape: Shape, bufs: Buffers, q, k, v, w_q=None, w_k=None, cos=None, sin=None,
             stream=None):
    """Pass 2: q8, q_scale, k8, k_scale, v8 (sage_quant_qk)."""
    _pass(lib.sage_quant_qk, "sage_quant_qk", shape, bufs, q, k, v, w_q, w_k, cos, sin, stream)


def attn_fwd(shape: Shape, bufs: Buffers, o: Optional[torch.Tensor] = None, stream=None):
    """Fused attention (sage_attn_fwd); returns BF16 [B, N, Hq, D]."""
    bufs.check(shape)
    if o is None:
        o = torch.empty((shape.B, shape.N, shape.Hq, shape.D), dtype=torch.bfloat16,
                        device=bufs.q8.device)
    if (o.dtype != torch.bfloat16 or o.dim() != 4 or o.shape[0] != shape.B or o.shape[1] < shape.N
            or o.shape[2] != shape.Hq or o.shape[3] != shape.D or o.device.type != "cuda"):
        raise ValueError("o must be a BF16 [B, >=N, Hq, D] tensor on the GPU")
    sb, sn, sh, sd = o.stride()
    if sd != 1:
        raise ValueError("o must have unit stride in d")
    check(lib.sage_attn_fwd(ctypes.byref(shape.c()), ctypes.byref(bufs.c()), o.data_ptr(),
                            sb, sn, sh, _stream(stream)), "sage_attn_fwd")
    return o


def attn_fwd_stamped(shape: Shape, bufs: Buffers, o: torch.Tensor, stream=None):
    """sage_attn_fwd_stamped: the attention launch of attn_fwd, writing o, plus
    per-work-group clock stamps.  Returns a uint64 tensor [work-groups, 4]:
    shader clock and constant-rate counter at the start and at the end of the
    work-group's first wave."""
    bufs.check(shape)
    n = ctypes.c_size_t()
    check(lib.sage_attn_stamp_bytes(ctypes.byref(shape.c()), ctypes.byref(n)), "sage_attn_stamp_bytes")
    stamps = torch.zeros(n.value // 8, dtype=torch.int64, device=o.device)
    sb, sn, sh, _ = o.stride()
    check(lib.sage_attn_fwd_stamped(ctypes.byref(shape.c()), ctypes.byref(bufs.c()), o.data_ptr(), sb, sn, sh,
                                    stamps.data_ptr(), n.value, _stream(stream)), "sage_attn_fwd_stamped")
    return stamps.view(-1, 4)


def wall_clock_hz() -> float:
    """Rate of the constant-rate counter of the current device (Hz)."""
    khz = ctypes.c_int32()
    check(lib.sage_wall_clock_khz(ctypes.byref(khz)), "sage_wall_clock_khz")
    return khz.value * 1e3


def attn_segmented_workspace(shape: Shape, nseg: int) -> int:
    n = ctypes.c_size_t()
    check(lib.sage_attn_segmented_workspace(ctypes.byref(shape.c()), nseg, ctypes.byref(n)),
          "sage_attn_segmented_workspace")
    return n.value


def attn_fwd_segmented(shape: Shape, bufs: Buffers, nseg: int, o: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """Segmented (split-KV) attention, an opt-in mode that is not the exact
    order of attn_fwd (sage_attn_fwd_segmented); returns BF16 [B, N, Hq, D]."""
    bufs.check(shape)
    if o is None:
        o = torch.empty((shape.B, shape.N, shape.Hq, shape.D), dtype=torch.bfloat16,
                        device=bufs.q8.device)
    if (o.dtype != torch.bfloat16 or o.dim() != 4 or o.shape[0] != shape.B or o.shape[1] < shape.N
            or o.shape[2] != shape.Hq or o.shape[3] != shape.D or o.device.type != "cuda"):
        raise ValueError("o must be a BF16 [B, >=N, Hq, D] tensor on the GPU")
    sb, sn, sh, sd = o.stride()
    if sd != 1:
        raise ValueError("o must have unit stride in d")
    need = attn_segmented_workspace(shape, nseg)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=o.device)
    _workspace(workspace, need)
    check(lib.sage_attn_fwd_segmented(ctypes.byref(shape.c()), ctypes.byref(bufs.c()), nseg, o.data_ptr(),
                                      sb, sn, sh, workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(), _stream(stream)),
          "sage_attn_fwd_segmented")
    return o


def forward(q, k, v, w_q=None, w_k=None, cos=None, sin=None, rope_dim: int = 0,
            hadamard: bool = False, eps: float = 1e-5, stream=None):
    """All three passes; returns (o, shape, bufs)."""
    B, N, Hq, D = q.shape
    shape = Shape(B, N, Hq, k.shape[2], D, rope_dim, hadamard, eps)
    bufs = Buffers.allocate(shape, q.device)
    prep(shape, bufs, q, k, v, w_q, w_k, cos, sin, stream)
    quant_qk(shape, bufs, q, k, v, w_q, w_k, cos, sin, stream)
    return attn_fwd(shape, bufs, stream=stream), shape, bufs


_PRIMITIVE_DTYPES = {0: torch.int16, 1: torch.int8, 2: torch.uint8, 9: torch.uint8}


def selftest_primitive(kind: int, first: int, count: int, out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Test hook (sage_selftest_primitive): device number-format primitive
    `kind` (0 BF16 bits as int16, 1 INT8, 2 and 9 E4M3 bytes, 3..8 FP32 results,
    10..15 the lane exchange at xor distance 2^(kind-10), FP32 bits moved) of
    the FP32 values with bit patterns first .. first + count - 1."""
    dt = _PRIMITIVE_DTYPES.get(kind, torch.float32)
    if out is None:
        out = torch.empty(count, dtype=dt, device="cuda")
    if out.dtype != dt or out.numel() < count or out.device.type != "cuda" or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {dt} GPU tensor of at least {count} elements")
    check(lib.sage_selftest_primitive(kind, first, count, out.data_ptr(), _stream(stream)),
          "sage_selftest_primitive")
    return out


def v8_slot_keys() -> list:
    """Key (0..63) stored at each slot of a v8 tile row."""
    return [lib.sage_v8_key_of_slot(s) for s in range(64)]


def v8_logical(shape: Shape, bufs: Buffers) -> torch.Tensor:
    """v8 rearranged to logical [B, Hkv, N, D] key order (for inspection)."""
    B, Hkv, nk, D, _ = bufs.v8.shape
    keys = torch.tensor(v8_slot_keys(), device=bufs.v8.device)
    inv = torch.empty_like(keys)
    inv[keys] = torch.arange(64, device=keys.device)
    t = bufs.v8.index_select(4, inv)                      # [B,Hkv,nk,D,64] in key order
    return t.permute(0, 1, 2, 4, 3).reshape(B, Hkv, nk * 64, D)[:, :, :shape.N]


# ----------------------------------------------------------------------------
# Decode-time INT8 K cache
# ----------------------------------------------------------------------------

@dataclass
class KvCache:
    """Device tensors behind sage_kv_cache (D = 256): V either BF16 (v) or
    rotated INT8 with one FP32 scale per (head, token) (v8, v_scale)."""
    k8: torch.Tensor                            # int8  [B, Hkv, capacity, D], rotated K rows
    k_scale: torch.Tensor                       # f32   [B, Hkv, capacity]
    v: Optional[torch.Tensor]                   # bf16  [B, Hkv, capacity / 8, D, 8], 8-token blocks per channel
    v8: Optional[torch.Tensor] = None           # int8  [B, Hkv, capacity / 8, D, 8], rotated V rows
    v_scale: Optional[torch.Tensor] = None      # f32   [B, Hkv, capacity]

    @classmethod
    def allocate(cls, B: int, Hkv: int, capacity: int, device, D: int = 256, int8_v: bool = False) -> "KvCache":
        """Zeroed cache; capacity must be a multiple of 8."""
        if capacity % 8:
            raise ValueError("capacity must be a multiple of 8")
        k8 = torch.zeros((B, Hkv, capacity, D), dtype=torch.int8, device=device)
        ks = torch.zeros((B, Hkv, capacity), dtype=torch.float32, device=device)
        if int8_v:
            return cls(k8, ks, None, torch.zeros((B, Hkv, capacity // 8, D, 8), dtype=torch.int8, device=device),
                       torch.zeros((B, Hkv, capacity), dtype=torch.float32, device=device))
        return cls(k8, ks, torch.zeros((B, Hkv, capacity // 8, D, 8), dtype=torch.bfloat16, device=device))

    def v_rows(self) -> torch.Tensor:
        """The cached V (BF16, or INT8 codes of the rotated rows) as
        [B, Hkv, capacity, D] (a copy)."""
        blocks = self.v if self.v is not None else self.v8
        B, Hkv, nb, D, _ = blocks.shape
        return blocks.permute(0, 1, 2, 4, 3).reshape(B, Hkv, nb * 8, D)

    def c(self) -> SageKvCache:
        """The C view of the cache, after checking that its tensors agree:
        the C ABI takes their pointers and sizes on trust."""
        if self.k8.dim() != 4:
            raise ValueError("k8 must be an int8 [B, Hkv, capacity, D] tensor")
        B, Hkv, cap, D = self.k8.shape
        if (self.v is None) == (self.v8 is None) or (self.v8 is None) != (self.v_scale is None):
            raise ValueError("a cache holds either v (BF16) or v8 with v_scale (INT8 V)")
        want = [(self.k8, (B, Hkv, cap, D), torch.int8), (self.k_scale, (B, Hkv, cap), torch.float32)]
        if self.v is not None:
            want.append((self.v, (B, Hkv, cap // 8, D, 8), torch.bfloat16))
        else:
            want += [(self.v8, (B, Hkv, cap // 8, D, 8), torch.int8), (self.v_scale, (B, Hkv, cap), torch.float32)]
        for t, shp, dt in want:
            if tuple(t.shape) != shp or t.dtype != dt or not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError(f"cache tensors must be contiguous GPU tensors: k8 int8 [B, Hkv, capacity, D], "
                                 f"k_scale float32 [B, Hkv, capacity], v bfloat16 [B, Hkv, capacity/8, D, 8] "
                                 f"or v8 int8 of that shape with v_scale float32 [B, Hkv, capacity]")
        ptr = lambda t: t.data_ptr() if t is not None else None
        return SageKvCache(self.k8.data_ptr(), self.k_scale.data_ptr(), ptr(self.v), B, Hkv, D, cap,
                           ptr(self.v8), ptr(self.v_scale))


def kv_append(cache: KvCache, k, v, t0: int, stream=None) -> None:
    """Rotate, quantize and store K (BF16 [B, n, Hkv, D]) and copy V (or, in
    an INT8 V cache, rotate and quantize it like K) at positions [t0, t0 + n)
    (sage_kv_append)."""
    kv, vv = _view(k, "k"), _view(v, "v")
    B, Hkv, D = cache.k8.shape[0], cache.k8.shape[1], cache.k8.shape[3]
    if k.shape[0] != B or k.shape[2] != Hkv or k.shape[3] != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k and v must both have shape [{B}, n, {Hkv}, {D}]")
    check(lib.sage_kv_append(ctypes.byref(cache.c()), ctypes.byref(kv), ctypes.byref(vv), t0,
                             k.shape[1], _stream(stream)), "sage_kv_append")


def decode_workspace(cache: KvCache, Hq: int, T: int) -> int:
    n = ctypes.c_size_t()
    check(lib.sage_decode_workspace(ctypes.byref(cache.c()), Hq, T, ctypes.byref(n)), "sage_decode_workspace")
    return n.value


def decode_attn(cache: KvCache, q, T: int, o: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Single-query attention of q (BF16 [B, Hq, D]) over cache positions
    [0, T) (sage_decode_attn); returns BF16 [B, Hq, D]."""
    B, Hq, D = q.shape
    if B != cache.k8.shape[0] or D != cache.k8.shape[3]:
        raise ValueError(f"q must have shape [{cache.k8.shape[0]}, Hq, {cache.k8.shape[3]}]")
    if o is None:
        o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    if (o.dtype != torch.bfloat16 or tuple(o.shape) != (B, Hq, D) or not o.is_contiguous()
            or o.device.type != "cuda"):
        raise ValueError("o must be a contiguous BF16 [B, Hq, D] GPU tensor")
    cc = cache.c()
    n = ctypes.c_size_t()
    check(lib.sage_decode_workspace(ctypes.byref(cc), Hq, T, ctypes.byref(n)), "sage_decode_workspace")
    need = n.value
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _workspace(workspace, need)
    qv = _view(q.unsqueeze(1), "q")
    check(lib.sage_decode_attn(ctypes.byref(cc), Hq, ctypes.byref(qv), T, o.data_ptr(),
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               _stream(stream)), "sage_decode_attn")
    return o


def decode_attn_noalloc(cache: KvCache, q, T: int, o: torch.Tensor, stream=None) -> torch.Tensor:
    """sage_decode_attn_noalloc: decode_attn with the chunk partials in the
    library's fixed per-GPU array; the caller passes the output, nothing is
    allocated.  Calls that overlap on one GPU race on that array."""
    B, Hq, D = q.shape
    if B != cache.k8.shape[0] or D != cache.k8.shape[3]:
        raise ValueError(f"q must have shape [{cache.k8.shape[0]}, Hq, {cache.k8.shape[3]}]")
    if (o.dtype != torch.bfloat16 or tuple(o.shape) != (B, Hq, D) or not o.is_contiguous()
            or o.device.type != "cuda"):
        raise ValueError("o must be a contiguous BF16 [B, Hq, D] GPU tensor")
    qv = _view(q.unsqueeze(1), "q")
    check(lib.sage_decode_attn_noalloc(ctypes.byref(cache.c()), Hq, ctypes.byref(qv), T, o.data_ptr(),
                                       _stream(stream)), "sage_decode_attn_noalloc")
    return o


def decode_noalloc_max_bytes() -> int:
    """Size of the fixed per-GPU array of decode_attn_noalloc."""
    return int(lib.sage_decode_noalloc_max_bytes())
