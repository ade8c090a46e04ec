"""CPU oracle of the quantized attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import this package.  The product path
(``quantized_exact_order_amd``) never imports it and shares no code with it.

The arithmetic lives in ``sage_oracle.c`` (plain C, built with gcc
``-O2 -fopenmp -ffp-contract=off``); this module only marshals numpy/torch
arrays into it and adds the FP64 unquantized reference attention used by the
accuracy gate.  Every function cites the page passage it follows in the C
source; see the header of ``sage_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sage_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "libsage_oracle.so")
_lib = None

# gcc flags of the oracle library: strict IEEE binary32, no contraction.
GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Werror",
             "-Wall", "-Wextra", "-Wno-unused-parameter", "-fPIC", "-shared"]

# Mutation testing of the pins: when set, this names an already compiled
# variant of sage_oracle.c that is loaded instead of the in-tree build.
_OVERRIDE = os.environ.get("SAGE_ORACLE_LIB_OVERRIDE")


def compile_source(src: str, out: str, werror: bool = True) -> None:
    """gcc ``src`` into the shared library ``out`` with the oracle's flags.
    werror=False keeps warnings as warnings: the mutation check compiles
    copies with planted mistakes, which may leave a variable unused."""
    flags = [f for f in GCC_FLAGS if werror or f != "-Werror"]
    subprocess.run(["gcc", *flags, src, "-o", out, "-lm"], check=True)


def build(force: bool = False) -> str:
    """Compile the oracle shared library with gcc (no GPU toolchain involved)."""
    if _OVERRIDE:
        return _OVERRIDE
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        compile_source(_SRC, tmp)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = f32
        L.oracle_f32_to_bf16.argtypes = [f32]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_f32.restype = f32
        L.oracle_f32_to_e4m3.argtypes = [f32]
        L.oracle_f32_to_e4m3.restype = ctypes.c_uint8
        L.oracle_f32_to_i8.argtypes = [f32]
        L.oracle_f32_to_i8.restype = ctypes.c_int8
        L.oracle_exp2.argtypes = [f32]
        L.oracle_exp2.restype = f32
        L.oracle_score_scale.argtypes = [i32]
        L.oracle_score_scale.restype = f32
        L.oracle_rmsnorm_rope.argtypes = [i32, i32, i32, i32, i32, f32, P, i64, i64, i64, P, P, P, P]
        L.oracle_k_mean.argtypes = [i32, i32, i32, i32, P, P]
        L.oracle_wht.argtypes = [P, i32]
        L.oracle_quant_q.argtypes = [i32, i32, i32, i32, i32, P, P, P]
        L.oracle_quant_k.argtypes = [i32, i32, i32, i32, i32, P, P, P, P]
        L.oracle_quant_v.argtypes = [i32, i32, i32, i32, P, i64, i64, i64, P, P]
        L.oracle_attn_rows.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, i64, P, P]
        L.oracle_attn_rows_mode.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, i64, P, P, i32]
        L.oracle_attn_rows_segmented.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, i64, P, i32, P]
        L.oracle_kv_quant.argtypes = [i32, i32, i32, i32, P, i64, i64, i64, P, P]
        L.oracle_decode_attn.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P]
        L.oracle_decode_attn_v8.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_f64_to_f16.restype = f32
        L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        L.oracle_num_threads.restype = i32
        for name in ("oracle_f32_to_bf16_n", "oracle_f32_to_e4m3_n", "oracle_f32_to_i8_n",
                     "oracle_exp2_n"):
            getattr(L, name).argtypes = [P, P, i64]
        L.oracle_wht_n.argtypes = [P, i64, i32]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"] or a.size == 0
    return a.ctypes.data


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    """View a BF16 tensor (any strides) as uint16 numpy with the same strides."""
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return t.view(torch.int16).numpy().view(np.uint16)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# ----------------------------------------------------------------------------
# Number formats (bulk)
# ----------------------------------------------------------------------------

def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_bf16_n(_ptr(x), _ptr(y), x.size)
    return y


def f32_to_e4m3(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint8)
    lib().oracle_f32_to_e4m3_n(_ptr(x), _ptr(y), x.size)
    return y


def e4m3_to_f32(c: np.ndarray) -> np.ndarray:
    table = np.array([lib().oracle_e4m3_to_f32(i) for i in range(256)], np.float32)
    return table[np.asarray(c, np.uint8)]


def f32_to_i8(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.int8)
    lib().oracle_f32_to_i8_n(_ptr(x), _ptr(y), x.size)
    return y


def exp2(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.float32)
    lib().oracle_exp2_n(_ptr(x), _ptr(y), x.size)
    return y


def wht(u: np.ndarray) -> np.ndarray:
    """Normalized Walsh-Hadamard transform along the last axis (copy)."""
    u = np.array(u, dtype=np.float32, copy=True, order="C")
    D = u.shape[-1]
    lib().oracle_wht_n(_ptr(u), u.size // D, D)
    return u


def score_scale(D: int) -> float:
    return float(lib().oracle_score_scale(D))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# Pipeline steps
# ----------------------------------------------------------------------------

def rmsnorm_rope(x: torch.Tensor, w: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
                 rope_dim: int, eps: float = 1e-5) -> np.ndarray:
    """x: BF16 [B,N,H,D] (unit d stride, any other strides) -> uint16 BF16 [B,H,N,D]."""
    B, N, H, D = x.shape
    assert x.stride(3) == 1
    xb = _bf16_bits(x)
    # base pointer of the view (numpy view keeps the torch storage offset)
    base = xb.__array_interface__["data"][0]
    wb = np.ascontiguousarray(_bf16_bits(w.contiguous()))
    cb = np.ascontiguousarray(_bf16_bits(cos.contiguous()))
    sb_ = np.ascontiguousarray(_bf16_bits(sin.contiguous()))
    z = np.empty((B, H, N, D), np.uint16)
    lib().oracle_rmsnorm_rope(B, N, H, D, rope_dim, eps, base, x.stride(0), x.stride(1),
                              x.stride(2), _ptr(wb), _ptr(cb), _ptr(sb_), _ptr(z))
    return z


def k_mean(zk: np.ndarray) -> np.ndarray:
    B, H, N, D = zk.shape
    zk = np.ascontiguousarray(zk)
    mean = np.empty((B, H, D), np.float32)
    lib().oracle_k_mean(B, H, N, D, _ptr(zk), _ptr(mean))
    return mean


def quant_q(zq: np.ndarray, hadamard: bool):
    B, H, N, D = zq.shape
    zq = np.ascontiguousarray(zq)
    nq = ((N + 127) // 128) * 4
    q8 = np.zeros((B, H, N, D), np.int8)
    qs = np.empty((B, H, nq), np.float32)
    lib().oracle_quant_q(B, H, N, D, int(hadamard), _ptr(zq), _ptr(q8), _ptr(qs))
    return q8, qs


def quant_k(zk: np.ndarray, mean: np.ndarray, hadamard: bool):
    B, H, N, D = zk.shape
    zk = np.ascontiguousarray(zk)
    mean = np.ascontiguousarray(mean, np.float32)
    nk = (N + 63) // 64
    k8 = np.zeros((B, H, N, D), np.int8)
    ks = np.empty((B, H, nk), np.float32)
    lib().oracle_quant_k(B, H, N, D, int(hadamard), _ptr(zk), _ptr(mean), _ptr(k8), _ptr(ks))
    return k8, ks


def quant_v(v: torch.Tensor):
    """v: BF16 [B,N,H,D] (unit d stride) -> (v8 uint8 [B,H,N,D], v_scale [B,H,D])."""
    B, N, H, D = v.shape
    assert v.stride(3) == 1
    vb = _bf16_bits(v)
    base = vb.__array_interface__["data"][0]
    v8 = np.empty((B, H, N, D), np.uint8)
    vs = np.empty((B, H, D), np.float32)
    lib().oracle_quant_v(B, N, H, D, base, v.stride(0), v.stride(1), v.stride(2), _ptr(v8), _ptr(vs))
    return v8, vs


@dataclass
class Prepared:
    zq: np.ndarray       # uint16 BF16 [B,Hq,N,D]
    zk: np.ndarray       # uint16 BF16 [B,Hkv,N,D]
    k_mean: np.ndarray   # f32 [B,Hkv,D]
    q8: np.ndarray       # int8 [B,Hq,N,D]
    q_scale: np.ndarray  # f32 [B,Hq,ceil(N/128)*4]
    k8: np.ndarray       # int8 [B,Hkv,N,D]
    k_scale: np.ndarray  # f32 [B,Hkv,ceil(N/64)]
    v8: np.ndarray       # uint8 E4M3 [B,Hkv,N,D] logical order
    v_scale: np.ndarray  # f32 [B,Hkv,D]


def prepare(inp, rope_dim: Optional[int] = None, hadamard: Optional[bool] = None,
            eps: Optional[float] = None) -> Prepared:
    """Run the whole preparation (RMSNorm, RoPE, K mean, Q/K/V quantization)."""
    cfg = inp.cfg
    R = cfg.rope_dim if rope_dim is None else rope_dim
    had = cfg.hadamard if hadamard is None else hadamard
    e = cfg.eps if eps is None else eps
    zq = rmsnorm_rope(inp.q, inp.w_q, inp.cos, inp.sin, R, e)
    zk = rmsnorm_rope(inp.k, inp.w_k, inp.cos, inp.sin, R, e)
    mean = k_mean(zk)
    q8, qs = quant_q(zq, had)
    k8, ks = quant_k(zk, mean, had)
    v8, vs = quant_v(inp.v)
    return Prepared(zq, zk, mean, q8, qs, k8, ks, v8, vs)


def attn_rows(p: Prepared, rows: np.ndarray, pv_fp16: bool = False) -> np.ndarray:
    """Quantized attention output (uint16 BF16 [len(rows), D]) for rows (b, h, i).

    pv_fp16 selects the emulation of the page's two-level PV accumulation
    (FP16 per-tile partial) instead of the FP32 per-tile partial."""
    B, Hq, N, D = p.q8.shape
    Hkv = p.k8.shape[1]
    rows = np.ascontiguousarray(rows, np.int32).reshape(-1, 3)
    o = np.empty((rows.shape[0], D), np.uint16)
    if rows.shape[0] == 0:
        return o
    lib().oracle_attn_rows_mode(B, N, Hq, Hkv, D, _ptr(p.q8), _ptr(p.q_scale), _ptr(p.k8),
                                _ptr(p.k_scale), _ptr(p.v8), _ptr(p.v_scale), rows.shape[0],
                                _ptr(rows), _ptr(o), int(bool(pv_fp16)))
    return o


def attn_rows_segmented(p: Prepared, rows: np.ndarray, nseg: int) -> np.ndarray:
    """Output of the segmented (split-KV, non-exact) schedule with nseg
    segments of key tiles, for rows (b, h, i); uint16 BF16 [len(rows), D]."""
    B, Hq, N, D = p.q8.shape
    Hkv = p.k8.shape[1]
    nk = (N + 63) // 64
    if not 1 <= nseg <= nk:
        raise ValueError(f"nseg must be in [1, {nk}]")
    rows = np.ascontiguousarray(rows, np.int32).reshape(-1, 3)
    o = np.empty((rows.shape[0], D), np.uint16)
    if rows.shape[0] == 0:
        return o
    lib().oracle_attn_rows_segmented(B, N, Hq, Hkv, D, _ptr(p.q8), _ptr(p.q_scale), _ptr(p.k8),
                                     _ptr(p.k_scale), _ptr(p.v8), _ptr(p.v_scale), rows.shape[0],
                                     _ptr(rows), int(nseg), _ptr(o))
    return o


def attention_segmented(p: Prepared, nseg: int) -> np.ndarray:
    """attn_rows_segmented over every row, as BF16 bits [B, N, Hq, D]."""
    B, Hq, N, D = p.q8.shape
    o = attn_rows_segmented(p, all_rows(B, Hq, N), nseg)
    return o.reshape(B, Hq, N, D).transpose(0, 2, 1, 3).copy()


def f64_to_f16(x: float) -> float:
    return float(lib().oracle_f64_to_f16(float(x)))


def all_rows(B: int, H: int, N: int) -> np.ndarray:
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1).astype(np.int32)


def attention(p: Prepared, pv_fp16: bool = False) -> np.ndarray:
    """Full quantized attention output as uint16 BF16 [B,N,Hq,D]."""
    B, Hq, N, D = p.q8.shape
    o = attn_rows(p, all_rows(B, Hq, N), pv_fp16)
    return o.reshape(B, Hq, N, D).transpose(0, 2, 1, 3).copy()


# ----------------------------------------------------------------------------
# FP64 unquantized reference (accuracy gate)
# ----------------------------------------------------------------------------

def reference_attention_f64(zq: np.ndarray, zk: np.ndarray, v: torch.Tensor,
                            rows: Optional[np.ndarray] = None) -> np.ndarray:
    """softmax(zq zk^T / sqrt(D)) V in FP64 on the prepared BF16 Q/K and BF16 V.

    zq [B,Hq,N,D], zk [B,Hkv,N,D] as BF16 bits; v BF16 [B,N,Hkv,D].  No K
    smoothing: subtracting a per-(head, dim) mean from K shifts every score of
    a query row by the same amount, which softmax ignores.  Returns float64
    [B,N,Hq,D], or [len(rows), D] when rows (b, h, i) are given.
    """
    B, Hq, N, D = zq.shape
    Hkv = zk.shape[1]
    grp = Hq // Hkv
    q = bf16_to_f32(zq).astype(np.float64)
    k = bf16_to_f32(zk).astype(np.float64)
    vv = v.float().numpy().astype(np.float64).transpose(0, 2, 1, 3)  # [B,Hkv,N,D]
    scale = 1.0 / np.sqrt(D)

    def one(b, h, qi):
        s = (q[b, h, qi] @ k[b, h // grp].T) * scale
        s -= s.max(axis=-1, keepdims=True)
        e = np.exp(s)
        return (e / e.sum(axis=-1, keepdims=True)) @ vv[b, h // grp]

    if rows is not None:
        rows = np.asarray(rows).reshape(-1, 3)
        out = np.empty((rows.shape[0], D), np.float64)
        for idx, (b, h, i) in enumerate(rows):
            out[idx] = one(b, h, np.array([i]))[0]
        return out
    out = np.empty((B, N, Hq, D), np.float64)
    for b in range(B):
        for h in range(Hq):
            for s0 in range(0, N, 1024):
                out[b, s0:s0 + 1024, h] = one(b, h, np.arange(s0, min(N, s0 + 1024)))
    return out


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


# ----------------------------------------------------------------------------
# Decode-time INT8 K cache (per-head Hadamard rotation, one scale per token)
# ----------------------------------------------------------------------------

def kv_quant(k: torch.Tensor):
    """Cache entries of BF16 K rows k [B, T, H, D] (CPU tensor, any strides,
    unit d stride): (k8 int8 [B, H, T, D], kscale float32 [B, H, T])."""
    B, T, H, D = k.shape
    if k.stride(3) != 1:
        k = k.contiguous()
    k8 = np.empty((B, H, T, D), np.int8)
    ks = np.empty((B, H, T), np.float32)
    sb, sn, sh, _ = k.stride()
    lib().oracle_kv_quant(B, T, H, D, ctypes.c_void_p(k.data_ptr()), sb, sn, sh, _ptr(k8), _ptr(ks))
    return k8, ks


def decode_attn(q: torch.Tensor, k8: np.ndarray, kscale: np.ndarray, v_cache: np.ndarray, T: int):
    """Single-query attention over the first T cached tokens.
    q BF16 [B, Hq, D]; k8 [B, Hkv, Tc, D]; kscale [B, Hkv, Tc]; v_cache BF16
    bits uint16 [B, Hkv, Tc, D].  Returns (o uint16 BF16 [B, Hq, D],
    weights float64 [B, Hq, T])."""
    B, Hq, D = q.shape
    Hkv, Tc = k8.shape[1], k8.shape[2]
    qb = np.ascontiguousarray(q.contiguous().view(torch.int16).numpy().view(np.uint16))
    k8 = np.ascontiguousarray(k8)
    kscale = np.ascontiguousarray(kscale, np.float32)
    v_cache = np.ascontiguousarray(v_cache, np.uint16)
    o = np.empty((B, Hq, D), np.uint16)
    w = np.empty((B, Hq, max(T, 1)), np.float64)
    lib().oracle_decode_attn(B, Hq, Hkv, D, T, Tc, _ptr(qb), _ptr(k8), _ptr(kscale), _ptr(v_cache),
                             _ptr(o), _ptr(w))
    return o, w[:, :, :T]


def decode_attn_v8(q: torch.Tensor, k8: np.ndarray, kscale: np.ndarray, v8: np.ndarray, vscale: np.ndarray,
                   T: int):
    """decode_attn over a cache whose V rows are stored like K rows (rotated
    INT8 v8 [B, Hkv, Tc, D], FP32 vscale [B, Hkv, Tc], as kv_quant gives them);
    the output is rotated back.  Returns (o uint16 BF16 [B, Hq, D], weights
    float64 [B, Hq, T])."""
    B, Hq, D = q.shape
    Hkv, Tc = k8.shape[1], k8.shape[2]
    qb = np.ascontiguousarray(q.contiguous().view(torch.int16).numpy().view(np.uint16))
    k8, v8 = np.ascontiguousarray(k8, np.int8), np.ascontiguousarray(v8, np.int8)
    kscale = np.ascontiguousarray(kscale, np.float32)
    vscale = np.ascontiguousarray(vscale, np.float32)
    o = np.empty((B, Hq, D), np.uint16)
    w = np.empty((B, Hq, max(T, 1)), np.float64)
    lib().oracle_decode_attn_v8(B, Hq, Hkv, D, T, Tc, _ptr(qb), _ptr(k8), _ptr(kscale), _ptr(v8), _ptr(vscale),
                                _ptr(o), _ptr(w))
    return o, w[:, :, :T]
