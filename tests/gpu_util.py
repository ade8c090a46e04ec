"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI, and bring results back in the oracle's logical
layouts.  Imports the HIP binding lazily so CPU-only collection never needs it."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerance on the BF16 attention output against the oracle: max-abs and cosine.
MAX_ABS = 2e-2
MIN_COS = 0.999


def banner(msg: str) -> None:
    """Name the case on stdout before a GPU step (a crash then still says which)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_device(inp, device="cuda:0"):
    """Q/K/V device views with the same strides as the host inputs."""
    if inp.qkv is not None:
        buf = inp.qkv.to(device)
        B, N, _ = buf.shape
        Hq, Hkv, D = inp.cfg.Hq, inp.cfg.Hkv, inp.cfg.D
        q = buf[:, :, 0:Hq * D].view(B, N, Hq, D)
        k = buf[:, :, Hq * D:(Hq + Hkv) * D].view(B, N, Hkv, D)
        v = buf[:, :, (Hq + Hkv) * D:].view(B, N, Hkv, D)
        keep = buf
    else:
        q, k, v = inp.q.to(device), inp.k.to(device), inp.v.to(device)
        keep = None
    return dict(q=q, k=k, v=v, w_q=inp.w_q.to(device), w_k=inp.w_k.to(device),
                cos=inp.cos.to(device).contiguous(), sin=inp.sin.to(device).contiguous(), keep=keep)


def shape_of(inp, **over):
    import quantized_exact_order_amd as sage
    c = inp.cfg
    B, N = inp.q.shape[0], inp.q.shape[1]
    kw = dict(B=B, N=N, Hq=c.Hq, Hkv=c.Hkv, D=c.D, rope_dim=c.rope_dim, hadamard=c.hadamard, eps=c.eps)
    kw.update(over)
    return sage.Shape(**kw)


def run_path(inp, dev=None, shape=None, attn=True, fill_sentinel=False):
    """Run sage_prep, sage_quant_qk and (optionally) sage_attn_fwd on the GPU."""
    import quantized_exact_order_amd as sage
    dev = dev or to_device(inp)
    shape = shape or shape_of(inp)
    bufs = sage.Buffers.allocate(shape, dev["q"].device)
    if fill_sentinel:
        for t in (bufs.q8, bufs.k8, bufs.v8):
            t.fill_(0x5A)
    args = (dev["q"], dev["k"], dev["v"], dev["w_q"], dev["w_k"], dev["cos"], dev["sin"])
    sage.prep(shape, bufs, *args)
    sage.quant_qk(shape, bufs, *args)
    o = None
    if attn:
        o = sage.attn_fwd(shape, bufs)
    torch.cuda.synchronize()
    return shape, bufs, o


def host_tensors(shape, bufs):
    """GPU buffers as numpy arrays in the oracle's logical layouts (valid rows)."""
    import quantized_exact_order_amd as sage
    N = shape.N
    return dict(
        q8=bufs.q8[:, :, :N].cpu().numpy(),
        q_scale=bufs.q_scale.cpu().numpy(),
        k8=bufs.k8[:, :, :N].cpu().numpy(),
        k_scale=bufs.k_scale.cpu().numpy(),
        k_mean=bufs.k_mean.cpu().numpy(),
        v8=sage.v8_logical(shape, bufs).cpu().numpy(),
        v_scale=bufs.v_scale.cpu().numpy(),
    )


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def assert_prep_bit_exact(ref, got, label=""):
    """Every prepared tensor byte-identical to the oracle's."""
    for name in ("k_mean", "v_scale", "q_scale", "k_scale", "q8", "k8", "v8"):
        a = getattr(ref, name)
        b = got[name]
        assert a.shape == b.shape, (label, name, a.shape, b.shape)
        if a.dtype == np.float32:
            same = a.view(np.uint32) == b.view(np.uint32)
        else:
            same = a == b
        if not same.all():
            idx = np.argwhere(~same)[:5]
            raise AssertionError(f"{label}: {name} differs at {len(np.argwhere(~same))} places, "
                                 f"first {idx.tolist()}: oracle {a[tuple(idx[0])]} gpu {b[tuple(idx[0])]}")


def compare_output(o_gpu_rows: np.ndarray, o_ref_rows: np.ndarray, label=""):
    """BF16 rows (as float) against the oracle: max-abs and cosine."""
    import oracle
    a = np.asarray(o_gpu_rows, np.float64)
    b = np.asarray(o_ref_rows, np.float64)
    err = float(np.abs(a - b).max()) if a.size else 0.0
    cos = oracle.cosine(a, b) if a.size else 1.0
    assert err <= MAX_ABS, f"{label}: max-abs {err:.4g} > {MAX_ABS}"
    assert cos >= MIN_COS, f"{label}: cosine {cos:.6f} < {MIN_COS}"
    return err, cos
