"""Seeded synthetic inputs for the quantized attention path.

This module is the only code shared by the CPU oracle (``oracle/``) and the HIP
path (``quantized_exact_order_amd/``).  It draws random numbers and rounds them
to BF16 storage; it performs none of the method's arithmetic (no RMSNorm, RoPE,
smoothing, quantization or attention).

Workloads follow the shapes the pages use ("Exact Numerical Contract",
section "Canonical Boundary": B=1, N=37,810, 56 heads, D=128, Q/K/V as views of
one interleaved QKV row of width 21,504 at element offsets 0 / 7,168 / 14,336;
the FP8-PV page's 729-key, 27-layer encoder) plus small and ragged cases.

Recipe (every config):
  * ``numpy.random.SeedSequence(seed).spawn(7)`` gives independent streams for
    q, k, v, k_bias, w_q, w_k and the outlier mask, in that order;
  * q, k, v ~ N(0,1) drawn in FP32; k += bias[h, d] with bias ~ N(0, 4)
    (standard deviation 2), added in FP32;
  * optional outliers: a Bernoulli(p) mask per Q/K entry multiplies the FP32
    value by a factor before rounding;
  * RMSNorm weights: ones, or U(lo, hi) drawn in FP32;
  * everything is rounded once to BF16 (round-to-nearest-even, torch's
    float32 -> bfloat16 conversion);
  * RoPE coefficient tables cos/sin[n, i] for positions n = 0..N-1 and
    frequencies theta_i = base**(-2 i / R), i < R/2, computed in FP64, then
    rounded to FP32 and then to BF16.  The pages fix that the coefficients are
    BF16 values; the frequency formula belongs to the model feeding the path.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    rope_dim: int
    hadamard: bool = False
    eps: float = 1e-5
    rope_base: float = 10000.0
    weights: Optional[tuple] = None      # None = unit weights, else (lo, hi) uniform
    outlier_frac: float = 0.0
    outlier_mult: float = 20.0
    interleaved: bool = False            # Q/K/V as views of one [N, (Hq+2Hkv)*D] buffer
    layers: int = 1                      # independent seeded layers (encoder config)
    seed: int = 0

    @property
    def scores(self) -> int:
        return self.B * self.N * self.N * self.Hq

    @property
    def attn_ops(self) -> int:
        """Algorithmic operations of one attention: 4 N^2 H D (QK^T and PV)."""
        return 4 * self.B * self.N * self.N * self.Hq * self.D


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", B=1, N=256, Hq=2, Hkv=2, D=128, rope_dim=96, seed=1),
    "tail": Config("tail", B=1, N=1000, Hq=8, Hkv=8, D=128, rope_dim=96,
                   weights=(0.5, 1.5), outlier_frac=0.01, outlier_mult=20.0, seed=2),
    "encoder": Config("encoder", B=1, N=729, Hq=16, Hkv=16, D=128, rope_dim=96,
                      layers=27, seed=1000),
    "gqa": Config("gqa", B=1, N=8192, Hq=16, Hkv=4, D=256, rope_dim=192,
                  hadamard=True, seed=4),
    "canonical": Config("canonical", B=1, N=37810, Hq=56, Hkv=56, D=128, rope_dim=96,
                        interleaved=True, seed=5),
}


def bf16_from_f32(x: np.ndarray) -> torch.Tensor:
    """Round an FP32 array to a BF16 torch tensor (RNE, torch's own conversion)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def rope_tables(N: int, rope_dim: int, base: float = 10000.0):
    """BF16 cos/sin tables [N, rope_dim/2] for positions 0..N-1 (FP64 -> FP32 -> BF16)."""
    half = rope_dim // 2
    if half == 0:
        z = torch.zeros((N, 0), dtype=torch.bfloat16)
        return z, z.clone()
    i = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * i / rope_dim)
    ang = np.arange(N, dtype=np.float64)[:, None] * theta[None, :]
    return (bf16_from_f32(np.cos(ang).astype(np.float32)),
            bf16_from_f32(np.sin(ang).astype(np.float32)))


@dataclasses.dataclass
class Inputs:
    """One layer's inputs on the host.  q/k/v are BF16 [B, N, H, D] views
    (strided views of one buffer when ``qkv`` is set)."""
    cfg: Config
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    w_q: torch.Tensor      # BF16 [D]
    w_k: torch.Tensor      # BF16 [D]
    cos: torch.Tensor      # BF16 [N, R/2]
    sin: torch.Tensor      # BF16 [N, R/2]
    qkv: Optional[torch.Tensor] = None   # BF16 [B, N, (Hq+2Hkv)*D] backing buffer


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_inputs(cfg: Config, layer: int = 0, N: Optional[int] = None) -> Inputs:
    """Deterministic inputs for ``cfg`` (layer ``layer``; ``N`` overrides the length)."""
    N = cfg.N if N is None else N
    B, Hq, Hkv, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.D
    ss = np.random.SeedSequence(cfg.seed + layer)
    rq, rk, rv, rb, rwq, rwk, rmask = [np.random.default_rng(s) for s in ss.spawn(7)]

    qf = _normal(rq, (B, N, Hq, D))
    kf = _normal(rk, (B, N, Hkv, D))
    vf = _normal(rv, (B, N, Hkv, D))
    bias = (_normal(rb, (Hkv, D)) * np.float32(2.0)).astype(np.float32)
    kf += bias[None, None, :, :]
    if cfg.outlier_frac > 0.0:
        mq = rmask.random(size=qf.shape, dtype=np.float32) < cfg.outlier_frac
        mk = rmask.random(size=kf.shape, dtype=np.float32) < cfg.outlier_frac
        qf[mq] *= np.float32(cfg.outlier_mult)
        kf[mk] *= np.float32(cfg.outlier_mult)
    if cfg.weights is None:
        wq = np.ones(D, np.float32)
        wk = np.ones(D, np.float32)
    else:
        lo, hi = cfg.weights
        wq = rwq.uniform(lo, hi, size=D).astype(np.float32)
        wk = rwk.uniform(lo, hi, size=D).astype(np.float32)
    cos, sin = rope_tables(N, cfg.rope_dim, cfg.rope_base)

    if cfg.interleaved:
        W = (Hq + 2 * Hkv) * D
        buf = torch.empty((B, N, W), dtype=torch.bfloat16)
        buf[:, :, 0:Hq * D] = bf16_from_f32(qf.reshape(B, N, Hq * D))
        del qf
        buf[:, :, Hq * D:(Hq + Hkv) * D] = bf16_from_f32(kf.reshape(B, N, Hkv * D))
        del kf
        buf[:, :, (Hq + Hkv) * D:] = bf16_from_f32(vf.reshape(B, N, Hkv * D))
        del vf
        q = buf[:, :, 0:Hq * D].view(B, N, Hq, D)
        k = buf[:, :, Hq * D:(Hq + Hkv) * D].view(B, N, Hkv, D)
        v = buf[:, :, (Hq + Hkv) * D:].view(B, N, Hkv, D)
        return Inputs(cfg, q, k, v, bf16_from_f32(wq), bf16_from_f32(wk), cos, sin, qkv=buf)
    return Inputs(cfg, bf16_from_f32(qf), bf16_from_f32(kf), bf16_from_f32(vf),
                  bf16_from_f32(wq), bf16_from_f32(wk), cos, sin)


def make_custom(B: int, N: int, Hq: int, Hkv: int, D: int, rope_dim: int, seed: int,
                hadamard: bool = False, weights=None, outlier_frac: float = 0.0,
                outlier_mult: float = 20.0, interleaved: bool = False) -> Inputs:
    """Inputs for an ad-hoc shape with the same recipe (edge sweeps)."""
    cfg = Config(f"custom_{B}x{N}x{Hq}x{Hkv}x{D}", B=B, N=N, Hq=Hq, Hkv=Hkv, D=D,
                 rope_dim=rope_dim, hadamard=hadamard, weights=weights,
                 outlier_frac=outlier_frac, outlier_mult=outlier_mult,
                 interleaved=interleaved, seed=seed)
    return make_inputs(cfg)
