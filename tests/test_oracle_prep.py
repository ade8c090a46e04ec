"""Pins of the oracle's preparation steps (RMSNorm, RoPE, K mean, quantization,
Walsh-Hadamard rotation) against closed forms, FP64 arithmetic, invariants and
library routines -- page "Exact Numerical Contract", sections "Preparation"
and "Q And K Quantization", and the NPU issue on Hadamard-rotated INT8 K.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import workloads


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)


def _ulp_bf16(y):
    """Spacing of BF16 numbers at |y| (FP64)."""
    a = np.maximum(np.abs(y), 2.0**-126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _run_norm(oracle_lib, x, w=None, R=0, cos=None, sin=None, eps=1e-5):
    B, N, H, D = x.shape
    w = _bf16(np.ones(D)) if w is None else w
    if cos is None:
        cos = torch.zeros((N, max(R // 2, 0)), dtype=torch.bfloat16)
        sin = cos.clone()
    return oracle_lib.bf16_to_f32(oracle_lib.rmsnorm_rope(x, w, cos, sin, R, eps))


# ---------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("c", [1.0, -3.5, 0.0078125, 0.001, 100.0])
def test_rmsnorm_constant_row_closed_form(oracle_lib, c):
    # x_d = c for every d: the mean square is exactly c^2, so y = c / sqrt(c^2 + eps)
    D = 128
    x = _bf16(np.full((1, 2, 1, D), c))
    cb = float(x.float()[0, 0, 0, 0])
    y = _run_norm(oracle_lib, x)
    exact = cb / math.sqrt(cb * cb + 1e-5)
    assert np.all(np.abs(y - exact) <= _ulp_bf16(exact))


def test_rmsnorm_zero_row_is_zero(oracle_lib):
    y = _run_norm(oracle_lib, _bf16(np.zeros((1, 3, 2, 128))))
    assert np.all(y == 0.0)


@pytest.mark.parametrize("D", [128, 256])
def test_rmsnorm_matches_fp64_within_one_bf16_ulp(oracle_lib, D):
    rng = np.random.default_rng(10)
    N, H = 64, 3
    x = rng.standard_normal((1, N, H, D)).astype(np.float32)
    x[0, :8] *= 1e-3     # mean square ~1e-6: eps = 1e-5 dominates here
    x[0, 8:16] *= 50.0
    xb = _bf16(x)
    w = _bf16(rng.uniform(0.5, 1.5, D))
    y = _run_norm(oracle_lib, xb, w=w)                      # [1,H,N,D]
    x64 = xb.double().numpy().transpose(0, 2, 1, 3)
    w64 = w.double().numpy()
    ref = x64 / np.sqrt(np.mean(x64 * x64, axis=-1, keepdims=True) + 1e-5) * w64
    assert np.all(np.abs(y - ref) <= _ulp_bf16(ref))


# ---------------------------------------------------------------- RoPE

def test_rope_position_zero_and_tail_dims_are_identity(oracle_lib):
    rng = np.random.default_rng(11)
    N, H, D, R = 40, 2, 128, 96
    x = _bf16(rng.standard_normal((1, N, H, D)))
    cos, sin = workloads.rope_tables(N, R)
    z = _run_norm(oracle_lib, x, R=R, cos=cos, sin=sin)
    y = _run_norm(oracle_lib, x, R=0)
    assert np.array_equal(z[:, :, 0], y[:, :, 0])            # cos=1, sin=0 at n=0
    assert np.array_equal(z[..., R:], y[..., R:])            # dims >= R unrotated


@pytest.mark.parametrize("D,R", [(128, 96), (256, 192), (128, 128), (128, 2)])
def test_rope_is_split_half_rotation_fp64(oracle_lib, D, R):
    rng = np.random.default_rng(12)
    N, H = 50, 2
    x = _bf16(rng.standard_normal((1, N, H, D)))
    cos, sin = workloads.rope_tables(N, R)
    z = _run_norm(oracle_lib, x, R=R, cos=cos, sin=sin)
    y = _run_norm(oracle_lib, x, R=0).astype(np.float64)
    c = cos.double().numpy()[None, None]
    s = sin.double().numpy()[None, None]
    h = R // 2
    a, b = y[..., :h], y[..., h:R]
    ref = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    assert np.all(np.abs(z[..., :R] - ref) <= _ulp_bf16(ref) * 0.5 + 1e-30)


def test_rope_preserves_pair_norms_and_relative_positions(oracle_lib):
    rng = np.random.default_rng(13)
    N, D, R = 64, 128, 96
    h = R // 2
    v = rng.standard_normal(D).astype(np.float32)
    x = _bf16(np.broadcast_to(v, (1, N, 1, D)).copy())       # the same vector at every position
    cos, sin = workloads.rope_tables(N, R)
    z = _run_norm(oracle_lib, x, R=R, cos=cos, sin=sin)[0, 0].astype(np.float64)
    y = _run_norm(oracle_lib, x, R=0)[0, 0].astype(np.float64)
    pn_z = np.hypot(z[:, :h], z[:, h:R])
    pn_y = np.hypot(y[:, :h], y[:, h:R])
    assert np.all(np.abs(pn_z - pn_y) <= 2.0**-6 * pn_y + 1e-6)
    # <z_m, z_n> depends on m - n only (up to BF16 coefficient error)
    dots = z[:, :R] @ z[:, :R].T
    for delta in (1, 5, 17):
        diag = np.diagonal(dots, offset=delta)
        assert np.ptp(diag) <= 0.05 * np.abs(dots[0, 0])


# ---------------------------------------------------------------- K mean

def test_k_mean_constant_column_exact(oracle_lib):
    for N in (1, 37, 64, 65, 1000):
        zk = np.full((1, 2, N, 128), 0, np.uint16)
        vals = np.float32([1.5, -0.3125, 2.0**-7, 100.0])
        for i, v in enumerate(vals):
            zk[..., i] = oracle_lib.f32_to_bf16(np.float32([v]))[0]
        mean = oracle_lib.k_mean(zk)
        for i, v in enumerate(vals):
            assert np.all(mean[..., i] == oracle_lib.bf16_to_f32(zk[0, 0, 0, i]))
        assert np.all(mean[..., 4:] == 0.0)


def test_k_mean_tree_has_no_padding_leaf_at_powers_of_two(oracle_lib):
    # IEEE 754: the sum of two zeros of the same sign is that zero, and
    # -0 + +0 = +0 under round-to-nearest.  A column of -0.0 over N = 2^k rows
    # fills the 2^ceil(log2 N) leaves of the tree exactly, so its sum and mean
    # are -0.0; one row more brings in a +0.0 padding leaf and gives +0.0.
    neg0 = np.uint16(0x8000)
    for N in (1, 2, 16, 32, 64, 128):
        zk = np.full((1, 1, N, 128), neg0, np.uint16)
        mean = oracle_lib.k_mean(zk)
        assert np.all(mean.view(np.uint32) == 0x80000000), N
    for N in (3, 17, 33, 65):
        zk = np.full((1, 1, N, 128), neg0, np.uint16)
        mean = oracle_lib.k_mean(zk)
        assert np.all(mean.view(np.uint32) == 0), N


@pytest.mark.parametrize("N", [1, 50, 64, 1000, 4097])
def test_k_mean_matches_fp64(oracle_lib, N):
    rng = np.random.default_rng(14)
    z = oracle_lib.f32_to_bf16(rng.standard_normal((1, 2, N, 128)).astype(np.float32) + 3.0)
    mean = oracle_lib.k_mean(z).astype(np.float64)
    zf = oracle_lib.bf16_to_f32(z).astype(np.float64)
    ref = zf.mean(axis=2)
    # pairwise summation error bound ~ log2(P) * 2^-24 * sum|z| / N
    bound = (math.ceil(math.log2(max(N, 64))) + 2) * 2.0**-24 * np.abs(zf).mean(axis=2)
    assert np.all(np.abs(mean - ref) <= bound + 1e-12)
    # the smoothed columns sum to ~0
    resid = (zf - mean[:, :, None, :]).sum(axis=2)
    assert np.all(np.abs(resid) <= N * 4 * 2.0**-24 * np.abs(zf).max())


# ---------------------------------------------------------------- quantization

def test_q_quant_bounds_groups_and_padding(oracle_lib):
    rng = np.random.default_rng(15)
    N, D = 200, 128                               # 7 groups hold rows; 8 groups allocated
    u = rng.standard_normal((1, 2, N, D)).astype(np.float32)
    u[0, 0, 31, 5] = 40.0                         # spike in the last row of group 0
    u[0, 0, 64:96] = 0.0                          # an all-zero group
    z = oracle_lib.f32_to_bf16(u)
    uf = oracle_lib.bf16_to_f32(z)
    q8, qs = oracle_lib.quant_q(z, hadamard=False)
    assert qs.shape == (1, 2, 8)
    for h in range(2):
        for g in range(8):
            rows = uf[0, h, 32 * g:min(N, 32 * g + 32)]
            amax = max(float(np.abs(rows).max()) if rows.size else 0.0, 1e-7)
            assert qs[0, h, g] == np.float32(np.float32(amax) / np.float32(127.0))
            if rows.size:
                err = np.abs(q8[0, h, 32 * g:32 * g + rows.shape[0]].astype(np.float64) * qs[0, h, g] - rows)
                assert np.all(err <= qs[0, h, g] * (0.5 + 1e-5))
                if amax > 1e-7:
                    assert np.abs(q8[0, h, 32 * g:32 * g + rows.shape[0]]).max() == 127
    assert qs[0, 0, 0] == np.float32(np.float32(40.0) / np.float32(127.0))
    assert qs[0, 0, 1] < qs[0, 0, 0] / 5
    assert np.all(q8[0, 0, 64:96] == 0) and qs[0, 0, 2] == np.float32(np.float32(1e-7) / np.float32(127.0))
    assert qs[0, 0, 7] == np.float32(np.float32(1e-7) / np.float32(127.0))   # no valid row
    assert np.abs(q8).max() <= 127


def test_k_smoothing_and_tile_scales(oracle_lib):
    rng = np.random.default_rng(16)
    N, D = 150, 128                                # tiles of 64, 64, 22 rows
    u = rng.standard_normal((1, 1, N, D)).astype(np.float32)
    u[..., 7] = 2.5                                # constant column: smoothed to exactly 0
    z = oracle_lib.f32_to_bf16(u)
    mean = oracle_lib.k_mean(z)
    k8, ks = oracle_lib.quant_k(z, mean, hadamard=False)
    assert ks.shape == (1, 1, 3)
    assert np.all(k8[..., 7] == 0)
    zf = oracle_lib.bf16_to_f32(z)
    sm = zf - mean[:, :, None, :]
    for t in range(3):
        rows = sm[0, 0, 64 * t:min(N, 64 * t + 64)]
        assert ks[0, 0, t] == np.float32(np.float32(np.abs(rows).max()) / np.float32(127.0))
        err = np.abs(k8[0, 0, 64 * t:64 * t + rows.shape[0]] * np.float64(ks[0, 0, t]) - rows)
        assert np.all(err <= ks[0, 0, t] * (0.5 + 1e-5))


def test_v_quant_per_channel(oracle_lib):
    rng = np.random.default_rng(17)
    N, H, D = 300, 2, 128
    v = rng.standard_normal((1, N, H, D)).astype(np.float32)
    v[:, :, 1, 3] = 0.0                            # all-zero channel: floor 1e-7
    vb = _bf16(v)
    v8, vs = oracle_lib.quant_v(vb)
    vf = vb.double().numpy().transpose(0, 2, 1, 3)
    amax = np.maximum(np.abs(vf).max(axis=2), 1e-7)
    assert np.array_equal(vs, (amax.astype(np.float32) / np.float32(2.25)).astype(np.float32))
    dq = oracle_lib.e4m3_to_f32(v8).astype(np.float64) * vs[:, :, None, :]
    assert np.all(np.abs(dq - vf) <= np.abs(vf) * 2.0**-4 + 2.0**-10 * vs[:, :, None, :] * 1.01)
    # the channel maximum maps to +-2.25 (code 0x41 / 0xC1)
    idx = np.abs(vf[0, 0]).argmax(axis=0)
    assert np.all(np.isin(v8[0, 0, idx, np.arange(D)], [0x41, 0xC1]))
    assert np.all(v8[0, 1, :, 3] == 0)


# ---------------------------------------------------------------- Hadamard

@pytest.mark.parametrize("D", [16, 256])
def test_wht_matches_scipy_and_is_involution(oracle_lib, D):
    rng = np.random.default_rng(18)
    u = rng.standard_normal((20, D)).astype(np.float32)
    w = oracle_lib.wht(u)
    Hm = scipy.linalg.hadamard(D).astype(np.float64) / math.sqrt(D)
    ref = u.astype(np.float64) @ Hm.T
    assert np.allclose(w, ref, rtol=0, atol=1e-5 * np.abs(u).max() * math.log2(D))
    back = oracle_lib.wht(w)
    assert np.allclose(back, u, rtol=0, atol=1e-5 * np.abs(u).max() * math.log2(D))


def test_wht_leaves_scores_unchanged(oracle_lib):
    rng = np.random.default_rng(19)
    q = rng.standard_normal((8, 256)).astype(np.float32)
    k = rng.standard_normal((32, 256)).astype(np.float32)
    s0 = q.astype(np.float64) @ k.T.astype(np.float64)
    s1 = oracle_lib.wht(q).astype(np.float64) @ oracle_lib.wht(k).T.astype(np.float64)
    assert np.max(np.abs(s1 - s0)) <= 1e-5 * np.abs(s0).max()


def test_hadamard_quant_rotates_before_scaling(oracle_lib):
    rng = np.random.default_rng(20)
    u = rng.standard_normal((1, 1, 64, 256)).astype(np.float32)
    u[..., 9] *= 30.0                              # outlier channel, spread by the rotation
    z = oracle_lib.f32_to_bf16(u)
    q8h, qsh = oracle_lib.quant_q(z, hadamard=True)
    rot = oracle_lib.wht(oracle_lib.bf16_to_f32(z))
    for g in range(2):
        rows = rot[0, 0, 32 * g:32 * g + 32]
        assert qsh[0, 0, g] == np.float32(np.float32(np.abs(rows).max()) / np.float32(127.0))
    q8p, qsp = oracle_lib.quant_q(z, hadamard=False)
    assert np.all(qsh[..., :2] < qsp[..., :2])     # rotation shrinks the outlier's range
