"""Metamorphic GPU-vs-GPU checks (bitwise) and untouched-memory sentinels.

Each check compares the HIP path with itself under a transformation that must
not change any byte: strided interleaved views vs contiguous copies, two runs
(no atomics, no split over keys), a batch of two vs two batches of one, a
permutation of heads.  Sentinels check that padding rows are zero and that
output rows beyond N, and bytes around the output, are never written.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import banner, run_path, shape_of, to_device

pytestmark = pytest.mark.gpu


def _all(bufs, o):
    return [bufs.q8, bufs.q_scale, bufs.k8, bufs.k_scale, bufs.k_mean, bufs.v8, bufs.v_scale, o]


def _equal(a, b):
    return all(torch.equal(x.view(torch.uint8) if x.dtype != torch.bfloat16 else x.view(torch.int16),
                           y.view(torch.uint8) if y.dtype != torch.bfloat16 else y.view(torch.int16))
               for x, y in zip(a, b))


def test_interleaved_views_equal_contiguous_copies():
    cfg = workloads.Config("mm", B=1, N=777, Hq=4, Hkv=4, D=128, rope_dim=96, interleaved=True, seed=60)
    inp = workloads.make_inputs(cfg)
    banner("interleaved vs contiguous")
    _, b1, o1 = run_path(inp)
    dev = to_device(inp)
    for key in ("q", "k", "v"):
        dev[key] = dev[key].contiguous()
    _, b2, o2 = run_path(inp, dev=dev)
    assert _equal(_all(b1, o1), _all(b2, o2))


def test_two_runs_are_identical():
    inp = workloads.make_inputs(workloads.CONFIGS["tail"])
    banner("determinism")
    _, b1, o1 = run_path(inp)
    _, b2, o2 = run_path(inp)
    assert _equal(_all(b1, o1), _all(b2, o2))


def test_batch_of_two_equals_two_batches_of_one():
    inp = workloads.make_custom(2, 300, 2, 2, 128, 96, seed=61)
    banner("batch split")
    shape, b2, o2 = run_path(inp)
    for bi in range(2):
        one = workloads.Inputs(inp.cfg, inp.q[bi:bi + 1].clone(), inp.k[bi:bi + 1].clone(),
                               inp.v[bi:bi + 1].clone(), inp.w_q, inp.w_k, inp.cos, inp.sin)
        _, b1, o1 = run_path(one)
        assert torch.equal(o1[0].view(torch.int16), o2[bi].view(torch.int16))
        assert torch.equal(b1.q8[0], b2.q8[bi]) and torch.equal(b1.v8[0], b2.v8[bi])
        assert torch.equal(b1.k_mean[0], b2.k_mean[bi])


def test_head_permutation_permutes_outputs():
    inp = workloads.make_custom(1, 200, 4, 4, 128, 96, seed=62)
    banner("head permutation")
    _, b1, o1 = run_path(inp)
    perm = [2, 0, 3, 1]
    pin = workloads.Inputs(inp.cfg, inp.q[:, :, perm].clone(), inp.k[:, :, perm].clone(),
                           inp.v[:, :, perm].clone(), inp.w_q, inp.w_k, inp.cos, inp.sin)
    _, b2, o2 = run_path(pin)
    assert torch.equal(o1[:, :, perm].view(torch.int16), o2.view(torch.int16))
    assert torch.equal(b1.k_mean[:, perm], b2.k_mean) and torch.equal(b1.q_scale[:, perm], b2.q_scale)


def test_padding_rows_zero_and_output_sentinels():
    import quantized_exact_order_amd as sage
    N = 150
    inp = workloads.make_custom(1, N, 2, 2, 128, 96, seed=63)
    banner("sentinels")
    shape, bufs, _ = run_path(inp, attn=False, fill_sentinel=True)
    assert bool((bufs.q8[:, :, N:] == 0).all()) and bool((bufs.k8[:, :, N:] == 0).all())
    slot_keys = torch.tensor(sage.v8_slot_keys(), device=bufs.v8.device)
    last = bufs.v8[:, :, -1]                                   # [B,Hkv,D,64]
    invalid = (slot_keys + 64 * (bufs.v8.shape[2] - 1)) >= N
    assert bool((last[..., invalid] == 0).all())
    # output written into the middle of a larger buffer: guard rows and the
    # rows >= N keep their sentinel
    big = torch.full((1, N + 40, 2, 128), -7.0, dtype=torch.bfloat16, device=bufs.q8.device)
    view = big[:, 8:8 + N + 16]                                # 16 extra rows past N
    sage.attn_fwd(shape, bufs, o=view)
    torch.cuda.synchronize()
    assert bool((big[:, :8] == -7.0).all()) and bool((big[:, 8 + N:] == -7.0).all())
    assert bool(torch.isfinite(big[:, 8:8 + N].float()).all())
