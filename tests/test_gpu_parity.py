"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Preparation outputs (k_mean, v_scale, q8, q_scale, k8, k_scale, v8) must be
byte-identical; the BF16 attention output must be within max-abs 2e-2 and
cosine 0.999 of the oracle (overall and per head).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (assert_prep_bit_exact, banner, bf16_bits, compare_output, host_tensors,
                      run_path, to_device)

pytestmark = pytest.mark.gpu


def _full_check(inp, label, attn_rows=None):
    banner(f"{label}: N={inp.q.shape[1]} Hq={inp.cfg.Hq} Hkv={inp.cfg.Hkv} D={inp.cfg.D}")
    ref = oracle.prepare(inp)
    shape, bufs, o = run_path(inp)
    assert_prep_bit_exact(ref, host_tensors(shape, bufs), label)
    B, N, Hq, D = o.shape
    if attn_rows is None:
        o_ref = oracle.bf16_to_f32(oracle.attention(ref))               # [B,N,Hq,D]
        o_gpu = oracle.bf16_to_f32(bf16_bits(o))
        compare_output(o_gpu, o_ref, label)
        for h in range(Hq):
            compare_output(o_gpu[:, :, h], o_ref[:, :, h], f"{label} head {h}")
    else:
        o_ref = oracle.bf16_to_f32(oracle.attn_rows(ref, attn_rows))
        o_gpu = oracle.bf16_to_f32(bf16_bits(o))[attn_rows[:, 0], attn_rows[:, 2], attn_rows[:, 1]]
        compare_output(o_gpu, o_ref, label)
        for h in np.unique(attn_rows[:, 1]):
            sel = attn_rows[:, 1] == h
            compare_output(o_gpu[sel], o_ref[sel], f"{label} head {h}")
    return ref, shape, bufs, o


@pytest.mark.parametrize("name", ["tiny", "tail"])
def test_config_full(name):
    _full_check(workloads.make_inputs(workloads.CONFIGS[name]), name)


@pytest.mark.parametrize("B,N,Hq,Hkv,rope", [(2, 700, 8, 2, 96), (1, 333, 14, 2, 96), (1, 200, 4, 1, 0)])
def test_gqa_d128(B, N, Hq, Hkv, rope):
    # grouped query heads on the D = 128 kernels: query head h reads KV head
    # h / (Hq / Hkv) (groups of 4, 7 and 4, two sequences, one without RoPE)
    inp = workloads.make_custom(B, N, Hq, Hkv, 128, rope, seed=90 + Hq, outlier_frac=0.01)
    _full_check(inp, f"gqa d128 {Hq}/{Hkv}")


@pytest.mark.parametrize("layer", [0, 13, 26])
def test_encoder_layer(layer):
    cfg = workloads.CONFIGS["encoder"]
    _full_check(workloads.make_inputs(cfg, layer=layer), f"encoder layer {layer}")


def _sample_rows(B, H, N, per_head, rng, tail=64):
    rows = []
    for b in range(B):
        for h in range(H):
            pick = set(rng.choice(N, size=min(per_head, N), replace=False).tolist())
            pick |= set(range(min(32, N)))                       # first Q group
            pick |= set(range(max(0, N - tail), N))              # ragged last Q tile
            rows += [(b, h, i) for i in sorted(pick)]
    return np.array(rows, np.int32)


@pytest.mark.timeout(600)
def test_gqa_hadamard_d256():
    cfg = workloads.CONFIGS["gqa"]
    inp = workloads.make_inputs(cfg)
    rng = np.random.default_rng(40)
    rows = _sample_rows(1, cfg.Hq, cfg.N, 48, rng, tail=8)
    _full_check(inp, "gqa", attn_rows=rows)


@pytest.mark.timeout(900)
def test_canonical_interleaved_sampled():
    # every one of the 56 heads: its first 32-row query group, the 50 valid
    # rows of its last 128-row query tile (the contract page's final Q128 CTA)
    # and 16 random rows; the tolerance holds per head
    cfg = workloads.CONFIGS["canonical"]
    inp = workloads.make_inputs(cfg)
    rng = np.random.default_rng(41)
    rows = []
    for h in range(cfg.Hq):
        pick = set(rng.choice(cfg.N, size=16, replace=False).tolist())
        pick |= set(range(0, 32)) | set(range(cfg.N - 50, cfg.N))     # first group, 50-row tail
        rows += [(0, h, i) for i in sorted(pick)]
    _full_check(inp, "canonical", attn_rows=np.array(rows, np.int32))


EDGE_N = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257, 768]


@pytest.mark.parametrize("N", EDGE_N)
def test_edge_lengths_d128(N):
    inp = workloads.make_custom(1, N, 2, 2, 128, 96, seed=100 + N)
    _full_check(inp, f"edge N={N}")


@pytest.mark.parametrize("N", [1, 17, 65, 200])
def test_edge_lengths_d256_gqa_hadamard(N):
    inp = workloads.make_custom(1, N, 4, 2, 256, 192, seed=200 + N, hadamard=True)
    _full_check(inp, f"edge d256 N={N}")


@pytest.mark.parametrize("N,D", [(1, 128), (64, 128), (129, 128), (1, 256), (100, 256)])
def test_single_head(N, D):
    inp = workloads.make_custom(1, N, 1, 1, D, D * 3 // 4, seed=600 + N + D)
    _full_check(inp, f"one head N={N} D={D}")


def test_d256_without_rotation_or_groups():
    inp = workloads.make_custom(2, 300, 2, 2, 256, 192, seed=650, outlier_frac=0.01)
    _full_check(inp, "d256 plain")


@pytest.mark.parametrize("R", [0, 2, 40, 128])
def test_rope_dims(R):
    # R/2 not a multiple of 8 takes the per-element RoPE path
    inp = workloads.make_custom(1, 150, 2, 1, 128, R, seed=300 + R)
    _full_check(inp, f"rope_dim={R}")


@pytest.mark.parametrize("R,D", [(0, 128), (64, 128), (0, 256), (128, 256)])
def test_absent_weights_and_tables(R, D):
    # NULL RMSNorm weights stand for unit weights, and with no rotation the
    # RoPE tables may be absent as well: the outputs equal those of the unit
    # weights the inputs are drawn with
    inp = workloads.make_custom(1, 200, 2, 1, D, R, seed=700 + R + D)
    banner(f"absent weights, rope_dim={R} D={D}")
    ref = oracle.prepare(inp)
    dev = to_device(inp)
    assert bool((inp.w_q.float() == 1).all()) and bool((inp.w_k.float() == 1).all())
    dev["w_q"] = dev["w_k"] = None
    if R == 0:
        dev["cos"] = dev["sin"] = None
    shape, bufs, o = run_path(inp, dev=dev)
    assert_prep_bit_exact(ref, host_tensors(shape, bufs), "absent weights")
    compare_output(oracle.bf16_to_f32(bf16_bits(o)), oracle.bf16_to_f32(oracle.attention(ref)), "absent weights")


def test_extreme_outliers_and_weights():
    inp = workloads.make_custom(1, 333, 3, 3, 128, 96, seed=400, weights=(0.5, 1.5),
                                outlier_frac=0.02, outlier_mult=1000.0)
    _full_check(inp, "outliers x1000")


def test_batch_two_and_zero_rows():
    inp = workloads.make_custom(2, 190, 2, 2, 128, 96, seed=500)
    inp.q[1, 5] = 0            # a zero query row (all scores 0, averages V)
    inp.k[0, 77] = 0           # a zero key row
    inp.v[:, :, 1, 9] = 0      # an all-zero V channel: amax floored at 1e-7
    _full_check(inp, "batch 2 with zero rows")


def test_constant_keys_give_uniform_weights():
    # every K row of head 0 equal and no RoPE: the pairwise K mean is that row
    # exactly (300 x a BF16 value is exact in FP32), so smoothing leaves
    # zeros, every key tile quantizes under the 1e-7 floor, all scores of the
    # head are 0 and each output row is the weighted mean of the V rows with
    # equal weights
    inp = workloads.make_custom(1, 300, 2, 2, 128, 0, seed=710)
    inp.k[:, :, 0] = inp.k[:, :1, 0]
    ref, shape, bufs, o = _full_check(inp, "constant keys")
    assert not ref.k8[0, 0, :300].any()


def test_matching_query_and_key_rows_give_peaked_weights():
    # q = k without RoPE: the diagonal score |y|^2 ~ D stands far above the
    # others, so every row's weights are sharply peaked at its own key
    inp = workloads.make_custom(1, 400, 2, 2, 128, 0, seed=720)
    inp.q[:] = inp.k
    _full_check(inp, "q = k")


@pytest.mark.parametrize("N", [1, 16, 17, 32, 64])
def test_negative_zero_key_channel(N):
    # a K channel of -0.0 in every row (a channel past the rotated ones, so
    # RMSNorm and RoPE keep the sign): over N = 2^k rows the K-mean tree has
    # no padding leaf and the mean is -0.0, else a +0.0 leaf makes it +0.0
    inp = workloads.make_custom(1, N, 2, 2, 128, 96, seed=740 + N)
    inp.k[:, :, 1, 100] = -0.0
    ref, shape, bufs, o = _full_check(inp, f"-0.0 key channel N={N}")
    want = 0x80000000 if N & (N - 1) == 0 else 0
    assert ref.k_mean.view(np.uint32)[0, 1, 100] == want


def test_constant_v():
    # head 1 has V = -0.5 everywhere (E4M3 code of -2.25 after scaling, exact)
    # and head 0 one constant channel
    inp = workloads.make_custom(1, 257, 2, 2, 128, 96, seed=730)
    inp.v[:, :, 1] = -0.5
    inp.v[:, :, 0, 5] = 3.0
    ref, shape, bufs, o = _full_check(inp, "constant V")
    assert (o[0, :, 1].float() - (-0.5)).abs().max().item() < 2e-2


def test_infinite_element_in_a_query_row():
    # one +Inf in a Q row: its RMSNorm scale becomes 0, so that element is
    # Inf * 0 = NaN (as is its RoPE partner) and the rest of the row is 0;
    # the INT8 conversion sends NaN to 0, so the row quantizes to zeros and
    # every prep tensor stays byte-identical to the oracle
    inp = workloads.make_custom(1, 150, 2, 2, 128, 96, seed=700)
    inp.q[0, 40, 1, 10] = float("inf")
    ref, shape, bufs, o = _full_check(inp, "Inf in a Q row")
    assert not ref.q8[0, 1, 40].any()
    assert torch.isfinite(o.float()).all()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,H,N,D,R", [(64, 64, 4200, 128, 96), (32, 32, 8400, 256, 192)])
def test_buffers_past_2_31_elements(B, H, N, D, R):
    # every Q/K/V, q8/k8/v8 and O tensor holds 2.2e9 elements (past 2^31; the
    # BF16 ones past 2^32 bytes), for each head width's kernel.  The GPU runs
    # the whole problem; heads are independent, so the oracle prepares single
    # (b, h) slices, among them the last one at the far end of every buffer
    import types
    import quantized_exact_order_amd as sage
    banner(f"buffers past 2^31 elements: B={B} H={H} N={N} D={D}")
    gen = torch.Generator(device="cuda").manual_seed(77)
    q, k, v = (torch.randn((B, N, H, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(3))
    cos, sin = workloads.rope_tables(N, R)
    shape = sage.Shape(B, N, H, H, D, R)
    bufs = sage.Buffers.allocate(shape, "cuda")
    args = (q, k, v, None, None, cos.cuda(), sin.cuda())
    sage.prep(shape, bufs, *args)
    sage.quant_qk(shape, bufs, *args)
    o = sage.attn_fwd(shape, bufs)
    torch.cuda.synchronize()
    assert q.numel() > 2 ** 31 and bufs.q8.numel() > 2 ** 31 and o.numel() > 2 ** 31
    one = torch.ones(D, dtype=torch.bfloat16)
    cfg = workloads.Config("slice", B=1, N=N, Hq=1, Hkv=1, D=D, rope_dim=R)
    sub = sage.Shape(1, N, 1, 1, D, R)
    for b, h in ((0, 0), (B // 2 - 1, H // 4 + 1), (B - 1, H - 1)):
        sl = lambda t: t[b:b + 1, :, h:h + 1].cpu()
        ref = oracle.prepare(workloads.Inputs(cfg, sl(q), sl(k), sl(v), one, one, cos, sin))
        got = dict(q8=bufs.q8[b:b + 1, h:h + 1, :N].cpu().numpy(),
                   q_scale=bufs.q_scale[b:b + 1, h:h + 1].cpu().numpy(),
                   k8=bufs.k8[b:b + 1, h:h + 1, :N].cpu().numpy(),
                   k_scale=bufs.k_scale[b:b + 1, h:h + 1].cpu().numpy(),
                   k_mean=bufs.k_mean[b:b + 1, h:h + 1].cpu().numpy(),
                   v8=sage.v8_logical(sub, types.SimpleNamespace(v8=bufs.v8[b:b + 1, h:h + 1])).cpu().numpy(),
                   v_scale=bufs.v_scale[b:b + 1, h:h + 1].cpu().numpy())
        assert_prep_bit_exact(ref, got, f"slice b={b} h={h}")
        rows = np.array([(0, 0, i) for i in (0, 1, 2047, 4095, N - 50, N - 1)], np.int32)
        o_ref = oracle.bf16_to_f32(oracle.attn_rows(ref, rows))
        o_gpu = np.stack([oracle.bf16_to_f32(bf16_bits(o[b, i, h])) for _, _, i in rows])
        compare_output(o_gpu, o_ref, f"slice b={b} h={h}")


@pytest.mark.timeout(600)
def test_long_sequence_k_mean_tree():
    # 1094 key tiles: the tree over tiles is padded to 2048 leaves, which the
    # K-mean reduction builds from 32-tile chunk subtrees
    inp = workloads.make_custom(1, 70001, 2, 2, 128, 96, seed=600)
    rng = np.random.default_rng(42)
    rows = _sample_rows(1, 2, 70001, 24, rng, tail=40)
    _full_check(inp, "N=70001", attn_rows=rows)


@pytest.mark.parametrize("name", ["tiny", "tail"])
def test_fp32_accumulation_is_closer_to_fp32_reading_than_to_fp16_partials(name):
    # the GPU's FP8 MFMA accumulates each tile's PV in FP32; the page's kernel
    # accumulates it in FP16 (emulated by the oracle): the GPU output must sit
    # nearer the oracle's FP32 reading
    inp = workloads.make_inputs(workloads.CONFIGS[name])
    banner(f"{name}: GPU vs oracle FP32 / FP16 PV partials")
    ref = oracle.prepare(inp)
    _, _, o = run_path(inp)
    g = oracle.bf16_to_f32(bf16_bits(o)).astype(np.float64)
    a = oracle.bf16_to_f32(oracle.attention(ref)).astype(np.float64)
    b = oracle.bf16_to_f32(oracle.attention(ref, pv_fp16=True)).astype(np.float64)
    da, db = np.abs(g - a), np.abs(g - b)
    print(f"[gpu] {name}: vs FP32 reading max-abs {da.max():.3g} differing {np.mean(g != a):.4f}; "
          f"vs FP16 partials max-abs {db.max():.3g} differing {np.mean(g != b):.4f}", flush=True)
    assert np.mean(g != a) < np.mean(g != b)
    assert 1.0 - oracle.cosine(g, a) < 1.0 - oracle.cosine(g, b)


def _pv16_cases():
    return ["tiny", "tail", "encoder", "gqa"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", _pv16_cases())
def test_within_tolerance_of_fp16_pv_partials(name):
    # the contract page accumulates each 64-key tile's PV in an FP16 fragment
    # before adding it to the FP32 output accumulator ("V And PV", two
    # accumulation levels); the GPU accumulates the tile in FP32.  The GPU
    # output must also meet the output bar (max-abs 2e-2, cosine 0.999)
    # against the oracle's emulation of that two-level form, overall and per
    # head.  GQA (N = 8192, 16 heads) is compared on sampled rows.
    cfg = workloads.CONFIGS[name]
    inp = workloads.make_inputs(cfg)
    banner(f"{name}: GPU vs oracle with FP16 PV partials")
    ref = oracle.prepare(inp)
    shape, _, o = run_path(inp)
    B, N, Hq, D = o.shape
    if name == "gqa":
        rows = _sample_rows(B, Hq, N, 24, np.random.default_rng(43), tail=8)
    else:
        rows = oracle.all_rows(B, Hq, N)
    o_ref = oracle.bf16_to_f32(oracle.attn_rows(ref, rows, pv_fp16=True))
    o_gpu = oracle.bf16_to_f32(bf16_bits(o))[rows[:, 0], rows[:, 2], rows[:, 1]]
    err, cos = compare_output(o_gpu, o_ref, f"{name} vs FP16 PV partials")
    print(f"[gpu] {name}: vs FP16 PV partials max-abs {err:.3g} cosine {cos:.6f}", flush=True)
    for h in range(Hq):
        sel = rows[:, 1] == h
        compare_output(o_gpu[sel], o_ref[sel], f"{name} head {h} vs FP16 PV partials")
