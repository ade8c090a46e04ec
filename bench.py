#!/usr/bin/env python3
"""Throughput of the quantized attention forward on one MI355X.

One step = the whole hot path on one batch of synthetic input already resident
in HBM: sage_prep (RMSNorm + RoPE of K, K mean, V maxima), sage_quant_qk (INT8
Q/K, E4M3 V) and sage_attn_fwd (INT8 QK, online softmax, E4M3 PV).  The
workload is the canonical boundary of the contract page: B=1, N=37,810, 56
heads, D=128, Q/K/V as strided views of one interleaved BF16 QKV buffer.

Prints one JSON line:
  value      4*N^2*H*D / (step time)  [TFLOPS], whole path
  roofline   the attention kernel alone against the dense INT8/FP8 MFMA peak,
             timed with HIP events on the stream the kernel runs on
  prep       sage_prep + sage_quant_qk time and their algorithmic HBM rate
  cpu_baseline  the CPU oracle on a bounded sample of the same workload

--workload encoder instead times the short-encoder workload: 27 independent
seeded layers of N=729, H=16, D=128, each prep + quant + attention, run (a) as
27 back-to-back single-layer calls, (b) as the same calls captured once in a
HIP graph and replayed, and (c) as one call with the layers stacked along the
batch dimension (B = 27), which gives the attention launch 27x the
work-groups of one layer.  All three must produce identical bytes.

--ab OTHER_LIB.so compares the attention launch of another build of the
library (same ABI) with the in-tree one on the canonical inputs: paired,
interleaved launches (A B, B A, ...), each timed with HIP events; it prints
both medians and the median of the paired ratios B/A.

--tails times the attention launch on the canonical inputs at N = 37,810 and,
on the same views cut to N = 37,760 (295 x 128 rows: no partial query or key
tile), the tail-free launch; the difference is what the tails cost.

--workload gqa times the same step on the wide-head grouped-query workload
(B=1, N=8,192, 16 query heads over 4 KV heads, D=256, normalized
Walsh-Hadamard rotation of Q and K, RoPE on dims 0-191).

--workload decode times the decode-time INT8 K cache (per-head Hadamard
rotation, one FP32 scale per (head, token), BF16 V): single-query attention
of B=4 sequences x 32 query heads over 4 KV heads of D=256 and 32,768 cached
tokens (HBM-bound: the cache is read once per step), and the append of a
32,768-token prefill into the cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 5000.0      # MI355X dense INT8 / FP8 MFMA (5.0 POP/s)
PEAK_CLOCK_GHZ = 2.4           # the shader clock that peak is quoted at
METRIC = "attention TFLOPS (4·N²·H·D/t) at N=37810,H=56,D=128; % INT8/FP8 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_canonical_traffic.json")


def _attn_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("attn.hip", "device.h"):
        with open(os.path.join(ROOT, "quantized_exact_order_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic():
    """HBM bytes per attention launch from committed counter runs, or None when
    the kernel source changed since they were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != _attn_source_hash():
        return None
    return rec.get("bytes_per_launch")


def measured_clock(sage, shape, bufs, o, stream, launches: int = 2):
    """Shader clock the attention launch runs at: the stamped variant of the
    same launch (same kernel, same inputs), run right after the timed region;
    each work-group's first wave gives (shader cycles) / (constant-counter
    ticks) x the counter's rate over its lifetime.  Median and interquartile
    range over the work-groups of the last launch."""
    import torch
    hz = sage.wall_clock_hz()
    for _ in range(launches):
        st = sage.attn_fwd_stamped(shape, bufs, o, stream)
    torch.cuda.synchronize()
    s = st.cpu().numpy().astype("int64")
    dc, dw = s[:, 2] - s[:, 0], s[:, 3] - s[:, 1]
    ok = dw > 0
    ghz = sorted((dc[ok] / dw[ok] * hz / 1e9).tolist())
    n = len(ghz)
    return {"GHz": round(ghz[n // 2], 4), "iqr": [round(ghz[n // 4], 4), round(ghz[(3 * n) // 4], 4)],
            "note": (f"median over {n} work-groups of a stamped launch of the same kernel after the timed "
                     f"region (s_memtime cycles / s_memrealtime ticks x {hz / 1e6:.0f} MHz); the peak "
                     f"{PEAK_MFMA_TFLOPS:.0f} TFLOP/s assumes {PEAK_CLOCK_GHZ} GHz")}


def _cpu_model():
    """The host CPU's model name, or None where /proc/cpuinfo does not give it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, cfg, budget_s: float = 12.0, heads=(0, 27, 55)):
    """The oracle, as it stands, on a bounded sample: the full preparation, then
    attention rows of `heads` in batches until about budget_s seconds of
    attention work are done; the attention time is extrapolated to all N*H
    rows."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    p = oracle.prepare(inp)
    t_prep = time.perf_counter() - t0
    rng = np.random.default_rng(7)
    order = [(h, i) for h in heads for i in rng.permutation(cfg.N)]
    rng.shuffle(order)
    done, t_rows, batch = 0, 0.0, 256
    while t_rows < budget_s and done < len(order):
        rows = np.array([[0, h, i] for h, i in order[done:done + batch]], np.int32)
        t0 = time.perf_counter()
        oracle.attn_rows(p, rows)
        t_rows += time.perf_counter() - t0
        done += len(rows)
        batch = min(batch * 2, 16384)
    total_rows = cfg.B * cfg.Hq * cfg.N
    t_full = t_prep + t_rows * total_rows / done
    return {
        "value": round(cfg.attn_ops / t_full / 1e12, 6),
        "unit": "TFLOPS",
        "cores": oracle.num_threads(),
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": (f"full preparation ({t_prep:.1f} s) + attention of {done} query rows of heads "
                   f"{list(heads)} ({t_rows:.1f} s), attention time extrapolated to all "
                   f"{total_rows} rows"),
    }


def decode_cpu_baseline(q, k, v, T: int, grp: int, budget_s: float = 8.0):
    """The oracle's decode step, as it stands, on a bounded sample: the first
    sequence's first KV head (its grp query heads over all T cached tokens),
    repeated until about budget_s seconds; the rate is cache bytes read per
    second (INT8 K, FP32 K scales, BF16 V of that head), the bench's unit."""
    import numpy as np
    import torch
    import oracle
    ks = k[0:1, :, 0:1].cpu()
    vs = v[0:1, :, 0:1].permute(0, 2, 1, 3).cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    qs = q[0:1, 0:grp].cpu()
    k8, kscale = oracle.kv_quant(ks)
    D = k.shape[3]
    done, t = 0, 0.0
    while t < budget_s and done < 512:
        t0 = time.perf_counter()
        oracle.decode_attn(qs, k8, kscale, vs, T)
        t += time.perf_counter() - t0
        done += 1
    nbytes = T * (D + 4 + 2 * D)
    return {
        "value": round(nbytes * done / t / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": (f"{done} decode steps of one KV head ({grp} query heads, {T} cached tokens, "
                   f"{nbytes} cache bytes each) in {t:.1f} s; the INT8 K quantization of the cache is not timed"),
    }


def encoder_cpu_baseline(layers, cfg, budget_s: float = 8.0):
    """The oracle, as it stands, on whole layers (preparation and every query
    row) until about budget_s seconds; the rate holds for all the layers,
    which are the same work."""
    import oracle
    t, done = 0.0, 0
    for x in layers:
        t0 = time.perf_counter()
        oracle.attention(oracle.prepare(x))
        t += time.perf_counter() - t0
        done += 1
        if t >= budget_s:
            break
    return {
        "value": round(done * cfg.attn_ops / t / 1e12, 6),
        "unit": "TFLOPS",
        "cores": oracle.num_threads(),
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": f"{done} of the {len(layers)} layers, preparation and all {cfg.Hq * cfg.N} query rows each, in {t:.1f} s",
    }


def run_encoder(args):
    """27 independent short-sequence layers: per-layer calls, a HIP graph of
    them, and one stacked call.  One JSON line."""
    import torch
    import workloads
    import quantized_exact_order_amd as sage

    cfg = workloads.CONFIGS["encoder"]
    L, N, H, D = 27, cfg.N, cfg.Hq, cfg.D
    print(f"[bench] generating {L} encoder layers N={N} H={H} D={D}", file=sys.stderr, flush=True)
    layers = [workloads.make_inputs(cfg, layer=l) for l in range(L)]
    for x in layers[1:]:
        assert torch.equal(x.w_q, layers[0].w_q) and torch.equal(x.w_k, layers[0].w_k)
    dev = torch.device("cuda:0")
    q = torch.cat([x.q for x in layers]).to(dev)             # [L, N, H, D], layer = batch row
    k = torch.cat([x.k for x in layers]).to(dev)
    v = torch.cat([x.v for x in layers]).to(dev)
    w_q, w_k = layers[0].w_q.to(dev), layers[0].w_k.to(dev)
    cos, sin = layers[0].cos.to(dev).contiguous(), layers[0].sin.to(dev).contiguous()
    one = sage.Shape(1, N, H, H, D, cfg.rope_dim, cfg.hadamard, cfg.eps)
    stacked = sage.Shape(L, N, H, H, D, cfg.rope_dim, cfg.hadamard, cfg.eps)
    bufs1 = [sage.Buffers.allocate(one, dev) for _ in range(L)]
    o1 = torch.empty((L, N, H, D), dtype=torch.bfloat16, device=dev)
    bufsL = sage.Buffers.allocate(stacked, dev)
    oL = torch.empty((L, N, H, D), dtype=torch.bfloat16, device=dev)

    def per_layer():
        st = torch.cuda.current_stream()
        for l in range(L):
            a = (q[l:l + 1], k[l:l + 1], v[l:l + 1], w_q, w_k, cos, sin, st)
            sage.prep(one, bufs1[l], *a)
            sage.quant_qk(one, bufs1[l], *a)
            sage.attn_fwd(one, bufs1[l], o1[l:l + 1], st)

    # segmented (split-KV, non-exact) schedule: up to 8 segments of a short
    # sequence run as the waves of one work-group and combine in LDS; 12
    # takes the two-launch form (partials in HBM, then a combine launch)
    nk = (N + 63) // 64
    seg_counts = [n for n in (2, 3, 4, 6, 8, 12) if n <= nk]
    stacked_counts = [n for n in (2, 3, 4) if n <= nk]
    ws_seg = torch.empty(max([sage.attn_segmented_workspace(one, n) for n in seg_counts]
                             + [sage.attn_segmented_workspace(stacked, n) for n in stacked_counts]),
                         dtype=torch.uint8, device=dev)
    o_seg = torch.empty((L, N, H, D), dtype=torch.bfloat16, device=dev)

    def attn_only(nseg):
        st = torch.cuda.current_stream()
        for l in range(L):
            if nseg:
                sage.attn_fwd_segmented(one, bufs1[l], nseg, o_seg[l:l + 1], ws_seg, st)
            else:
                sage.attn_fwd(one, bufs1[l], o1[l:l + 1], st)

    def stacked_segmented(nseg):
        sage.attn_fwd_segmented(stacked, bufsL, nseg, o_seg, ws_seg, torch.cuda.current_stream())

    attn_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def batched(ev=False):
        st = torch.cuda.current_stream()
        a = (q, k, v, w_q, w_k, cos, sin, st)
        sage.prep(stacked, bufsL, *a)
        sage.quant_qk(stacked, bufsL, *a)
        if ev:
            attn_ev[0].record(st)
        sage.attn_fwd(stacked, bufsL, oL, st)
        if ev:
            attn_ev[1].record(st)

    # graph of the per-layer sequence (captured after an eager warmup)
    per_layer()
    torch.cuda.synchronize()
    ref = o1.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        per_layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        per_layer()
    torch.cuda.synchronize()

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = max(args.steps, 1)
    print(f"[bench] timing {reps} runs of each mode", file=sys.stderr, flush=True)
    t_layers = timed(per_layer, reps)
    o1.zero_()
    t_graph = timed(graph.replay, reps)
    graph_ok = bool(torch.equal(o1.view(torch.int16), ref.view(torch.int16)))
    t_batched = timed(batched, reps)
    batched_ok = bool(torch.equal(oL.view(torch.int16), ref.view(torch.int16)))
    attn_ms = []
    for _ in range(reps):
        batched(ev=True)
        torch.cuda.synchronize()
        attn_ms.append(attn_ev[0].elapsed_time(attn_ev[1]))
    attn_avg = sum(attn_ms) / len(attn_ms)
    if not (graph_ok and batched_ok):
        print("[bench] encoder modes disagree", file=sys.stderr, flush=True)
        sys.exit(1)
    t_attn = {"exact": timed(lambda: attn_only(0), reps)}
    seg_err = {}
    for n in seg_counts:
        t_attn[f"nseg={n}"] = timed(lambda: attn_only(n), reps)
        seg_err[f"nseg={n}"] = float((o_seg.float() - ref.float()).abs().max())
    t_stacked_seg, stacked_seg_err = {}, {}
    for n in stacked_counts:
        t_stacked_seg[f"nseg={n}"] = timed(lambda: stacked_segmented(n), reps)
        stacked_seg_err[f"nseg={n}"] = float((o_seg.float() - ref.float()).abs().max())
    ops = L * 4 * N * N * H * D
    best = min(t_layers, t_graph, t_batched)
    result = {
        "metric": "encoder attention TFLOPS (27 layers x 4*N^2*H*D / t) at N=729,H=16,D=128",
        "value": round(ops / (best * 1e-3) / 1e12, 3),
        "unit": "TFLOPS",
        "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": round(best, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8+e4m3", "data": "synthetic",
        "config": {"workload": "short encoder: 27 independent seeded layers, B=1 N=729 H=16 D=128 each, "
                               "prep + quant + attention per layer",
                   "layers": L, "N": N, "H": H, "D": D},
        "modes_ms_per_27_layers": {"per_layer_calls": round(t_layers, 4),
                                   "per_layer_calls_hip_graph": round(t_graph, 4),
                                   "stacked_batch_27": round(t_batched, 4)},
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_ilv_kernel<128, false>, the 27 layers stacked (B = 27)",
            "achieved": round(ops / (attn_avg * 1e-3) / 1e12, 3),
            "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ops / (attn_avg * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
            "traffic": None,
            "avg_launch_ms": round(attn_avg, 4),
            "ops_per_launch": ops,
        },
        "stacked_attention_launch_ms": round(attn_avg, 4),
        "outputs_identical_across_modes": True,
        "segmented_non_exact": {
            "attention_only_ms_per_27_layers": {k: round(t, 4) for k, t in t_attn.items()},
            "max_abs_vs_exact": seg_err,
            "stacked_27_attention_ms": {k: round(t, 4) for k, t in t_stacked_seg.items()},
            "stacked_max_abs_vs_exact": stacked_seg_err,
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle, whole layers)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = encoder_cpu_baseline(layers, cfg)
    print(json.dumps(result), flush=True)


def run_decode(args):
    """Decode step over the INT8 K cache and a prefill-sized append.  One JSON line."""
    import torch
    import quantized_exact_order_amd as sage

    B, Hq, Hkv, D, T = 4, 32, 4, 256, 32768
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(7)
    print(f"[bench] decode cache B={B} Hq={Hq} Hkv={Hkv} D={D} T={T}", file=sys.stderr, flush=True)
    kvbuf = torch.randn((B, T, 2 * Hkv * D), generator=g, device=dev).to(torch.bfloat16)
    k = kvbuf[:, :, :Hkv * D].view(B, T, Hkv, D)
    v = kvbuf[:, :, Hkv * D:].view(B, T, Hkv, D)
    q = torch.randn((B, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    cache = sage.KvCache.allocate(B, Hkv, T, dev)
    ws = torch.empty(sage.decode_workspace(cache, Hq, T), dtype=torch.uint8, device=dev)
    _calibration_copy(args, dev)
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)

    def timed(fn, reps):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def per_launch(fn, reps):
        # one event pair per call: median, min and interquartile range in ms
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, c in ev:
            a.record()
            fn()
            c.record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(c) for a, c in ev)
        return {"median_ms": round(t[len(t) // 2], 5), "min_ms": round(t[0], 5),
                "iqr_ms": [round(t[len(t) // 4], 5), round(t[(3 * len(t)) // 4], 5)]}

    reps = max(args.steps, 1) * 10
    t_append = timed(lambda: sage.kv_append(cache, k, v, 0), max(args.steps, 1))
    t_decode = timed(lambda: sage.decode_attn(cache, q, T, o, ws), reps)
    dist = per_launch(lambda: sage.decode_attn(cache, q, T, o, ws), reps)
    cache_bytes = B * Hkv * T * (D + 4 + 2 * D)            # k8 + k_scale + BF16 V, read once
    step_bytes = cache_bytes + 2 * B * Hq * D * 2
    append_bytes = B * T * Hkv * D * 2 * 2 + cache_bytes   # read K, V BF16; write the cache
    gbps = step_bytes / (t_decode * 1e-3) / 1e9
    # the same step over a cache with rotated INT8 V (one scale per head and token)
    cache8 = sage.KvCache.allocate(B, Hkv, T, dev, int8_v=True)
    t_append8 = timed(lambda: sage.kv_append(cache8, k, v, 0), max(args.steps, 1))
    t_decode8 = timed(lambda: sage.decode_attn(cache8, q, T, o, ws), reps)
    dist8 = per_launch(lambda: sage.decode_attn(cache8, q, T, o, ws), reps)
    step_bytes8 = B * Hkv * T * (D + 4 + D + 4) + 2 * B * Hq * D * 2
    del cache8
    result = {
        "metric": "decode attention over the INT8 K cache: HBM GB/s (cache bytes / step time)",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": reps, "warmup": max(args.warmup, 1),
        "ms_per_step": round(t_decode, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8 K (i8 MFMA) + bf16 V (bf16 MFMA), fp32 accumulation", "data": "synthetic",
        "config": {"workload": "decode: B=4 sequences, 32 query heads over 4 KV heads, D=256, "
                               "32,768 cached tokens, INT8 K (Hadamard-rotated, one scale per head and "
                               "token) + BF16 V", "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "T": T},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbps / 8000.0, 4), "bytes_per_step": step_bytes,
                     "kernels": "decode_chunk_kernel + decode_combine_kernel"},
        "decode_steps_per_s": round(1e3 / t_decode, 1),
        "step_ms_per_launch": dist,
        "append": {"tokens": B * T, "ms": round(t_append, 4),
                   "GB_per_s": round(append_bytes / (t_append * 1e-3) / 1e9, 1)},
        "int8_v": {"ms_per_step": round(t_decode8, 5), "bytes_per_step": step_bytes8,
                   "GB_per_s": round(step_bytes8 / (t_decode8 * 1e-3) / 1e9, 1),
                   "decode_steps_per_s": round(1e3 / t_decode8, 1), "append_ms": round(t_append8, 4),
                   "step_ms_per_launch": dist8},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle decode)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = decode_cpu_baseline(q, k, v, T, Hq // Hkv)
    print(json.dumps(result), flush=True)


def _calibration_copy(args, dev):
    """A plain device copy of known size (reads and writes calib_copy_mib MiB
    once), to scale the HBM byte counters of a profiled run."""
    if args.calib_copy_mib:
        import torch
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def run_tails(args):
    """Attention launch time at the canonical N and at the largest tail-free N
    below it (a multiple of 128 query rows and 64 keys): same inputs, paired
    and interleaved launches in one run."""
    import statistics
    import torch
    import workloads
    import quantized_exact_order_amd as sage

    cfg = workloads.CONFIGS["canonical"]
    inp = workloads.make_inputs(cfg)
    dev = torch.device("cuda:0")
    buf = inp.qkv.to(dev)
    Hq, Hkv, D, B, N = cfg.Hq, cfg.Hkv, cfg.D, cfg.B, cfg.N
    w_q, w_k = inp.w_q.to(dev), inp.w_k.to(dev)
    cos, sin = inp.cos.to(dev).contiguous(), inp.sin.to(dev).contiguous()
    n_free = (N // 128) * 128
    stream = torch.cuda.current_stream()
    runs = []
    for n in (N, n_free):
        q = buf[:, :n, 0:Hq * D].view(B, n, Hq, D)
        k = buf[:, :n, Hq * D:(Hq + Hkv) * D].view(B, n, Hkv, D)
        v = buf[:, :n, (Hq + Hkv) * D:].view(B, n, Hkv, D)
        shape = sage.Shape(B, n, Hq, Hkv, D, cfg.rope_dim, cfg.hadamard, cfg.eps)
        bufs = sage.Buffers.allocate(shape, dev)
        c, s_ = cos[:n].contiguous(), sin[:n].contiguous()          # RoPE rows of positions 0..n-1
        sage.prep(shape, bufs, q, k, v, w_q, w_k, c, s_)
        sage.quant_qk(shape, bufs, q, k, v, w_q, w_k, c, s_)
        o = torch.empty((B, n, Hq, D), dtype=torch.bfloat16, device=dev)
        runs.append((shape, bufs, o))
    for _ in range(max(args.warmup, 1)):
        for shape, bufs, o in runs:
            sage.attn_fwd(shape, bufs, o, stream)
    torch.cuda.synchronize()
    times = [[], []]
    for i in range(args.steps):
        order = (0, 1) if i % 2 == 0 else (1, 0)
        evs = []
        for which in order:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            shape, bufs, o = runs[which]
            e0.record(stream)
            sage.attn_fwd(shape, bufs, o, stream)
            e1.record(stream)
            evs.append((which, e0, e1))
        torch.cuda.synchronize()
        for which, e0, e1 in evs:
            times[which].append(e0.elapsed_time(e1))
    t_full, t_free = statistics.median(times[0]), statistics.median(times[1])
    diffs = [a - b for a, b in zip(times[0], times[1])]
    print(json.dumps({
        "tails": {"N": N, "median_launch_ms": round(t_full, 4),
                  "N_tail_free": n_free, "median_launch_ms_tail_free": round(t_free, 4),
                  "median_paired_extra_ms": round(statistics.median(diffs), 4),
                  "extra_work_fraction": round((N * N - n_free * n_free) / (n_free * n_free), 5),
                  "pairs": args.steps,
                  "note": "the extra time covers the 50-row query tail, the 50-key tail tile and the 0.26% more "
                          "query-key pairs at the canonical N"},
        "config": {"workload": "canonical attention launch, B=1 H=56 D=128, N=37810 against N=37760"}}),
        flush=True)


def run_ab(args):
    """Paired, interleaved A/B timing of sage_attn_fwd: the in-tree library (A)
    against another build of the same ABI (B), on the canonical inputs."""
    import ctypes
    import statistics
    import torch
    import workloads
    import quantized_exact_order_amd as sage

    cfg = workloads.CONFIGS["canonical"]
    inp = workloads.make_inputs(cfg)
    dev = torch.device("cuda:0")
    buf = inp.qkv.to(dev)
    Hq, Hkv, D, B, N = cfg.Hq, cfg.Hkv, cfg.D, cfg.B, cfg.N
    q = buf[:, :, 0:Hq * D].view(B, N, Hq, D)
    k = buf[:, :, Hq * D:(Hq + Hkv) * D].view(B, N, Hkv, D)
    v = buf[:, :, (Hq + Hkv) * D:].view(B, N, Hkv, D)
    w_q, w_k = inp.w_q.to(dev), inp.w_k.to(dev)
    cos, sin = inp.cos.to(dev).contiguous(), inp.sin.to(dev).contiguous()
    shape = sage.Shape(B, N, Hq, Hkv, D, cfg.rope_dim, cfg.hadamard, cfg.eps)
    bufs = sage.Buffers.allocate(shape, dev)
    sage.prep(shape, bufs, q, k, v, w_q, w_k, cos, sin)
    sage.quant_qk(shape, bufs, q, k, v, w_q, w_k, cos, sin)

    other = ctypes.CDLL(os.path.abspath(args.ab))
    other.sage_attn_fwd.argtypes = sage.lib.sage_attn_fwd.argtypes
    other.sage_attn_fwd.restype = ctypes.c_int32
    o_a = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device=dev)
    o_b = torch.empty_like(o_a)
    stream = torch.cuda.current_stream()
    sb, sn, sh, _ = o_b.stride()

    def launch(which):
        if which == 0:
            sage.attn_fwd(shape, bufs, o_a, stream)
        else:
            sage.check(other.sage_attn_fwd(ctypes.byref(shape.c()), ctypes.byref(bufs.c()), o_b.data_ptr(),
                                           sb, sn, sh, ctypes.c_void_p(stream.cuda_stream)), "B sage_attn_fwd")

    for _ in range(max(args.warmup, 1)):
        launch(0)
        launch(1)
    torch.cuda.synchronize()
    times = [[], []]
    for i in range(args.pairs):
        order = (0, 1) if i % 2 == 0 else (1, 0)
        evs = []
        for which in order:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch(which)
            e1.record(stream)
            evs.append((which, e0, e1))
        torch.cuda.synchronize()
        for which, e0, e1 in evs:
            times[which].append(e0.elapsed_time(e1))
    ratios = [tb / ta for ta, tb in zip(times[0], times[1])]
    print(json.dumps({
        "ab": {"A": sage.LIB_PATH, "B": os.path.abspath(args.ab), "pairs": args.pairs,
               "median_ms_A": round(statistics.median(times[0]), 4),
               "median_ms_B": round(statistics.median(times[1]), 4),
               "median_ratio_B_over_A": round(statistics.median(ratios), 4),
               "identical_output": bool(torch.equal(o_a.view(torch.int16), o_b.view(torch.int16)))},
        "config": {"workload": "canonical attention launch, B=1 N=37810 H=56 D=128"}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (HBM counter calibration)")
    ap.add_argument("--workload", choices=("canonical", "gqa", "encoder", "decode"), default="canonical")
    ap.add_argument("--ab", metavar="OTHER_LIB", default=None,
                    help="paired interleaved A/B of sage_attn_fwd against another build of the library")
    ap.add_argument("--pairs", type=int, default=10, help="A/B pairs (with --ab)")
    ap.add_argument("--tails", action="store_true",
                    help="attention launch at the canonical N against the largest tail-free N below it")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (got --gpus {args.gpus}); the path "
              "shards by head with no exchange, so one GPU's throughput is the measured figure.",
              file=sys.stderr)
        sys.exit(2)
    if args.ab:
        return run_ab(args)
    if args.tails:
        return run_tails(args)
    if args.workload == "encoder":
        return run_encoder(args)
    if args.workload == "decode":
        return run_decode(args)
    if args.workload == "gqa":
        return run_prefill(args, "gqa")

    return run_prefill(args, "canonical")


def run_prefill(args, name):
    """One step = sage_prep + sage_quant_qk + sage_attn_fwd on the named
    workload; one JSON line with the attention roofline and the CPU oracle."""
    import torch
    import workloads
    import quantized_exact_order_amd as sage

    cfg = workloads.CONFIGS[name]
    print(f"[bench] generating {name} inputs N={cfg.N} Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D}", file=sys.stderr,
          flush=True)
    inp = workloads.make_inputs(cfg)
    dev = torch.device("cuda:0")
    Hq, Hkv, D, B, N = cfg.Hq, cfg.Hkv, cfg.D, cfg.B, cfg.N
    if inp.qkv is not None:
        buf = inp.qkv.to(dev)
        q = buf[:, :, 0:Hq * D].view(B, N, Hq, D)
        k = buf[:, :, Hq * D:(Hq + Hkv) * D].view(B, N, Hkv, D)
        v = buf[:, :, (Hq + Hkv) * D:].view(B, N, Hkv, D)
    else:
        q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    w_q, w_k = inp.w_q.to(dev), inp.w_k.to(dev)
    cos, sin = inp.cos.to(dev).contiguous(), inp.sin.to(dev).contiguous()
    shape = sage.Shape(B, N, Hq, Hkv, D, cfg.rope_dim, cfg.hadamard, cfg.eps)
    bufs = sage.Buffers.allocate(shape, dev)
    o = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[2].record(stream)
        sage.prep(shape, bufs, q, k, v, w_q, w_k, cos, sin, stream)
        sage.quant_qk(shape, bufs, q, k, v, w_q, w_k, cos, sin, stream)
        if ev is not None:
            ev[0].record(stream)
        sage.attn_fwd(shape, bufs, o, stream)
        if ev is not None:
            ev[1].record(stream)

    _calibration_copy(args, dev)
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attn_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    attn_avg_ms = sum(attn_ms) / len(attn_ms)
    prep_ms = sorted(e[2].elapsed_time(e[0]) for e in evs)
    prep_avg_ms = sum(prep_ms) / len(prep_ms)
    z = sage.buffer_sizes(shape)
    # algorithmic prep bytes: read Q, K, V once (BF16), write q8, k8, v8 and the scales
    prep_bytes = (2 * B * N * (Hq + 2 * Hkv) * D + B * N * (Hq + 2 * Hkv) * D
                  + z.q_scale + z.k_scale + z.k_mean + z.v_scale)
    ms_step = elapsed * 1e3 / args.steps

    ops = cfg.attn_ops
    achieved = ops / (attn_avg_ms * 1e-3) / 1e12
    clock = measured_clock(sage, shape, bufs, o, stream)
    kernel = "attn_ilv_kernel<128, false>" if D == 128 else "attn_pair256_kernel<false>"
    if name == "canonical":
        metric = METRIC
        workload = ("canonical: B=1 N=37810 H=56 D=128, Q/K/V strided views of one BF16 [N,21504] QKV buffer, "
                    "RMSNorm+RoPE(0-95), K smoothing, INT8 QK, E4M3 PV, non-causal")
    else:
        metric = f"attention TFLOPS (4·N²·Hq·D/t) at N={N},Hq={Hq},Hkv={Hkv},D={D}; % INT8/FP8 MFMA peak"
        workload = (f"{name}: B={B} N={N} Hq={Hq} Hkv={Hkv} D={D}, RMSNorm+RoPE(0-{cfg.rope_dim - 1})"
                    + (", normalized Walsh-Hadamard rotation of Q and K" if cfg.hadamard else "")
                    + ", K smoothing, INT8 QK, E4M3 PV, non-causal")
    result = {
        "metric": metric,
        "value": round(ops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+e4m3",
        "data": "synthetic",
        "config": {"workload": workload, "B": B, "N": N, "H": Hq, "Hkv": Hkv, "D": D,
                   "step": "sage_prep+sage_quant_qk+sage_attn_fwd"},
        "roofline": {
            "bound": "mfma",
            "kernel": kernel,
            "achieved": round(achieved, 3),
            "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
            "traffic": _traffic() if name == "canonical" else None,
            "avg_launch_ms": round(attn_avg_ms, 4),
            "median_launch_ms": round(attn_ms[len(attn_ms) // 2], 4),
            "ops_per_launch": ops,
            "iqr_launch_ms": [round(attn_ms[len(attn_ms) // 4], 4), round(attn_ms[(3 * len(attn_ms)) // 4], 4)],
            "min_launch_ms": round(attn_ms[0], 4),
            "clock_GHz": clock["GHz"],
            "clock_GHz_iqr": clock["iqr"],
            "peak_at_measured_clock": round(PEAK_MFMA_TFLOPS * clock["GHz"] / PEAK_CLOCK_GHZ, 1),
            "frac_at_measured_clock": round(achieved / (PEAK_MFMA_TFLOPS * clock["GHz"] / PEAK_CLOCK_GHZ), 4),
            "clock_note": clock["note"],
        },
        "prep": {
            "kernels": "sage_prep + sage_quant_qk (3 launches: prep_stats, prep_reduce, quant)",
            "avg_ms": round(prep_avg_ms, 4),
            "algorithmic_bytes": int(prep_bytes),
            "GB_per_s": round(prep_bytes / (prep_avg_ms * 1e-3) / 1e9, 1),
            "hbm_peak_GB_per_s": 8000.0,
        },
    }
    # co-bounds of the attention launch, beside the MFMA roofline:
    #  - one exp2 per score; the issue floor takes v_exp_f32 at the measured 9.0
    #    SIMD cycles per wave64 instruction on all 1024 SIMDs at 2.4 GHz;
    #  - every 128-row query tile streams its KV head's INT8 K and E4M3 V from
    #    L2/MALL once (padded key rows);
    #  - HBM: q8, k8, v8 and their scales read once, O written once.
    exps = B * Hq * N * N
    exp_floor_ms = exps / (1024 * (64 / 9.0) * 2.4e9) * 1e3
    restream = 2 * z.k_rows * D * ((N + 127) // 128) * Hq * B
    hbm = z.q8 + z.k8 + z.v8 + z.q_scale + z.k_scale + z.v_scale + 2 * B * N * Hq * D
    t = attn_avg_ms * 1e-3
    result["co_bounds"] = {
        "exp2": {"count": exps, "per_s": round(exps / t, 1), "issue_floor_ms": round(exp_floor_ms, 3),
                 "floor_frac_of_launch": round(exp_floor_ms / attn_avg_ms, 4)},
        "kv_restream_l2": {"bytes": int(restream), "GB_per_s": round(restream / t / 1e9, 1)},
        "hbm": {"algorithmic_bytes": int(hbm), "GB_per_s": round(hbm / t / 1e9, 1),
                "frac": round(hbm / t / 1e9 / 8000.0, 4)},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        heads = (0, 27, 55) if name == "canonical" else (0, Hq // 2 - 1, Hq - 1)
        result["cpu_baseline"] = cpu_baseline(inp, cfg, heads=heads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
