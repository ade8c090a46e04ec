"""Mutation check of the oracle's pins.

Each case below plants one plausible mistake in a copy of ``oracle/sage_oracle.c``
(a dropped term, a wrong sign, a wrong index or group size, another rounding
mode, a missing rotation), compiles the copy with the oracle's own gcc flags and
runs the oracle pin suite against it in a fresh process.  The pins must fail
for every case; an unmodified copy must pass.  The mistakes are planted on the
CPU, in the oracle only.

The reduction order of the K sequence-mean tree and the FMA in the exponent
argument are readings that the pins cannot fix: any order, fused or not, stays
within their FP32 bounds.  The GPU tests compare the K mean bit for bit.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PIN_FILES = ["tests/test_oracle_formats.py", "tests/test_oracle_prep.py", "tests/test_oracle_attn.py",
             "tests/test_oracle_segmented.py", "tests/test_oracle_decode.py", "tests/test_oracle_pv16.py",
             "tests/test_golden_boundary.py"]

# (name, pin file run first, exact text in sage_oracle.c, replacement)
MUTANTS = [
    # number formats
    ("bf16_ties_away", "formats", "u += 0x7fffu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    ("bf16_truncate", "formats", "u += 0x7fffu + ((u >> 16) & 1u);", "u += 0u;"),
    ("e4m3_overflow_to_nan", "formats", "if (a >= 448.0) return (uint8_t)(sign | 0x7e);",
     "if (a >= 448.0) return (uint8_t)(sign | 0x7f);"),
    ("e4m3_subnormal_floor", "formats", "double q = rint(a * 512.0);", "double q = floor(a * 512.0);"),
    ("e4m3_mantissa_floor", "formats", "double q = rint((2.0 * fr - 1.0) * 8.0);",
     "double q = floor((2.0 * fr - 1.0) * 8.0);"),
    ("e4m3_decode_bias", "formats", "else v = ldexp(1.0 + m / 8.0, e - 7);",
     "else v = ldexp(1.0 + m / 8.0, e - 8);"),
    ("i8_ties_away", "formats", "double r = rint((double)x);", "double r = round((double)x);"),
    ("i8_clamp_symmetric", "formats", "if (r < -128.0) r = -128.0;", "if (r < -127.0) r = -127.0;"),
    ("exp2_no_flush", "formats", "if (r < 0x1p-126f) r = 0.0f;", ""),
    ("score_scale_without_log2e", "formats", "* 1.4426950408889634073599246810019);", "* 1.0);"),
    ("f16_subnormal_quantum", "formats", "ldexp(1.0, -24)", "ldexp(1.0, -25)"),
    ("f16_fraction_bits", "formats", "ldexp(1.0, E - 10)", "ldexp(1.0, E - 9)"),
    # preparation
    ("rms_no_eps", "prep", "sqrtf(ss / (float)D + eps)", "sqrtf(ss / (float)D)"),
    ("rms_no_weight", "prep", "float n2 = n1 * oracle_bf16_to_f32(w[d]);", "float n2 = n1;"),
    ("rms_no_bf16_before_rope", "prep", "y[d] = oracle_bf16_to_f32(oracle_f32_to_bf16(n2));", "y[d] = n2;"),
    ("rope_sign", "prep", "float r0 = a * c - bb * s;", "float r0 = a * c + bb * s;"),
    ("rope_interleaved_pairs", "prep", "float a = y[i], bb = y[i + half];",
     "float a = y[2 * i], bb = y[2 * i + 1];"),
    ("k_mean_over_padded_count", "prep", "* D + d] = S / (float)N;", "* D + d] = S / (float)P;"),
    ("k_mean_64_leaf_floor", "prep", "int64_t P = 1;\n    while (P < N)", "int64_t P = 64;\n    while (P < N)"),
    ("wht_difference_sign", "prep", "u[j + span] = a - b;", "u[j + span] = b - a;"),
    ("wht_scale_1_over_d", "prep", "float s = (float)(1.0 / sqrt((double)D));",
     "float s = (float)(1.0 / (double)D);"),
    ("quant_scale_over_128", "prep", "float scale = amax / 127.0f;", "float scale = amax / 128.0f;"),
    ("quant_no_amax_floor", "prep", "float amax = (m > 1e-7f) ? m : 1e-7f;\n    float scale",
     "float amax = m;\n    float scale"),
    ("quant_q_skips_rotation", "prep", "oracle_bf16_to_f32(src[d]);\n                    if (hadamard)",
     "oracle_bf16_to_f32(src[d]);\n                    if (0)"),
    ("k_smoothing_sign", "prep", "oracle_bf16_to_f32(src[d]) - mu[d];", "oracle_bf16_to_f32(src[d]) + mu[d];"),
    ("v_multiplier_448", "prep", "float mul = 2.25f / amax;", "float mul = 448.0f / amax;"),
    ("v_no_amax_floor", "prep", "float amax = (m > 1e-7f) ? m : 1e-7f;\n                v_scale",
     "float amax = m;\n                v_scale"),
    # attention
    ("attn_q_group_64_rows", "attn", "nq + i / 32];", "nq + i / 64];"),
    ("attn_no_fp8_offset", "attn", "float M = mx - 8.807f;", "float M = mx;"),
    ("attn_no_rescale", "attn", "for (int e = 0; e < D; e++) RO[e] = RO[e] * alpha;", ""),
    ("attn_no_v_scale", "attn", "oracle_f32_to_bf16((RO[e] * rcp) * vs[e]);", "oracle_f32_to_bf16(RO[e] * rcp);"),
    ("attn_gqa_modulo", "attn", "    int hk = h / grp;\n", "    int hk = h % Hkv;\n"),
    ("attn_invalid_keys_in_denominator", "attn",
     "float p = (key < N) ? oracle_exp2(fmaf((float)S[j], f, -mn)) : 0.0f;",
     "float p = oracle_exp2(fmaf((float)S[j], f, -mn));"),
    ("attn_first_tile_scale_only", "attn", "float f = (qs * c) * ks[t];", "float f = (qs * c) * ks[0];"),
    ("attn_fp16_partial_not_rounded", "pv16", "frag = (double)oracle_f64_to_f16(acc);", "frag = acc;"),
    # segmented (split-KV) schedule
    ("seg_combine_d_unweighted", "segmented", "d = d + ds[s] * a;", "d = d + ds[s];"),
    ("seg_combine_ro_unweighted", "segmented", "RO[e] = RO[e] + ROs[(int64_t)s * D + e] * a;",
     "RO[e] = RO[e] + ROs[(int64_t)s * D + e];"),
    ("seg_overlapping_runs", "segmented", "int t0 = (int)((int64_t)s * nk / nseg), t1",
     "int t0 = (int)((int64_t)s * nk / nseg) - (s > 0), t1"),
    # decode cache
    ("kv_cache_skips_rotation", "decode", "oracle_wht(u, D);\n                int64_t r", "int64_t r"),
    ("decode_query_not_rotated", "decode", "oracle_wht(qr, D);", ""),
    ("decode_no_sqrt_d", "decode", "s[t] = dot * (double)kscale[base + t] / sqrt((double)D);",
     "s[t] = dot * (double)kscale[base + t];"),
    ("decode_no_row_scale", "decode", "s[t] = dot * (double)kscale[base + t] / sqrt((double)D);",
     "s[t] = dot / sqrt((double)D);"),
    ("decode_gqa_modulo", "decode", "const int hk = h / grp;", "const int hk = h % Hkv;"),
]


def _source() -> str:
    with open(os.path.join(ROOT, "oracle", "sage_oracle.c")) as f:
        return f.read()


def _run_pins(src_text: str, workdir: str, first: str) -> int:
    """Compile ``src_text`` and run the pin files against it; pytest's exit code."""
    os.makedirs(workdir, exist_ok=True)
    src = os.path.join(workdir, "sage_oracle.c")
    lib = os.path.join(workdir, "libsage_oracle.so")
    with open(src, "w") as f:
        f.write(src_text)
    oracle.compile_source(src, lib, werror=False)
    files = sorted(PIN_FILES, key=lambda p: first not in p)
    env = dict(os.environ, SAGE_ORACLE_LIB_OVERRIDE=lib, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *files]
    r = subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       timeout=600)
    with open(os.path.join(workdir, "pytest.log"), "wb") as f:
        f.write(r.stdout)
    return r.returncode


def test_mutant_texts_are_unique():
    src = _source()
    names = [m[0] for m in MUTANTS]
    assert len(set(names)) == len(names)
    for name, _, old, new in MUTANTS:
        assert src.count(old) == 1, name
        assert old != new, name


def test_unmodified_copy_passes_the_pins(tmp_path):
    assert _run_pins(_source(), str(tmp_path / "control"), "formats") == 0


@pytest.mark.slow
def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = _source()

    def one(m):
        name, first, old, new = m
        return name, _run_pins(src.replace(old, new), str(tmp_path / name), first)

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        codes = dict(ex.map(one, MUTANTS))
    # exit code 1: tests ran and at least one failed (2+ would be a collection
    # or usage error, which proves nothing about the pins)
    survivors = sorted(n for n, c in codes.items() if c == 0)
    broken = sorted(f"{n}:{c}" for n, c in codes.items() if c not in (0, 1))
    assert not survivors, f"pins did not catch: {survivors}"
    assert not broken, f"mutant runs did not complete: {broken}"
