"""The oracle's C code (oracle/sage_oracle.c) built with AddressSanitizer and
UndefinedBehaviorSanitizer (float-to-int overflow included) and driven through
every entry point on small and edge shapes by tests/sanitize_oracle.c: no
out-of-bounds access, no undefined behaviour, no leak.  Host only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "sanitize_oracle")
    build = [gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
             os.path.join(ROOT, "tests", "sanitize_oracle.c"), os.path.join(ROOT, "oracle", "sage_oracle.c"),
             "-lm", "-o", exe]
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    assert "sanitize_oracle ok" in r.stdout
