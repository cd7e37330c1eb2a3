"""The oracle's pins rerun under AddressSanitizer + UndefinedBehaviorSanitizer
(host only): the oracle is plain C, so out-of-bounds accesses, overflows or
a float -> int conversion of NaN would otherwise pass silently. The oracle
is rebuilt with the sanitizers (oracle/build.py, sanitize=True) and the pin
modules run in a child Python with gcc's ASan runtime preloaded; every
sanitizer report is fatal there.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PIN_MODULES = ["tests/test_oracle_decode.py", "tests/test_oracle_route_sort.py",
               "tests/test_oracle_forward_requant.py"]


@pytest.fixture(scope="module")
def san_env():
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    lib = ob.build(sanitize=True)
    rt = ob.asan_runtime()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("gcc's ASan runtime is not installed")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, MOE_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:allocator_may_return_null=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2",
               PYTHONDONTWRITEBYTECODE="1")
    return env


def test_oracle_pins_under_sanitizers(san_env):
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           *PIN_MODULES]
    r = subprocess.run(cmd, cwd=ROOT, env=san_env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail


def test_requant_out_of_domain_scales_defined_under_sanitizers(san_env):
    """e8m0 bytes 253-255 are outside the requant's domain (decoded values
    overflow bf16, or the scale is NaN): the oracle must still be defined
    there -- no float -> int conversion of NaN, no out-of-bounds access."""
    code = (
        "import numpy as np, oracle\n"
        "rng = np.random.default_rng(1)\n"
        "w = rng.integers(0, 256, size=(2, 4, 64), dtype=np.uint8)\n"
        "s = np.array([253, 254, 255, 127], dtype=np.uint8)[rng.integers(0, 4, size=(2, 4, 4))]\n"
        "s[0, 0, :] = [253, 254, 255, 255]\n"
        "q, qs = oracle.requant_int4g32(w, s)\n"
        "assert q.shape == w.shape and qs.shape == s.shape\n"
        "print('ok')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=san_env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout + r.stderr)[-4000:]
