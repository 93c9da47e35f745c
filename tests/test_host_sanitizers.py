"""The host half of libmagi_bca (mask builders, schedulers, argument
validation of every entry point) under AddressSanitizer and
UndefinedBehaviorSanitizer: a host-sanitized build of the library, loaded
with the sanitizer runtime preloaded, runs the whole host test file
(tests/test_plan.py).  Any sanitizer report aborts that run."""
import os
import subprocess
import sys

import pytest

from block_causal_attention_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    lib = B.build_host_sanitized(str(tmp_path / "libmagi_bca.so"))
    env = dict(os.environ)
    env.update(LD_PRELOAD=B.asan_runtime(), MAGI_BCA_LIBRARY=lib,
               # Python itself keeps memory until exit; leak reports are not about this library
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    check = ("import block_causal_attention_amd._lib as L; L.lib(); "
             f"assert L.LIB_PATH == {lib!r}, L.LIB_PATH; print('sanitized library loaded')")
    res = subprocess.run([sys.executable, "-c", check], cwd=ROOT, env=env, capture_output=True, text=True)
    assert res.returncode == 0 and "sanitized library loaded" in res.stdout, res.stdout + res.stderr
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_plan.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
