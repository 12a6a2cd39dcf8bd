"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize_oracle.c drives every oracle entry point on ragged, tiny and
empty shapes with inputs holding NaN, Inf, zeros, subnormals and extremes,
every output buffer allocated to its exact documented size.  Built here with
gcc -fsanitize=address,undefined and run as its own process, any
out-of-bounds access, leak or undefined arithmetic in the oracle fails it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "sanitize_oracle"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-ffp-contract=off", "-fno-fast-math",
           os.path.join(ROOT, "oracle", "mxq_oracle.c"),
           os.path.join(ROOT, "tests", "sanitize_oracle.c"), "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "sanitized oracle run: ok" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
