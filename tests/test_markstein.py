"""The reciprocal-plus-correction quotient the block-FP8 and NVFP4 kernels use
for their fp32 divisions (x / S, b / (6g), x / eff) equals IEEE division in
the domain the kernels take it: divisors in [2^-60, 2^60], quotients up to
512 (test infrastructure: tests/markstein_check.c replays the kernels' fp32
operations on the host; gcc, SSE arithmetic, no flush to zero).

The default test sweeps a sample of the domain in about a second; the full
sweep (4.7e10 cases) is marked slow and runs with --runslow."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(tmp_path, mode, timeout):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "markstein_check"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-Wall", "-Werror", os.path.join(ROOT, "tests", "markstein_check.c"), "-lm",
                    "-o", str(exe)], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(max(1, min(16, os.cpu_count() or 1))))
    r = subprocess.run([str(exe), mode], capture_output=True, text=True, timeout=timeout, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert f"markstein check: ok ({mode})" in r.stdout, r.stdout
    return r.stdout


def test_markstein_quotient_equals_ieee_division_sampled(tmp_path):
    out = _run(tmp_path, "quick", 300)
    # the only differences allowed are same-sign quotients below 2^-30, and
    # the sweep reaches them (bf16 subnormals over the largest divisors)
    assert "equal-sign quotients below 2^-30" in out


@pytest.mark.slow
def test_markstein_quotient_equals_ieee_division_full(tmp_path):
    _run(tmp_path, "full", 3600)
