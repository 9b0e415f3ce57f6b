"""The quantiser kernels replace the per-element division x / scale by a
reciprocal and one Markstein correction step.  This runs the exhaustive CPU
replay of those single-precision steps (quant_division_exhaustive.c) over
every finite fp16 block maximum and every fp16 |x| <= maximum, both signs
(about 1.0e9 pairs), and requires int8 results identical to the definition
clamp(rint_half_even(fl32(x / fl32(a / 127))), -127, 127).  CPU only."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _compile(tmp_path, src, omp=True):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / (os.path.basename(src) + ".bin"))
    base = [gcc, "-O2", "-fno-fast-math", "-ffp-contract=off", src, "-o", exe, "-lm"]
    if omp and subprocess.run(base[:1] + ["-fopenmp"] + base[1:], capture_output=True).returncode == 0:
        return exe
    r = subprocess.run(base, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_quantiser_division_steps_exhaustive(tmp_path):
    exe = _compile(tmp_path, os.path.join(HERE, "quant_division_exhaustive.c"))
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(min(8, os.cpu_count() or 1)))
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout.strip())
    fields = dict(kv.split("=") for kv in r.stdout.split())
    assert int(fields["pairs"]) == 1007713278          # 2 * sum over a of (#fp16 |x| <= a), a = 1 .. 0x7BFF
    assert int(fields["byte_mismatch"]) == 0
    assert int(fields["quotient_mismatch"]) == 0
    assert int(fields["over_range"]) == 0
    assert r.returncode == 0
