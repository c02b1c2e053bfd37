"""The FP8 quantisers' division (x * RN(1/s) with one FMA correction) against the correctly
rounded fp32 division, over every pair of bf16 inputs that can reach it (host C, gcc)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_one_fma_division_matches_correct_rounding(tmp_path):
    exe = tmp_path / "exhaustive"
    # -ffp-contract=off: the products and the FMAs stay exactly as written
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", os.path.join(HERE, "markstein", "exhaustive.c"), "-o", str(exe),
                    "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("0 of ")
