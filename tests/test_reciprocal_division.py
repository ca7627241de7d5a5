"""The NVFP4 encoder divides each element of a group by the group's divisor
e through a correctly rounded reciprocal and one FMA correction (Markstein's
theorem on division).  The quantized codes must equal those of an IEEE
division, so this CPU test compiles tests/arith/reciprocal_division.c (plain
C, strict IEEE binary32 with FMA) and runs it over every finite bf16 input
for all E4M3 block scales and several tensor scales."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_division_gives_the_ieee_quotients_e2m1_code(tmp_path):
    exe = str(tmp_path / "reciprocal_division")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                    os.path.join(HERE, "arith", "reciprocal_division.c"), "-lm"], check=True)
    r = subprocess.run([exe, "8", "5"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "differing 0" in r.stdout
    checked = int(r.stdout.split("checked ")[1].split()[0])
    assert checked > 30_000_000
