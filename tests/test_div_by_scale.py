"""The FP8 quantizers divide by the block scale through a reciprocal and one
FMA correction; tests/div_by_scale_check.c checks, over every bf16 block
maximum and every bf16 value, that this gives the e4m3 code of the correctly
rounded quotient (the arithmetic the oracle and the pages' recipe use)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_div_by_scale_exhaustive(tmp_path):
    exe = tmp_path / "check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "div_by_scale_check.c"), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "mismatches 0" in r.stdout
