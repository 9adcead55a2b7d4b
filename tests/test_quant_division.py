"""The route-BS quantiser's quotient method (csrc/quant.hip) checked on the host against IEEE
division: every bf16 (value, group maximum) pair whose scale is at least 2^-90, and random fp32
pairs. The kernel takes the fp64 product path for smaller scales."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_corrected_quotient_is_correctly_rounded():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "quant_division_check")
        # no contraction: every product and fused multiply-add is the one written
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "quant_division_check.c"),
                        "-lm"], check=True)
        p = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(p.stdout)
    assert p.returncode == 0, p.stdout + p.stderr
