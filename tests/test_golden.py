"""The oracle reproduces its stored regression fixtures (tests/golden, written by
tests/golden/make_golden.py from the oracle alone)."""
import hashlib
import os

import numpy as np
import pytest

import workload

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read(name):
    lines = [ln for ln in open(os.path.join(HERE, name)) if not ln.startswith("#")]
    digest = lines[0].split()[1]
    picks = [ln.split() for ln in lines[1:]]
    return digest, picks


@pytest.mark.parametrize("route", ["bs", "mx", "pt"])
def test_golden_tiny(oracle, route):
    if route == "bs":
        x = workload.bs_inputs(128, 256, 512, 0)
        acc, bits = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    elif route == "pt":
        z = workload.pt_inputs(128, 256, 512, 0)
        acc, bits = oracle.pt_gemm(z.A, z.a_scale, z.B, z.b_scale)
    else:
        y = workload.mx_inputs(128, 256, 512, 0)
        acc, bits = oracle.mx_gemm(y.A, y.a_e8m0, y.B, y.b_e8m0)
    digest, picks = _read(f"tiny_{route}_seed0.txt")
    assert hashlib.sha256(np.ascontiguousarray(bits).tobytes()).hexdigest() == digest
    for m, n, b, a in picks:
        assert int(bits[int(m), int(n)]) == int(b, 16)
        assert float(acc[int(m), int(n)]) == float(a)
