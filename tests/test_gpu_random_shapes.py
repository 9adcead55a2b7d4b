"""Seeded random shapes through the plain entry points of all three routes (each shape lands in
whichever kernel and configuration the library selects for it), full C against the oracle."""
import numpy as np
import pytest

import workload
from gpu_util import parity, run_bs, run_mx, run_pt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb():
    import fp8_block_scaled_e4m3_amd as fb
    return fb


def _shapes(route, n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        if route == "mx":
            M = 64 * int(rng.integers(1, 9))
            N = 64 * int(rng.integers(1, 17))
            K = 128 * int(rng.integers(2, 13))
        else:
            M = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 700))]))
            N = (128 if route == "bs" else 64) * int(rng.integers(1, 13))
            K = 128 * int(rng.integers(1, 17))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _shapes("bs", 12, 2024))
def test_random_bs(fb, oracle, M, N, K):
    x = workload.bs_inputs(M, N, K, M + N + K)
    _, ref = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    parity(run_bs(fb, x), ref, f"bs {M}x{N}x{K} ({fb.fp8bs_select_config(fb.ROUTE_BS, M, N, K)})")


@pytest.mark.parametrize("M,N,K", _shapes("pt", 8, 2025))
def test_random_pt(fb, oracle, M, N, K):
    z = workload.pt_inputs(M, N, K, M * 3 + N + K)
    _, ref = oracle.pt_gemm(z.A, z.a_scale, z.B, z.b_scale)
    parity(run_pt(fb, z), ref, f"pt {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", _shapes("mx", 8, 2026))
def test_random_mx(fb, oracle, M, N, K):
    y = workload.mx_inputs(M, N, K, M + 5 * N + K)
    _, ref = oracle.mx_gemm(y.A, y.a_e8m0, y.B, y.b_e8m0)
    parity(run_mx(fb, y), ref, f"mx {M}x{N}x{K}")
