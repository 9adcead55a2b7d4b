"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Small shapes are compared in full, including ragged M tails and several tiles in each
direction; the five bench workloads are compared on seeded samples of whole rows and whole
columns (the oracle computes each element independently, so a sample is exact)."""
import numpy as np
import pytest

import workload
from gpu_util import parity, run_bs, run_mx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb():
    import fp8_block_scaled_e4m3_amd as fb
    return fb


BS_SMALL = [(128, 256, 512), (1, 128, 128), (63, 256, 384), (65, 384, 256), (200, 512, 640),
            (257, 128, 1024), (512, 896, 128)]


@pytest.mark.parametrize("M,N,K", BS_SMALL)
@pytest.mark.parametrize("seed", [0, 1])
def test_bs_small_full(fb, oracle, M, N, K, seed):
    x = workload.bs_inputs(M, N, K, seed)
    got = run_bs(fb, x)
    _, ref = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    parity(got, ref, f"bs {M}x{N}x{K} seed {seed}")


MX_SMALL = [(128, 256, 512), (64, 64, 256), (192, 320, 384), (256, 128, 1280)]


@pytest.mark.parametrize("M,N,K", MX_SMALL)
@pytest.mark.parametrize("seed", [0, 1])
def test_mx_small_full(fb, oracle, M, N, K, seed):
    y = workload.mx_inputs(M, N, K, seed)
    got = run_mx(fb, y)
    _, ref = oracle.mx_gemm(y.A, y.a_e8m0, y.B, y.b_e8m0)
    parity(got, ref, f"mx {M}x{N}x{K} seed {seed}")


def _sampled(M, N, seed, n=48):
    return workload.sample_indices(M, n, seed), workload.sample_indices(N, n, seed + 1)


@pytest.mark.parametrize("name", ["narrow_n", "k_light", "wide_n"])
def test_bs_workload_sampled(fb, oracle, name):
    cfg = workload.CONFIGS[name]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    x = workload.bs_inputs(M, N, K, 0)
    got = run_bs(fb, x)
    rows, cols = _sampled(M, N, 0)
    _, ref_rows = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale, rows=rows)
    parity(got[rows], ref_rows, f"{name} rows")
    _, ref_cols = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale, cols=cols)
    parity(got[:, cols], ref_cols, f"{name} cols")


def test_mx_workload_sampled(fb, oracle):
    cfg = workload.CONFIGS["mxfp8"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    y = workload.mx_inputs(M, N, K, 0)
    got = run_mx(fb, y)
    rows, cols = _sampled(M, N, 0)
    _, ref_rows = oracle.mx_gemm(y.A, y.a_e8m0, y.B, y.b_e8m0, rows=rows)
    parity(got[rows], ref_rows, "mxfp8 rows")
    _, ref_cols = oracle.mx_gemm(y.A, y.a_e8m0, y.B, y.b_e8m0, cols=cols)
    parity(got[:, cols], ref_cols, "mxfp8 cols")
