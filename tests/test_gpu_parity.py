"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Small shapes are compared in full, including ragged M tails and several tiles in each
direction. The large benchmark workloads are compared in full for seed 0 and on seeded
samples of 512 whole rows and 512 whole columns for seeds 1-3 (the oracle computes each
element independently, so a sample is exact)."""
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


# ragged M through the plain entry on shapes where the selector takes paths the workloads do
# not: 8200 x 7168 x 768 the warp-specialised 128x256 tile in 8-row bands with loader priority
# (route BS, K <= 1536), its last tile row 8 rows deep; 2000 x 8192 x 1536 the 256x256 tile with
# C written through the L2; 4100 x 4352 x 7168 the 128x256 tile at deep K, C written through;
# 8195 x 16896 x 256 a C over 256 MiB, written through as non-temporal lines
@pytest.mark.parametrize("M,N,K", [(8200, 7168, 768), (2000, 8192, 1536), (4100, 4352, 7168), (8195, 16896, 256)])
def test_bs_selector_paths_ragged_full(fb, oracle, M, N, K):
    c = fb.fp8bs_select_config(fb.ROUTE_BS, M, N, K)
    x = workload.bs_inputs(M, N, K, 3)
    got = run_bs(fb, x)
    _, ref = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    parity(got, ref, f"bs {M}x{N}x{K} ({c})")


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_tiny_workload_full_every_seed(fb, oracle, seed):
    """The tiny workload (128 x 256 x 512) in full for seeds 0-3, through the plain entry point
    and its own kernel choice (page "Flydsl Fp8 Blockscale Gemm", front matter: seeds 0-3)."""
    cfg, x = _inputs("tiny", seed)
    got = _run(fb, cfg, x)
    parity(got, _ref(oracle, cfg, x), f"tiny full C seed {seed}")


def _sampled(M, N, seed, n=512):
    return workload.sample_indices(M, n, seed), workload.sample_indices(N, n, seed + 1)


def _inputs(name, seed):
    cfg = workload.CONFIGS[name]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    if cfg["route"] == "bs":
        return cfg, workload.bs_inputs(M, N, K, seed)
    return cfg, workload.mx_inputs(M, N, K, seed)


def _run(fb, cfg, x):
    return run_bs(fb, x) if cfg["route"] == "bs" else run_mx(fb, x)


def _ref(oracle, cfg, x, rows=None, cols=None):
    if cfg["route"] == "bs":
        return oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale, rows=rows, cols=cols)[1]
    return oracle.mx_gemm(x.A, x.a_e8m0, x.B, x.b_e8m0, rows=rows, cols=cols)[1]


@pytest.mark.parametrize("name", ["narrow_n", "k_light", "wide_n", "mxfp8", "narrow_n_16k", "mxfp8_k2048",
                                  "wide_n_shard8"])
def test_workload_full_seed0(fb, oracle, name):
    """Every element of C at the benchmark size, in the launch configuration the benchmark
    times (the library's own choice for the shape), seed 0."""
    cfg, x = _inputs(name, 0)
    got = _run(fb, cfg, x)
    ref = _ref(oracle, cfg, x)
    parity(got, ref, f"{name} full C seed 0")


@pytest.mark.parametrize("name", ["narrow_n", "k_light", "wide_n", "mxfp8", "narrow_n_16k", "mxfp8_k2048",
                                  "wide_n_shard8"])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_workload_sampled(fb, oracle, name, seed):
    """512 whole rows and 512 whole columns of C at the benchmark size for seeds 1-3 (the
    oracle computes each element on its own, so a sample is exact)."""
    cfg, x = _inputs(name, seed)
    got = _run(fb, cfg, x)
    rows, cols = _sampled(cfg["M"], cfg["N"], seed)
    parity(got[rows], _ref(oracle, cfg, x, rows=rows), f"{name} seed {seed} rows")
    parity(got[:, cols], _ref(oracle, cfg, x, cols=cols), f"{name} seed {seed} cols")
