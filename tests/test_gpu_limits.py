"""Operands at the largest sizes the library accepts (M * K and N * K just below 2^31 bytes,
the range of its 32-bit buffer offsets) on the GPU: routes BS and MX with the most activation
rows, the main and the small-M kernels with the most weight rows. The rows of A and the weight
blocks repeat with odd periods (workload.tiled_*), so an offset that wrapped at a power of two
would read different data; the output is compared with the oracle on rows and columns that
include the first and the last ones."""
import numpy as np
import pytest
import torch

import workload
from gpu_util import bits, dev, parity, to_dev

pytestmark = pytest.mark.gpu

K_MAX = 8192
ROWS_MAX = (2 ** 31 - 1) // K_MAX  # 262143: M * K = 2^31 - 8192


@pytest.fixture(scope="module")
def fb():
    import fp8_block_scaled_e4m3_amd as fb
    return fb


def _rows(n):
    pick = set(workload.sample_indices(n, 24, 5).tolist())
    pick.update([0, 1, n // 2, n - 2, n - 1, 262144 // 2 - 1, min(n - 1, 262143)])
    return np.array(sorted(p for p in pick if p < n), dtype=np.int64)


def test_bs_max_rows(fb, oracle):
    M, N = ROWS_MAX, 256
    x = workload.tiled_bs_inputs(M, N, K_MAX, seed=21)
    print(f"bs {M}x{N}x{K_MAX}", flush=True)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    A = to_dev(x.A)
    fb.fp8bs_gemm(A, to_dev(x.a_scale_kmajor), fb.prep_weights(to_dev(x.B)), to_dev(x.b_scale), C)
    torch.cuda.synchronize()
    rows = _rows(M)
    got = bits(C[torch.from_numpy(rows).to(dev())])
    _, ref = oracle.bs_gemm(x.A[rows], x.a_scale[rows], x.B, x.b_scale)
    parity(got, ref, f"bs max rows {M}x{N}x{K_MAX}")


def test_mx_max_rows(fb, oracle):
    M, N = (ROWS_MAX // 64) * 64, 128
    y = workload.tiled_mx_inputs(M, N, K_MAX, seed=22)
    print(f"mx {M}x{N}x{K_MAX}", flush=True)
    Bp, pb = fb.mx_prep_weights(to_dev(y.B), to_dev(y.b_e8m0))
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8mx_gemm(to_dev(y.A), fb.mx_pack_a_scale(to_dev(y.a_e8m0)), Bp, pb, C)
    torch.cuda.synchronize()
    rows = _rows(M)
    got = bits(C[torch.from_numpy(rows).to(dev())])
    _, ref = oracle.mx_gemm(y.A[rows], y.a_e8m0[rows], y.B, y.b_e8m0)
    parity(got, ref, f"mx max rows {M}x{N}x{K_MAX}")


def test_bs_max_weight_rows(fb, oracle):
    """The most weight rows (N * K just below 2^31), through the main kernel (M = 200) and the
    small-M kernel (M = 16), checked on the first, a middle and the last 128-row weight block."""
    N = (ROWS_MAX // 128) * 128
    x = workload.tiled_bs_inputs(200, N, K_MAX, seed=23)
    print(f"bs 200/16 x{N}x{K_MAX}", flush=True)
    Bp = fb.prep_weights(to_dev(x.B))
    sb = to_dev(x.b_scale)
    blocks = [0, N // 256, N // 128 - 1]
    cols = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
    B_sub = np.concatenate([x.B[128 * b:128 * b + 128] for b in blocks])
    sb_sub = x.b_scale[blocks]
    for M in (200, 16):
        A, sa = x.A[:M], np.ascontiguousarray(x.a_scale[:M])
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
        fb.fp8bs_gemm(to_dev(A), to_dev(np.ascontiguousarray(sa.T)), Bp, sb, C)
        torch.cuda.synchronize()
        assert fb.fp8bs_select_config(fb.ROUTE_BS, M, N, K_MAX).small_m == (1 if M == 16 else 0)
        got = bits(C[:, torch.from_numpy(cols).to(dev())])
        _, ref = oracle.bs_gemm(A, sa, B_sub, sb_sub)
        parity(got, ref, f"bs max weight rows M={M} N={N}")
        del C
