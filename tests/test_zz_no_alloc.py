"""The allocation-free split-K entry (fp8bs_gemm_splitk_noalloc, through the C ABI): its output
is the workspace entry's (fp8bs_gemm_splitk) bit for bit and meets the parity bar against the
oracle, on two calls in a row, the second with a smaller input; a call whose partial tiles
exceed the static scratch is rejected with C untouched."""
import numpy as np
import pytest
import torch

import workload
from gpu_util import bits, dev, parity, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb():
    import fp8_block_scaled_e4m3_amd as fb
    return fb


def _noalloc(fb, A, sa, Bp, sb, C, M, N, K, splits):
    """The entry point through the C ABI: plain device pointers, sizes and the current stream."""
    return fb.lib.fp8bs_gemm_splitk_noalloc(A.data_ptr(), sa.data_ptr(), Bp.data_ptr(), sb.data_ptr(),
                                           C.data_ptr(), M, N, K, splits,
                                           torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry(fb, oracle, order):
    # first call 16 MiB of partial tiles (2 ranges), the second a smaller input (600 rows,
    # 2 ranges, 9.4 MiB): the second reads only what it wrote itself
    for i, (M, N, K) in enumerate([(1024, 2048, 7168), (600, 2048, 5120)]):
        x = workload.bs_inputs(M, N, K, 21 + i)
        A, sa, Bp, sb = to_dev(x.A), to_dev(x.a_scale_kmajor), fb.prep_weights(to_dev(x.B)), to_dev(x.b_scale)
        assert 0 < fb.fp8bs_splitk_workspace_bytes(M, N, K, 0) <= fb.SPLITK_SCRATCH_BYTES
        ws = fb.splitk_workspace(M, N, K, 0, device=dev())
        C_ws = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
        fb.fp8bs_gemm_splitk(A, sa, Bp, sb, C_ws, ws)
        C = torch.full((M, N), 9.0, dtype=torch.bfloat16, device=dev())
        assert _noalloc(fb, A, sa, Bp, sb, C, M, N, K, 0) == 0
        torch.cuda.synchronize()
        got = bits(C)
        assert np.array_equal(got, bits(C_ws)), f"call {i}: differs from the workspace entry"
        rows = workload.sample_indices(M, 64, 30 + i)
        _, ref = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale, rows=rows)
        parity(got[rows], ref, f"noalloc call {i} {M}x{N}x{K} sampled rows")


def test_noalloc_rejects_beyond_scratch(fb):
    M, N, K = 1024, 2048, 7168
    assert fb.fp8bs_splitk_workspace_bytes(M, N, K, 8) > fb.SPLITK_SCRATCH_BYTES  # 64 MiB
    x = workload.bs_inputs(M, N, K, 23)
    A, sa, Bp, sb = to_dev(x.A), to_dev(x.a_scale_kmajor), fb.prep_weights(to_dev(x.B)), to_dev(x.b_scale)
    C = torch.full((M, N), 9.0, dtype=torch.bfloat16, device=dev())
    assert _noalloc(fb, A, sa, Bp, sb, C, M, N, K, 8) == 6
    torch.cuda.synchronize()
    assert torch.all(C == 9.0)
