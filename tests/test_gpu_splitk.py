"""Route BS with split K (fp8bs_gemm_splitk): each output tile's K blocks are cut into equal
ranges computed by separate workgroups, whose fp32 sums a second kernel adds in order. Parity
with the oracle on shapes where the library splits and with explicit splits, the one-range call
bitwise equal to fp8bs_gemm, every split bitwise repeatable, tiles bitwise equal to each other
for the same splits, and a short workspace rejected with C untouched."""
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


def _operands(fb, x):
    return to_dev(x.A), to_dev(x.a_scale_kmajor), fb.prep_weights(to_dev(x.B)), to_dev(x.b_scale)


@pytest.mark.parametrize("M,N,K", [(1024, 2048, 7168), (600, 2048, 5120), (128, 7168, 7168), (1000, 1536, 7168)])
def test_splitk_library_choice(fb, oracle, M, N, K):
    x = workload.bs_inputs(M, N, K, 11)
    A, sa, Bp, sb = _operands(fb, x)
    ws = fb.splitk_workspace(M, N, K, 0, device=dev())
    assert ws is not None, "these shapes split"
    C = torch.full((M, N), 5.0, dtype=torch.bfloat16, device=dev())
    fb.fp8bs_gemm_splitk(A, sa, Bp, sb, C, ws)
    torch.cuda.synchronize()
    got = bits(C)
    _, ref = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    parity(got, ref, f"splitk auto {M}x{N}x{K}")
    # bitwise repeatable, workspace reused
    C2 = torch.empty_like(C)
    fb.fp8bs_gemm_splitk(A, sa, Bp, sb, C2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(C2), got)


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 8, 12])
def test_splitk_explicit(fb, oracle, splits):
    M, N, K = 600, 2048, 3072  # K/128 = 24; 600 rows: a ragged last row of tiles
    x = workload.bs_inputs(M, N, K, 12)
    A, sa, Bp, sb = _operands(fb, x)
    ws = fb.splitk_workspace(M, N, K, splits, device=dev())
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8bs_gemm_splitk(A, sa, Bp, sb, C, ws, splits)
    torch.cuda.synchronize()
    got = bits(C)
    _, ref = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    parity(got, ref, f"splitk {splits} {M}x{N}x{K}")
    if splits == 1:  # no workspace, the plain kernel
        assert ws is None
        C0 = torch.empty_like(C)
        fb.fp8bs_gemm(A, sa, Bp, sb, C0)
        torch.cuda.synchronize()
        assert np.array_equal(bits(C0), got)


def test_splitk_ranges_bitwise_repeatable(fb):
    """Every number of ranges is deterministic (fixed-order sum), workspace reused between
    calls with different numbers of ranges."""
    M, N, K = 512, 2048, 4096
    x = workload.bs_inputs(M, N, K, 13)
    A, sa, Bp, sb = _operands(fb, x)
    ws = fb.splitk_workspace(M, N, K, 8, device=dev())  # large enough for 2 and 4 ranges too
    out = {}
    for splits in (4, 2, 4, 2):
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
        fb.fp8bs_gemm_splitk(A, sa, Bp, sb, C, ws, splits)
        torch.cuda.synchronize()
        b = bits(C)
        if splits in out:
            assert np.array_equal(out[splits], b), f"{splits} ranges not repeatable"
        out[splits] = b


def test_splitk_rejections_leave_c_untouched(fb):
    M, N, K = 1024, 2048, 7168
    x = workload.bs_inputs(M, N, K, 14)
    A, sa, Bp, sb = _operands(fb, x)
    need = fb.fp8bs_splitk_workspace_bytes(M, N, K, 0)
    assert need == 2 * M * N * 4
    short = torch.empty(need - 256, dtype=torch.uint8, device=dev())
    C = torch.full((M, N), 5.0, dtype=torch.bfloat16, device=dev())
    with pytest.raises(fb.Fp8bsError) as e:
        fb.fp8bs_gemm_splitk(A, sa, Bp, sb, C, short)
    assert e.value.status == 6
    with pytest.raises(fb.Fp8bsError) as e:  # 56 K blocks do not split 3 ways
        fb.fp8bs_gemm_splitk(A, sa, Bp, sb, C, fb.splitk_workspace(M, N, K, 4, device=dev()), 3)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert torch.all(C == 5.0)
