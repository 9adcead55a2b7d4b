"""Error paths of the C ABI on the GPU: rejected shapes and pointers return status codes,
launch nothing and leave C untouched."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb():
    import fp8_block_scaled_e4m3_amd as fb
    return fb


def _bufs(M, N, K):
    d = torch.device("cuda:0")
    A = torch.zeros((M, K), dtype=torch.uint8, device=d)
    sa = torch.ones((max(K // 128, 1), M), dtype=torch.float32, device=d)
    B = torch.zeros((N, K), dtype=torch.uint8, device=d)
    sb = torch.ones((max(N // 128, 1), max(K // 128, 1)), dtype=torch.float32, device=d)
    C = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=d)
    return A, sa, B, sb, C


@pytest.mark.parametrize("M,N,K", [(128, 100, 128), (128, 128, 100), (128, 128, 0), (-1, 128, 128), (64, 64, 128)])
def test_bs_rejects_bad_shapes(fb, M, N, K):
    A, sa, B, sb, C = _bufs(max(M, 1), max(N, 1), max(K, 1))
    st = fb.lib.fp8bs_gemm(A.data_ptr(), sa.data_ptr(), B.data_ptr(), sb.data_ptr(), C.data_ptr(),
                           M, N, K, None)
    torch.cuda.synchronize()
    assert st == 2
    assert torch.all(C == 7.0)


def test_bs_rejects_null_and_misaligned(fb):
    A, sa, B, sb, C = _bufs(128, 128, 256)
    st = fb.lib.fp8bs_gemm(None, sa.data_ptr(), B.data_ptr(), sb.data_ptr(), C.data_ptr(), 128, 128, 256, None)
    assert st == 1
    st = fb.lib.fp8bs_gemm(A.data_ptr() + 8, sa.data_ptr(), B.data_ptr(), sb.data_ptr(), C.data_ptr(),
                           120, 128, 256, None)
    assert st == 3
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)


@pytest.mark.parametrize("M,N,K", [(100, 128, 256), (128, 96, 256), (128, 128, 128), (128, 128, 200)])
def test_mx_rejects_bad_shapes(fb, M, N, K):
    A, _, B, _, C = _bufs(M, N, K)
    pa = torch.zeros(4096, dtype=torch.uint8, device=A.device)
    st = fb.lib.fp8mx_gemm(A.data_ptr(), pa.data_ptr(), B.data_ptr(), pa.data_ptr(), C.data_ptr(),
                           M, N, K, None)
    torch.cuda.synchronize()
    assert st == 2
    assert torch.all(C == 7.0)


def test_zero_rows_is_noop(fb):
    A, sa, B, sb, C = _bufs(1, 128, 128)
    assert fb.lib.fp8bs_gemm(A.data_ptr(), sa.data_ptr(), B.data_ptr(), sb.data_ptr(), C.data_ptr(),
                             0, 128, 128, None) == 0
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)


def test_python_wrapper_raises(fb):
    """A shape the library rejects (N % 128 != 0) surfaces as Fp8bsError with its status code."""
    A, sa, _, sb, _ = _bufs(128, 128, 256)
    B = torch.zeros((100, 256), dtype=torch.uint8, device=A.device)
    C = torch.full((128, 100), 7.0, dtype=torch.bfloat16, device=A.device)
    with pytest.raises(fb.Fp8bsError) as e:
        fb.fp8bs_gemm(A, sa, B, sb, C)
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)


def test_zero_rows_is_noop_every_route(fb):
    """M = 0 is valid for every GEMM entry point: nothing is launched and C is untouched."""
    d = torch.device("cuda:0")
    A = torch.zeros((64, 256), dtype=torch.uint8, device=d)
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device=d)
    fbuf = torch.ones(1 << 14, dtype=torch.float32, device=d)
    C = torch.full((64, 256), 7.0, dtype=torch.bfloat16, device=d)
    L = fb.lib
    assert L.fp8mx_gemm(A.data_ptr(), buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), C.data_ptr(), 0, 256, 256,
                        None) == 0
    assert L.fp8pt_gemm(A.data_ptr(), fbuf.data_ptr(), buf.data_ptr(), fbuf.data_ptr(), C.data_ptr(), 0, 256, 256,
                        None) == 0
    assert L.fp8mx_gemm_small_m(A.data_ptr(), buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), C.data_ptr(), 0, 256,
                                256, None) == 0
    assert L.fp8mx_quantize_act(fbuf.data_ptr(), 0, A.data_ptr(), buf.data_ptr(), 0, 256, None) == 0
    torch.cuda.synchronize()
    assert torch.all(C == 7.0) and torch.all(A == 0)
