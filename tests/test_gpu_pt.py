"""Route PT (the promote-free twin: one fp32 scale per row of A and per row of B) on the GPU,
through the C ABI, against the oracle: full C on small and ragged shapes and at the two
benchmark sizes it is measured on, bit-exact on integer operands, every kernel configuration
bitwise equal to the default, and the error paths."""
import itertools

import numpy as np
import pytest
import torch

import workload
from gpu_util import bits, dev, parity, run_pt, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb():
    import fp8_block_scaled_e4m3_amd as fb
    return fb


class _Z:
    def __init__(self, A, sa, B, sb):
        self.A, self.a_scale, self.B, self.b_scale = A, sa, B, sb


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (1, 64, 128), (63, 192, 384), (200, 512, 640),
                                   (257, 128, 1024), (512, 896, 128)])
@pytest.mark.parametrize("seed", [0, 1])
def test_pt_small_full(fb, oracle, M, N, K, seed):
    z = workload.pt_inputs(M, N, K, seed)
    got = run_pt(fb, z)
    _, ref = oracle.pt_gemm(z.A, z.a_scale, z.B, z.b_scale)
    parity(got, ref, f"pt {M}x{N}x{K} seed {seed}")


@pytest.mark.parametrize("name", ["narrow_n", "k_light"])
def test_pt_workload_full(fb, oracle, name):
    """Every element of C at the benchmark size, seed 0 (the twin is timed on these shapes)."""
    cfg = workload.CONFIGS[name]
    z = workload.pt_inputs(cfg["M"], cfg["N"], cfg["K"], 0)
    got = run_pt(fb, z)
    _, ref = oracle.pt_gemm(z.A, z.a_scale, z.B, z.b_scale)
    parity(got, ref, f"pt {name} full C")


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (77, 384, 384)])
def test_pt_integer_exact(fb, oracle, M, N, K):
    """Small-integer codes with power-of-two row scales: the fp32 accumulation and the scale
    product are exact, so the output equals the oracle bit for bit."""
    rng = np.random.default_rng(M * 3 + N + K)
    A = workload.e4m3_encode(rng.integers(-4, 5, size=(M, K)).astype(np.float32))
    B = workload.e4m3_encode(rng.integers(-4, 5, size=(N, K)).astype(np.float32))
    sa = np.exp2(rng.integers(-3, 4, size=M)).astype(np.float32)
    sb = np.exp2(rng.integers(-3, 4, size=N)).astype(np.float32)
    got = run_pt(fb, _Z(A, sa, B, sb))
    _, ref = oracle.pt_gemm(A, sa, B, sb)
    assert np.array_equal(got, ref)


TILES = [(128, 128, 2, 2, 3, 0), (256, 256, 4, 2, 2, 0), (256, 256, 2, 4, 2, 0), (128, 256, 2, 2, 3, 0),
         (256, 128, 2, 2, 3, 0), (128, 256, 2, 4, 3, 0), (256, 128, 4, 2, 3, 0), (128, 64, 2, 1, 3, 0),
         (256, 128, 4, 2, 2, 0), (128, 128, 2, 2, 4, 0), (128, 128, 2, 2, 2, 0), (256, 128, 4, 2, 2, 1),
         (128, 256, 2, 4, 2, 1), (256, 128, 4, 2, 3, 2), (128, 256, 2, 4, 3, 2), (256, 128, 2, 2, 3, 2),
         (128, 128, 2, 2, 3, 2)]


@pytest.mark.parametrize("M,N,K", [(300, 512, 384), (4160, 3072, 640)])
def test_pt_all_configs_bitwise_equal(fb, oracle, M, N, K):
    z = workload.pt_inputs(M, N, K, 5)
    ref_bits = run_pt(fb, z)
    _, ref = oracle.pt_gemm(z.A, z.a_scale, z.B, z.b_scale)
    parity(ref_bits, ref, f"pt default {M}x{N}x{K}")
    n = 0
    for (bm, bn, wm, wn, st, pp), (gm, xcd, pers, cst) in itertools.product(
            TILES, ((1, 0, 0, 1), (3, 1, 1, 0), (2, 2, 1, 2))):
        if N % bn:
            continue
        got = run_pt(fb, z, fb.Config(bm, bn, wm, wn, st, gm, xcd, pers, pp, 0, cst))
        assert np.array_equal(got, ref_bits), f"{(bm, bn, wm, wn, st, pp, gm, xcd, pers, cst)}: differs"
        n += 1
    assert n >= 20


def test_pt_errors_leave_c_untouched(fb):
    d = dev()
    M, N, K = 128, 128, 256
    A = torch.zeros((M, K), dtype=torch.uint8, device=d)
    B = torch.zeros((N, K), dtype=torch.uint8, device=d)
    Bp = fb.prep_weights(B)
    sa = torch.ones(M, dtype=torch.float32, device=d)
    sb = torch.ones(N + 4, dtype=torch.float32, device=d)
    C = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=d)
    call = lambda *a: fb.lib.fp8pt_gemm(*a, None)
    assert call(A.data_ptr(), sa.data_ptr(), Bp.data_ptr(), sb.data_ptr(), C.data_ptr(), M, 96, K) == 2
    assert call(A.data_ptr(), sa.data_ptr(), Bp.data_ptr(), sb.data_ptr(), C.data_ptr(), M, N, 200) == 2
    assert call(None, sa.data_ptr(), Bp.data_ptr(), sb.data_ptr(), C.data_ptr(), M, N, K) == 1
    assert call(A.data_ptr(), sa.data_ptr(), Bp.data_ptr(), sb.data_ptr() + 4, C.data_ptr(), M, N, K) == 3
    assert call(A.data_ptr(), sa.data_ptr(), Bp.data_ptr(), sb.data_ptr(), C.data_ptr(), 0, N, K) == 0
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)
