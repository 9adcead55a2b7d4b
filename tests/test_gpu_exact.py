"""Bit-exact GPU checks where the arithmetic is exact on both sides, plus GPU invariants.

Small-integer operands with power-of-two scales make every product, partial sum and promote
exact in fp32, so the HIP output must equal the oracle bit for bit: this pins the operand
layout, the K-block and scale indexing and the output layout. One-hot operands pin the
indexing element by element."""
import numpy as np
import pytest

import workload
from gpu_util import bits, dev, parity, run_bs, run_mx, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb():
    import fp8_block_scaled_e4m3_amd as fb
    return fb


def _int_codes(rng, shape, lo=-4, hi=4):
    return workload.e4m3_encode(rng.integers(lo, hi + 1, size=shape).astype(np.float32))


class _X:
    def __init__(self, A, sa, B, sb):
        self.A, self.a_scale, self.B, self.b_scale = A, sa, B, sb


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (77, 384, 384), (256, 128, 1280)])
def test_bs_integer_exact(fb, oracle, M, N, K):
    rng = np.random.default_rng(M + N + K)
    A = _int_codes(rng, (M, K))
    B = _int_codes(rng, (N, K))
    # distinct power-of-two scales per (row, K block) and per (weight block, K block)
    sa = np.exp2(rng.integers(-3, 4, size=(M, K // 128))).astype(np.float32)
    sb = np.exp2(rng.integers(-3, 4, size=(N // 128, K // 128))).astype(np.float32)
    got = run_bs(fb, _X(A, sa, B, sb))
    _, ref = oracle.bs_gemm(A, sa, B, sb)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (64, 192, 256)])
def test_mx_integer_exact(fb, oracle, M, N, K):
    rng = np.random.default_rng(M * 3 + N + K)
    y = workload.MXInputs(M, N, K, _int_codes(rng, (M, K)),
                          rng.integers(124, 131, size=(M, K // 32)).astype(np.uint8),
                          _int_codes(rng, (N, K)),
                          rng.integers(124, 131, size=(N, K // 32)).astype(np.uint8))
    got = run_mx(fb, y)
    _, ref = oracle.mx_gemm(y.A, y.a_e8m0, y.B, y.b_e8m0)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"


def test_bs_one_hot_indexing(fb, oracle):
    """Each A row holds one non-zero at a distinct K position: C[m, n] picks B[n, k_m]
    scaled by a_s[m, k_m/128] b_s[n/128, k_m/128]; compared bit for bit."""
    rng = np.random.default_rng(11)
    M, N, K = 128, 384, 512
    A = np.zeros((M, K), np.uint8)
    ks = rng.permutation(K)[:M]
    A[np.arange(M), ks] = 0x38
    B = _int_codes(rng, (N, K), -8, 8)
    sa = np.exp2(rng.integers(-5, 6, size=(M, K // 128))).astype(np.float32)
    sb = np.exp2(rng.integers(-5, 6, size=(N // 128, K // 128))).astype(np.float32)
    got = run_bs(fb, _X(A, sa, B, sb))
    _, ref = oracle.bs_gemm(A, sa, B, sb)
    assert np.array_equal(got, ref)


def test_bs_scale_doubling_and_permutation(fb):
    """Doubling every activation scale doubles C bitwise (catches an unscaled product);
    permuting rows of A with their scales permutes rows of C bitwise; reruns are bitwise
    identical (deterministic: no atomics, no split K)."""
    x = workload.bs_inputs(192, 256, 768, 5)
    c1 = run_bs(fb, x)
    c1b = run_bs(fb, x)
    assert np.array_equal(c1, c1b)
    x2 = workload.BSInputs(x.M, x.N, x.K, x.A, x.a_scale * np.float32(2), x.B, x.b_scale)
    c2 = run_bs(fb, x2)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f(c2), 2 * f(c1))
    perm = np.random.default_rng(3).permutation(192)
    x3 = workload.BSInputs(x.M, x.N, x.K, x.A[perm], x.a_scale[perm], x.B, x.b_scale)
    c3 = run_bs(fb, x3)
    assert np.array_equal(c3, c1[perm])


def test_bs_single_block_scale_sensitivity(fb, oracle):
    """Changing one activation scale a_s[m, kb] changes row m only, as the oracle says."""
    x = workload.bs_inputs(128, 256, 512, 9)
    sa = x.a_scale.copy()
    sa[37, 2] *= np.float32(3.0)
    x2 = workload.BSInputs(x.M, x.N, x.K, x.A, sa, x.B, x.b_scale)
    c1 = run_bs(fb, x)
    c2 = run_bs(fb, x2)
    other = np.arange(128) != 37
    assert np.array_equal(c1[other], c2[other])
    _, ref = oracle.bs_gemm(x.A, sa, x.B, x.b_scale, rows=[37])
    parity(c2[37:38], ref, "row 37 after scale change")


def test_mx_exponent_shift_is_lossless(fb):
    """Adding one to every activation exponent doubles C bitwise (ue8m0 scaling is exact)."""
    y = workload.mx_inputs(128, 256, 512, 4)
    c1 = run_mx(fb, y)
    y2 = workload.MXInputs(y.M, y.N, y.K, y.A, (y.a_e8m0 + 1).astype(np.uint8), y.B, y.b_e8m0)
    c2 = run_mx(fb, y2)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f(c2), 2 * f(c1))


def test_cross_route_pow2(fb):
    """Route BS with power-of-two block scales and route MX with the same exponents broadcast
    over 32-groups and weight rows agree within the parity bar."""
    rng = np.random.default_rng(21)
    M, N, K = 128, 256, 512
    x = workload.bs_inputs(M, N, K, 21)
    ea = rng.integers(118, 124, size=(M, K // 128))
    eb = rng.integers(118, 124, size=(N // 128, K // 128))
    sa = np.exp2(ea - 127.0).astype(np.float32)
    sb = np.exp2(eb - 127.0).astype(np.float32)
    c_bs = run_bs(fb, _X(x.A, sa, x.B, sb))
    y = workload.MXInputs(M, N, K, x.A, np.repeat(ea, 4, axis=1).astype(np.uint8), x.B,
                          np.repeat(np.repeat(eb, 128, axis=0), 4, axis=1).astype(np.uint8))
    c_mx = run_mx(fb, y)
    parity(c_mx, c_bs, "mx vs bs (pow2 scales)")
