"""The oracle against its pins (CPU only): codecs against torch's float8/bf16 conversions,
the GEMM against exact brute force, closed forms and scale invariants."""
import numpy as np
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(oracle, pin):
    pin(oracle)


def test_sampled_grid_matches_full(oracle):
    """Computing a sampled grid of rows x columns gives the same values as the full C."""
    import workload
    x = workload.bs_inputs(64, 384, 256, 3)
    acc, bits = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    rows = np.array([0, 5, 63], np.int32)
    cols = np.array([1, 200, 383], np.int32)
    acc_s, bits_s = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale, rows, cols)
    assert np.array_equal(acc_s, acc[np.ix_(rows, cols)])
    assert np.array_equal(bits_s, bits[np.ix_(rows, cols)])


def test_rejects_bad_shapes(oracle):
    A = np.zeros((4, 100), np.uint8)
    with pytest.raises(ValueError):
        oracle.bs_gemm(A, np.ones((4, 1), np.float32), A, np.ones((1, 1), np.float32))
    A = np.zeros((4, 128), np.uint8)
    with pytest.raises(ValueError):
        oracle.bs_gemm(A, np.ones((4, 2), np.float32), A, np.ones((1, 1), np.float32))


def test_nan_propagates(oracle):
    """e4m3 NaN codes and ue8m0 byte 255 are out of contract; the oracle propagates NaN."""
    A = np.full((1, 128), 0x38, np.uint8)
    A[0, 5] = 0x7F
    B = np.full((1, 128), 0x38, np.uint8)
    acc, bits = oracle.bs_gemm(A, np.ones((1, 1), np.float32), B, np.ones((1, 1), np.float32))
    assert np.isnan(acc[0, 0]) and (int(bits[0, 0]) & 0x7FFF) > 0x7F80
    acc, _ = oracle.mx_gemm(B, np.full((1, 4), 255, np.uint8), B, np.full((1, 4), 127, np.uint8))
    assert np.isnan(acc[0, 0])
