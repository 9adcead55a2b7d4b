"""The seeded input generator (host logic, CPU only): the quantisers do what the workload
recipe says -- per-group fp32 scale amax/448 with codes reaching +-448, ue8m0 exponents that
are the smallest power of two covering amax/448, and e4m3 encoding that round-trips."""
import numpy as np
import torch

import pins
import workload


def test_e4m3_encode_round_trips_every_finite_code():
    vals = pins.torch_e4m3_values()
    codes = np.arange(256, dtype=np.uint8)
    ok = ~np.isnan(vals)
    back = workload.e4m3_encode(vals[ok].astype(np.float32))
    assert np.array_equal(back, codes[ok])


def test_e4m3_encode_saturates_and_rounds_to_nearest_even():
    x = np.array([500.0, -1e6, 448.0, 464.0, 1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11], np.float32)
    got = pins.torch_e4m3_values()[workload.e4m3_encode(x)]
    # 1.0625 is halfway between 1.0 and 1.125 -> even (1.0); 1.1875 between 1.125 and 1.25
    # -> even (1.25); 2^-10 is halfway between 0 and 2^-9 -> 0; 3*2^-11 -> 2^-9.
    assert list(got) == [448.0, -448.0, 448.0, 448.0, 1.0, 1.25, 0.0, 2.0 ** -9]


def test_bs_quantiser_groups():
    x = workload.bs_inputs(130, 256, 384, 5)
    assert x.a_scale.shape == (130, 3) and x.b_scale.shape == (2, 3)
    A, B = workload.draw(130, 256, 384, 5)
    amax_a = np.abs(A.reshape(130, 3, 128)).max(axis=2)
    assert np.array_equal(x.a_scale, (amax_a / np.float32(448)).astype(np.float32))
    vals = pins.torch_e4m3_values()
    qa = np.abs(vals[x.A]).reshape(130, 3, 128).max(axis=2)
    assert np.all(qa == 448.0)
    amax_b = np.abs(B.reshape(2, 128, 3, 128)).max(axis=(1, 3))
    assert np.array_equal(x.b_scale, (amax_b / np.float32(448)).astype(np.float32))
    # dequantised values stay within half an e4m3 step (relative 2^-4) of the draw
    deq = vals[x.A] * np.repeat(x.a_scale, 128, axis=1)
    assert np.all(np.abs(deq - A) <= 2.0 ** -4 * np.abs(A) + np.repeat(x.a_scale, 128, axis=1) * 2.0 ** -9)
    assert np.array_equal(x.a_scale_kmajor, x.a_scale.T)


def test_mx_quantiser_exponents():
    y = workload.mx_inputs(64, 96, 256, 6)
    A, B = workload.draw(64, 96, 256, 6)
    for x, e8 in ((A, y.a_e8m0), (B, y.b_e8m0)):
        amax = np.abs(x.reshape(x.shape[0], -1, 32)).max(axis=2).astype(np.float64)
        e = e8.astype(np.int64) - 127
        assert np.all(amax <= np.ldexp(448.0, e))
        assert np.all(amax > np.ldexp(448.0, e - 1))


def test_e8m0_exponent_edges():
    amax = np.array([0.0, 448.0, 448.0 * (1 + 2 ** -20), 224.0, 1e-45, 3e38])
    e = workload.e8m0_exponents(amax)
    assert list(e[:4]) == [0, 0, 1, -1]
    assert e[4] == -127 and e[5] <= 127


def test_generator_is_seeded():
    a = workload.bs_inputs(8, 128, 128, 1)
    b = workload.bs_inputs(8, 128, 128, 1)
    c = workload.bs_inputs(8, 128, 128, 2)
    assert np.array_equal(a.A, b.A) and np.array_equal(a.B, b.B)
    assert not np.array_equal(a.A, c.A)
    assert torch.equal(torch.from_numpy(a.a_scale), torch.from_numpy(b.a_scale))


def test_tiled_inputs_repeat_with_odd_periods():
    x = workload.tiled_bs_inputs(300, 1024, 256, seed=3, row_period=37, block_period=3)
    ref = workload.bs_inputs(37, 384, 256, seed=3)
    assert np.array_equal(x.A[:37], ref.A) and np.array_equal(x.A[37:74], ref.A)
    assert np.array_equal(x.a_scale[259:296], ref.a_scale)
    assert np.array_equal(x.B[:384], ref.B) and np.array_equal(x.B[768:], ref.B[:256])
    assert np.array_equal(x.b_scale[6:], ref.b_scale[:2])
    y = workload.tiled_mx_inputs(100, 64, 256, seed=4, row_period=33)
    yr = workload.mx_inputs(33, 33, 256, seed=4)
    assert np.array_equal(y.A[66:99], yr.A) and np.array_equal(y.b_e8m0[33:64], yr.b_e8m0[:31])
