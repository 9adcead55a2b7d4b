"""Activation quantisers on the GPU (through the C ABI) against the oracle's quantisers:
codes and scales bit for bit, for fp32 and bf16 input, on gaussian rows and rows that stress
the encoder (all zero, one huge value, tiny values, exact e4m3 values times 2^k, NaN of
either sign), at
small, ragged and benchmark-sized shapes, and on every finite bf16 value under ~200 group
maxima; then quantise -> GEMM end to end for both routes."""
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


def _stress(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    if M > 6:
        x[1] = 0
        x[2] *= np.float32(2.0 ** -20)
        x[3, 5] = 3.0e5
        codes = rng.integers(0, 256, K).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x7E
        x[4] = (torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy() * 2.0 ** 7)
        x[5, :] = -1.0
        x[6, 3] = np.nan
        x[6, 100 % K] = -np.nan
    return x


def _as_input(x, dtype):
    """(device tensor, the exact fp32 values the kernel sees)."""
    t = torch.from_numpy(x)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(dev()), t.to(torch.float32).numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,K", [(1, 128), (8, 256), (77, 384), (300, 1280), (1024, 7168)])
def test_quantize_bs_bitwise(fb, oracle, dtype, M, K):
    xd, xf = _as_input(_stress(M, K, M + K), dtype)
    A, sa = fb.quantize_bs(xd)
    torch.cuda.synchronize()
    codes, scale = oracle.quantize_bs(xf)
    got_scale = sa.cpu().numpy().T  # [K/128, M] -> [M, K/128]
    assert np.array_equal(got_scale.view(np.uint32), scale.view(np.uint32)), "scales differ"
    got = A.cpu().numpy()
    bad = np.flatnonzero(got != codes)
    assert bad.size == 0, [(int(i // K), int(i % K), float(xf.flat[i]), int(got.flat[i]), int(codes.flat[i]))
                           for i in bad[:5]]


def _every_bf16_under(amaxes, group, K):
    """Rows of bf16-exact fp32 values: for each amax, every finite bf16 value v with |v| <= amax,
    in groups of `group` whose first element is amax (so amax is the group's amax)."""
    u = np.arange(1 << 16, dtype=np.uint32) << 16
    allv = u.view(np.float32)
    allv = allv[np.isfinite(allv)]
    groups = []
    for a in amaxes:
        v = allv[np.abs(allv) <= a]
        v = np.concatenate([v, np.zeros((-len(v)) % (group - 1), np.float32)])
        g = v.reshape(-1, group - 1)
        groups.append(np.concatenate([np.full((len(g), 1), a, np.float32), g], axis=1))
    x = np.concatenate(groups).reshape(-1)
    x = np.concatenate([x, np.zeros((-len(x)) % K, np.float32)])
    return x.reshape(-1, K)


def _bf16_amaxes():
    out = []
    for e in range(-133, 128, 4):
        for m in (1.0, 1.5078125, 1.9921875):
            a = np.float32(np.ldexp(m, e))
            b = torch.tensor([float(a)], dtype=torch.float32).to(torch.bfloat16).to(torch.float32).item()
            if 0 < b < 3.4e38:
                out.append(np.float32(b))
    return sorted(set(out + [np.float32(448.0), np.float32(1.0), np.float32(3.5)]))


@pytest.mark.parametrize("route", ["bs", "mx"])
def test_quantize_every_bf16_value(fb, oracle, route):
    """Every finite bf16 value, quantised in groups whose amax runs over ~200 values from the
    subnormal range to near the bf16 maximum: codes and scales bit for bit. This covers every
    (value, scale) pair of the encoder's arithmetic that bf16 input can reach at these scales,
    ties and near-ties of the e4m3 rounding included."""
    group = 128 if route == "bs" else 32
    x = _every_bf16_under(_bf16_amaxes(), group, 1024)
    print(f"{route}: {x.size} values", flush=True)
    xd = torch.from_numpy(x).to(torch.bfloat16).to(dev())
    if route == "bs":
        A, sc = fb.quantize_bs(xd)
        torch.cuda.synchronize()
        codes, ref = oracle.quantize_bs(x)
        assert np.array_equal(sc.cpu().numpy().T.view(np.uint32), ref.view(np.uint32)), "scales differ"
    else:
        A, sc = fb.quantize_mx(xd)
        torch.cuda.synchronize()
        codes, ref = oracle.quantize_mx(x)
        assert np.array_equal(sc.cpu().numpy(), ref), "exponents differ"
    got = A.cpu().numpy()
    bad = np.flatnonzero(got != codes)
    assert bad.size == 0, [(float(x.flat[i]), int(got.flat[i]), int(codes.flat[i])) for i in bad[:5]]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,K", [(1, 32), (8, 256), (77, 384), (320, 1280), (1024, 7168)])
def test_quantize_mx_bitwise(fb, oracle, dtype, M, K):
    xd, xf = _as_input(_stress(M, K, M * 3 + K), dtype)
    A, e8 = fb.quantize_mx(xd)
    torch.cuda.synchronize()
    codes, e8ref = oracle.quantize_mx(xf)
    assert np.array_equal(e8.cpu().numpy(), e8ref), "exponents differ"
    got = A.cpu().numpy()
    bad = np.flatnonzero(got != codes)
    assert bad.size == 0, [(int(i // K), int(i % K), float(xf.flat[i]), int(got.flat[i]), int(codes.flat[i]))
                           for i in bad[:5]]


def test_quantize_then_bs_gemm(fb, oracle):
    """bf16 activations -> fp8bs_quantize_act -> fp8bs_gemm equals the oracle's quantiser
    followed by the oracle's GEMM."""
    M, N, K = 200, 512, 1024
    rng = np.random.default_rng(3)
    xd, xf = _as_input(rng.standard_normal((M, K)).astype(np.float32), "bf16")
    wb = workload.bs_inputs(8, N, K, 3)
    A, sa = fb.quantize_bs(xd)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8bs_gemm(A, sa, fb.prep_weights(to_dev(wb.B)), to_dev(wb.b_scale), C)
    torch.cuda.synchronize()
    codes, scale = oracle.quantize_bs(xf)
    _, ref = oracle.bs_gemm(codes, scale, wb.B, wb.b_scale)
    parity(bits(C), ref, "quantise -> bs gemm")


def test_quantize_then_mx_gemm(fb, oracle):
    M, N, K = 192, 256, 1280
    rng = np.random.default_rng(4)
    xd, xf = _as_input(rng.standard_normal((M, K)).astype(np.float32), "f32")
    wm = workload.mx_inputs(64, N, K, 4)
    A, e8 = fb.quantize_mx(xd)
    Bp, pb = fb.mx_prep_weights(to_dev(wm.B), to_dev(wm.b_e8m0))
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8mx_gemm(A, fb.mx_pack_a_scale(e8), Bp, pb, C)
    torch.cuda.synchronize()
    codes, e8ref = oracle.quantize_mx(xf)
    _, ref = oracle.mx_gemm(codes, e8ref, wm.B, wm.b_e8m0)
    parity(bits(C), ref, "quantise -> mx gemm")


def test_quantize_errors(fb):
    x = torch.zeros((64, 256), dtype=torch.float32, device=dev())
    A = torch.full((64, 256), 0x11, dtype=torch.uint8, device=dev())
    s = torch.zeros((2, 64), dtype=torch.float32, device=dev())
    e = torch.zeros((64, 8), dtype=torch.uint8, device=dev())
    L = fb.lib
    assert L.fp8bs_quantize_act(x.data_ptr(), 0, A.data_ptr(), s.data_ptr(), 64, 200, None) == 2
    assert L.fp8bs_quantize_act(x.data_ptr(), 7, A.data_ptr(), s.data_ptr(), 64, 256, None) == 4
    assert L.fp8bs_quantize_act(None, 0, A.data_ptr(), s.data_ptr(), 64, 256, None) == 1
    assert L.fp8bs_quantize_act(x.data_ptr() + 4, 0, A.data_ptr(), s.data_ptr(), 64, 128, None) == 3
    assert L.fp8mx_quantize_act(x.data_ptr(), 0, A.data_ptr(), e.data_ptr(), 64, 48, None) == 2
    assert L.fp8mx_quantize_act(x.data_ptr(), 1, A.data_ptr() + 8, e.data_ptr(), 64, 256, None) == 3
    assert L.fp8bs_quantize_act(x.data_ptr(), 0, A.data_ptr(), s.data_ptr(), 0, 256, None) == 0
    torch.cuda.synchronize()
    assert torch.all(A == 0x11)
