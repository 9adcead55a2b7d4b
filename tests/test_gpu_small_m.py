"""The small-M kernel (the decode regime; 64-row chunks of A beyond 64 rows) on the GPU through
the C ABI: full-C parity with the oracle for routes BS, PT and MX, for both variants (fragments
loaded straight into registers, operands staged through LDS), over row counts that fill 1 to 4
sixteen-row blocks (ragged included) and several chunks, and K ranges that leave some waves
without K blocks; the two variants agree bit for bit where they split K the same way; chunking
leaves every row as a call on that chunk alone computes it; bit-exact on integer operands; the
plain entry points pick the kernel by shape; errors are rejected."""
import numpy as np
import pytest
import torch

import workload
from gpu_util import bits, dev, parity, run_bs, run_pt, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb():
    import fp8_block_scaled_e4m3_amd as fb
    return fb


AUTO, DIRECT, LDS, PAIR = 1, 2, 3, 4  # PAIR: LDS-staged, two weight sub-tiles per workgroup


def _small(fb, variant=AUTO):
    c = fb.Config()
    c.small_m = variant
    return c


SHAPES = [(1, 128, 128), (5, 256, 256), (16, 384, 1024), (17, 512, 896), (33, 192, 2048), (64, 1024, 7168),
          (40, 4096, 384), (2, 192, 4096), (3, 512, 2048), (49, 256, 1408), (65, 256, 512), (100, 384, 1024),
          (130, 512, 896), (257, 192, 1280)]


def _run_bs_cfg(fb, x, cfg):
    A, sa, sb = to_dev(x.A), to_dev(x.a_scale_kmajor), to_dev(x.b_scale)
    C = torch.full((x.M, x.N), 3.0, dtype=torch.bfloat16, device=dev())
    fb.fp8bs_gemm_with_config(A, sa, fb.prep_weights(to_dev(x.B)), sb, C, cfg)
    torch.cuda.synchronize()
    return bits(C)


def _applies(variant, M):
    return variant != PAIR or M <= 32


@pytest.mark.parametrize("variant", [DIRECT, LDS, PAIR])
@pytest.mark.parametrize("M,N,K", [s for s in SHAPES if s[1] % 128 == 0])
def test_small_m_bs(fb, oracle, M, N, K, variant):
    if not _applies(variant, M):
        pytest.skip("two sub-tiles per workgroup take at most 32 rows")
    x = workload.bs_inputs(M, N, K, M + N)
    got = _run_bs_cfg(fb, x, _small(fb, variant))
    _, ref = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    parity(got, ref, f"small-M bs {M}x{N}x{K} variant {variant}")
    again = _run_bs_cfg(fb, x, _small(fb, variant))
    assert np.array_equal(got, again)  # deterministic: fixed-order sum of the wave partials


@pytest.mark.parametrize("variant", [DIRECT, LDS, PAIR])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_small_m_pt(fb, oracle, M, N, K, variant):
    if not _applies(variant, M):
        pytest.skip("two sub-tiles per workgroup take at most 32 rows")
    z = workload.pt_inputs(M, N, K, M * 7 + N)
    got = run_pt(fb, z, _small(fb, variant))
    _, ref = oracle.pt_gemm(z.A, z.a_scale, z.B, z.b_scale)
    parity(got, ref, f"small-M pt {M}x{N}x{K} variant {variant}")


@pytest.mark.parametrize("M,N,K", [s for s in SHAPES if s[1] % 128 == 0 and s[0] <= 48])
def test_small_m_variants_bitwise_equal(fb, M, N, K):
    """Up to 48 rows both variants give each of 8 waves the same K blocks and do the same
    arithmetic per block, so they agree bit for bit (with 49-64 rows the LDS-staged variant
    runs 7 waves and sums in another order); the shape-chosen variant is one of the two."""
    x = workload.bs_inputs(M, N, K, 5 * M + K)
    direct = _run_bs_cfg(fb, x, _small(fb, DIRECT))
    staged = _run_bs_cfg(fb, x, _small(fb, LDS))
    assert np.array_equal(direct, staged), f"{int((direct != staged).sum())} differ"
    if M <= 32:
        pair = _run_bs_cfg(fb, x, _small(fb, PAIR))
        assert np.array_equal(pair, staged), f"pair: {int((pair != staged).sum())} differ"
    assert np.array_equal(_run_bs_cfg(fb, x, _small(fb, AUTO)), direct)


@pytest.mark.parametrize("M,N,K", [s for s in SHAPES if s[2] >= 256] + [(24, 8192, 1024), (32, 8192, 4096)])
def test_small_m_mx(fb, oracle, M, N, K):
    y = workload.mx_inputs(M, N, K, M + 3 * N)
    Bp, pb = fb.mx_prep_weights(to_dev(y.B), to_dev(y.b_e8m0))
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8mx_gemm_small_m(to_dev(y.A), to_dev(y.a_e8m0), Bp, pb, C)
    torch.cuda.synchronize()
    _, ref = oracle.mx_gemm(y.A, y.a_e8m0, y.B, y.b_e8m0)
    parity(bits(C), ref, f"small-M mx {M}x{N}x{K}")


@pytest.mark.parametrize("variant", [AUTO, DIRECT, LDS])
@pytest.mark.parametrize("M,N,K", [(64, 256, 512), (128, 384, 1024), (192, 512, 2048), (64, 4096, 384),
                                   (320, 192, 1280)])
def test_small_m_mx_packed_scales(fb, oracle, M, N, K, variant):
    """Route MX through the main entry's packed activation scales (fp8mx_gemm_with_config with
    a small-M configuration): parity with the oracle, and bitwise equal to the row-major entry
    fp8mx_gemm_small_m (the same exponents reach the same instructions)."""
    y = workload.mx_inputs(M, N, K, M + 5 * N + K)
    Bp, pb = fb.mx_prep_weights(to_dev(y.B), to_dev(y.b_e8m0))
    A = to_dev(y.A)
    C = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=dev())
    fb.fp8mx_gemm_with_config(A, fb.mx_pack_a_scale(to_dev(y.a_e8m0)), Bp, pb, C, _small(fb, variant))
    C2 = torch.full((M, N), 5.0, dtype=torch.bfloat16, device=dev())
    fb.fp8mx_gemm_small_m(A, to_dev(y.a_e8m0), Bp, pb, C2)
    torch.cuda.synchronize()
    _, ref = oracle.mx_gemm(y.A, y.a_e8m0, y.B, y.b_e8m0)
    got = bits(C)
    parity(got, ref, f"small-M mx packed {M}x{N}x{K} variant {variant}")
    if variant == AUTO:
        assert np.array_equal(got, bits(C2))


@pytest.mark.parametrize("variant", [DIRECT, LDS, PAIR])
@pytest.mark.parametrize("M,K", [(7, 512), (48, 1280), (64, 3072)])
def test_small_m_integer_exact(fb, oracle, M, K, variant):
    if not _applies(variant, M):
        pytest.skip("two sub-tiles per workgroup take at most 32 rows")
    """Small-integer codes with power-of-two scales: every partial and the fixed-order sum of
    the wave partials are exact in fp32, so the output equals the oracle bit for bit."""
    N = 256
    rng = np.random.default_rng(M + K)
    A = workload.e4m3_encode(rng.integers(-4, 5, size=(M, K)).astype(np.float32))
    B = workload.e4m3_encode(rng.integers(-4, 5, size=(N, K)).astype(np.float32))
    sa = np.exp2(rng.integers(-3, 4, size=(M, K // 128))).astype(np.float32)
    sb = np.exp2(rng.integers(-3, 4, size=(N // 128, K // 128))).astype(np.float32)
    x = workload.BSInputs(M, N, K, A, sa, B, sb)
    got = _run_bs_cfg(fb, x, _small(fb, variant))
    _, ref = oracle.bs_gemm(A, sa, B, sb)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("variant", [DIRECT, LDS])
def test_small_m_chunks_are_independent(fb, variant):
    """130 rows run as three 64-row chunks (the last ragged) give bit for bit what separate
    calls on rows 0-63, 64-127 and 128-129 give."""
    M, N, K = 130, 512, 1024
    x = workload.bs_inputs(M, N, K, 31)
    whole = _run_bs_cfg(fb, x, _small(fb, variant))
    for lo, hi in ((0, 64), (64, 128), (128, 130)):
        part = workload.BSInputs(hi - lo, N, K, x.A[lo:hi], x.a_scale[lo:hi], x.B, x.b_scale)
        got = _run_bs_cfg(fb, part, _small(fb, variant))
        assert np.array_equal(got, whole[lo:hi]), (lo, hi)


def test_plain_entry_picks_small_m(fb, oracle):
    """fp8bs_gemm and fp8pt_gemm use the small-M kernel for few rows and narrow outputs, the
    main kernel when the main kernel's tiles fill the device."""
    assert fb.fp8bs_select_config(fb.ROUTE_BS, 8, 7168, 7168).small_m == 1
    assert fb.fp8bs_select_config(fb.ROUTE_BS, 64, 2048, 7168).small_m == 1
    assert fb.fp8bs_select_config(fb.ROUTE_BS, 64, 65536, 1536).small_m == 0
    assert fb.fp8bs_select_config(fb.ROUTE_BS, 65, 2048, 7168).small_m == 1  # 64-row chunks
    assert fb.fp8bs_select_config(fb.ROUTE_BS, 1024, 2048, 7168).small_m == 0
    assert fb.fp8bs_select_config(fb.ROUTE_PT, 1, 4096, 512).small_m == 1
    assert fb.fp8bs_select_config(fb.ROUTE_MX, 64, 4096, 512).small_m == 1  # packed activation scales
    assert fb.fp8bs_select_config(fb.ROUTE_MX, 64, 32768, 1536).small_m == 0
    x = workload.bs_inputs(24, 2048, 1024, 2)
    got = run_bs(fb, x)  # plain entry point
    assert np.array_equal(got, _run_bs_cfg(fb, x, _small(fb)))


@pytest.mark.parametrize("route,M,N,K", [("bs", 200, 2048, 4096), ("pt", 130, 1536, 4608), ("mx", 128, 2048, 4096),
                                         ("mx", 64, 512, 1280), ("bs", 128, 256, 512), ("bs", 256, 1024, 2048),
                                         ("pt", 192, 512, 1024), ("mx", 256, 1024, 2048)])
def test_plain_entry_small_m_routes(fb, oracle, route, M, N, K):
    """Shapes on which the plain entry points select the small-M kernel (64-row chunks while the
    main kernel's grid would be small; route MX on its packed activation scales): full-C parity
    with the oracle."""
    rid = {"bs": fb.ROUTE_BS, "pt": fb.ROUTE_PT, "mx": fb.ROUTE_MX}[route]
    assert fb.fp8bs_select_config(rid, M, N, K).small_m == 1, (route, M, N, K)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    if route == "bs":
        x = workload.bs_inputs(M, N, K, M + N)
        got = run_bs(fb, x, C)
        _, ref = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    elif route == "pt":
        z = workload.pt_inputs(M, N, K, M + N)
        got = run_pt(fb, z)
        _, ref = oracle.pt_gemm(z.A, z.a_scale, z.B, z.b_scale)
    else:
        y = workload.mx_inputs(M, N, K, M + N)
        Bp, pb = fb.mx_prep_weights(to_dev(y.B), to_dev(y.b_e8m0))
        fb.fp8mx_gemm(to_dev(y.A), fb.mx_pack_a_scale(to_dev(y.a_e8m0)), Bp, pb, C)
        torch.cuda.synchronize()
        got = bits(C)
        _, ref = oracle.mx_gemm(y.A, y.a_e8m0, y.B, y.b_e8m0)
    parity(got, ref, f"plain {route} {M}x{N}x{K}")


def test_small_m_rejects(fb):
    y = workload.bs_inputs(8, 256, 256, 0)
    for variant in (-1, 5):  # no such variant
        with pytest.raises(fb.Fp8bsError) as e:
            _run_bs_cfg(fb, y, _small(fb, variant))
        assert e.value.status == 4
    z = workload.bs_inputs(33, 256, 256, 0)  # two sub-tiles per workgroup take at most 32 rows
    with pytest.raises(fb.Fp8bsError) as e:
        _run_bs_cfg(fb, z, _small(fb, PAIR))
    assert e.value.status == 4
    # shapes past the small-M kernel's chunk limit are rejected on the host: covered on the CPU
    # with placeholder pointers (tests/test_abi.py), so no device call here gets a short buffer
