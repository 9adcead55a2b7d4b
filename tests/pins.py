"""Pins for the oracle: checks that tie it to something other than itself.

Each ``pin_*`` function takes an oracle handle (``oracle.Oracle``) and raises
``AssertionError`` on a mismatch. The test files run them against the real oracle (all must
pass) and against deliberately broken copies of it (at least one must fail per copy), which
shows that a plausible mistake anywhere in the oracle is caught.

Independent references used here, none of which calls the oracle's own arithmetic:

* e4m3 and ue8m0 decoding: torch's ``float8_e4m3fn`` / ``float8_e8m0fnu`` dtypes;
* bf16 rounding: torch's fp32 -> bf16 conversion (round to nearest even) on fp32-exact
  values, and exact rational rounding (``fractions.Fraction``, ``round`` = half-to-even);
* the GEMM: exact integer block sums (every e4m3 value is an integer times 2^-9) combined
  with the scales as exact rationals, then rounded once to bf16.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

import workload

# -------------------------------------------------------------------------------------
# Independent references
# -------------------------------------------------------------------------------------


def torch_e4m3_values() -> np.ndarray:
    """All 256 e4m3 codes decoded by torch (float64; NaN for the two NaN codes)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


_E4M3_INT = None


def e4m3_int(codes: np.ndarray) -> np.ndarray:
    """Codes -> the integer i with value = i * 2^-9 (from torch's decoding; NaN codes -> 0)."""
    global _E4M3_INT
    if _E4M3_INT is None:
        vals = torch_e4m3_values()
        ints = np.where(np.isnan(vals), 0.0, vals) * 512.0
        assert np.all(ints == np.round(ints))
        _E4M3_INT = ints.astype(np.int64)
    return _E4M3_INT[np.asarray(codes, dtype=np.uint8)]


def exact_bf16_bits(v: Fraction) -> int:
    """Round an exact rational to bf16 (nearest, ties to even) and return its bit pattern."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = -v if v < 0 else v
    # e = floor(log2 a), found exactly.
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q_exp = max(e, -126) - 7
    quantum = Fraction(2) ** q_exp
    r = round(a / quantum)  # Fraction.__round__ rounds half to even
    value = r * quantum
    if value >= Fraction(2) ** 128:
        return sign | 0x7F80
    f = np.float32(float(value))  # exact: value has <= 8 significant bits in fp32 range
    assert Fraction(float(f)) == value
    return sign | int(np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16)


def bf16_neighbourhood_tie(v: Fraction, slack: Fraction) -> bool:
    """True when v lies within ``slack`` of a bf16 rounding midpoint (fp64 round-off in the
    oracle may then legitimately pick the other side)."""
    return exact_bf16_bits(v - slack) != exact_bf16_bits(v + slack)


def exact_bs(A, a_scale, B, b_scale):
    """Exact route-BS result as Fractions [M][N] plus the sum of |terms| per element.

    Integer block sums via int64 (exact: |sum| < 2^43), combined with the fp32 scales as
    exact rationals."""
    M, K = A.shape
    N = B.shape[0]
    KB = K // 128
    ai = e4m3_int(A)
    bi = e4m3_int(B)
    sums = [ai[:, kb * 128:(kb + 1) * 128] @ bi[:, kb * 128:(kb + 1) * 128].T for kb in range(KB)]
    sa = [[Fraction(float(a_scale[m, kb])) for kb in range(KB)] for m in range(M)]
    sb = [[Fraction(float(b_scale[nb, kb])) for kb in range(KB)] for nb in range(b_scale.shape[0])]
    two18 = Fraction(1, 2 ** 18)
    out = [[None] * N for _ in range(M)]
    mag = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            ab = Fraction(0)
            for kb in range(KB):
                t = int(sums[kb][m, n]) * two18 * sa[m][kb] * sb[n // 128][kb]
                tot += t
                ab += abs(t)
            out[m][n] = tot
            mag[m][n] = ab
    return out, mag


def exact_mx(A, a_e8m0, B, b_e8m0):
    """Exact route-MX result as Fractions [M][N] plus sum of |terms|."""
    M, K = A.shape
    N = B.shape[0]
    G = K // 32
    ai = e4m3_int(A)
    bi = e4m3_int(B)
    sums = [ai[:, g * 32:(g + 1) * 32] @ bi[:, g * 32:(g + 1) * 32].T for g in range(G)]
    out = [[None] * N for _ in range(M)]
    mag = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            ab = Fraction(0)
            for g in range(G):
                ex = int(a_e8m0[m, g]) + int(b_e8m0[n, g]) - 254 - 18
                t = int(sums[g][m, n]) * (Fraction(2) ** ex)
                tot += t
                ab += abs(t)
            out[m][n] = tot
            mag[m][n] = ab
    return out, mag


def compare_exact(acc, bits, exact, mag, n_blocks):
    """Oracle (fp64 sums, bf16 bits) against the exact result: fp64 error within the
    n_blocks-term summation bound, bf16 bits identical except where a tie sits inside it."""
    M, N = len(exact), len(exact[0])
    skipped = 0
    for m in range(M):
        for n in range(N):
            ex = exact[m][n]
            bound = mag[m][n] * Fraction(2 * (n_blocks + 1), 2 ** 53)
            err = abs(Fraction(float(acc[m, n])) - ex)
            assert err <= bound, f"fp64 sum off at ({m},{n}): {float(acc[m, n])} vs {float(ex)}"
            want = exact_bf16_bits(ex)
            if int(bits[m, n]) != want:
                assert bf16_neighbourhood_tie(ex, bound), \
                    f"bf16 bits differ at ({m},{n}): {int(bits[m, n]):#06x} vs {want:#06x}"
                skipped += 1
    assert skipped <= max(1, M * N // 1000)


def special_codes(rng, shape):
    """Random e4m3 codes mixing ordinary values with +-0, subnormals, +-448 (no NaN)."""
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E  # no NaN: replace by 448 of the same sign
    special = np.array([0x00, 0x80, 0x01, 0x81, 0x07, 0x87, 0x7E, 0xFE, 0x38, 0xB8], np.uint8)
    mask = rng.random(shape) < 0.2
    c[mask] = rng.choice(special, size=int(mask.sum()))
    return c


def random_fp32_scales(rng, shape):
    """Positive fp32 scales with arbitrary mantissas over a range of binades."""
    return (rng.uniform(0.5, 1.0, size=shape) * np.exp2(rng.integers(-12, 4, size=shape))).astype(np.float32)


# -------------------------------------------------------------------------------------
# Pins
# -------------------------------------------------------------------------------------


def pin_e4m3_decode(o):
    """All 256 codes decode as torch's float8_e4m3fn does (NaN codes to NaN)."""
    want = torch_e4m3_values()
    got = o.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def pin_e8m0_decode(o):
    """All 256 ue8m0 bytes decode as torch's float8_e8m0fnu does."""
    want = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu)
    want = want.to(torch.float64).numpy()
    got = o.e8m0_decode(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def pin_bf16_round_fp32_exact(o, seed=0):
    """fp32-exact inputs round as torch's fp32 -> bf16 conversion does, including
    constructed ties, subnormals, the overflow boundary and signed zeros."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, size=4000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # ties: bf16 value +- half a bf16 ulp, for odd and even mantissas, normal and subnormal
    base = rng.integers(0, 2 ** 16, size=2000, dtype=np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    near = np.concatenate([(base | 0x7FFF).view(np.float32), (base | 0x8001).view(np.float32)])
    extra = np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 3.4028235e38, -3.4028235e38,
                      1e-40, -1e-40, 1.4e-45, 9.2e-41, 1.1754942e-38], dtype=np.float32)
    x = np.concatenate([x, ties, near, extra])
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]


def pin_bf16_round_exact(o, seed=1):
    """Inputs that are not fp32-exact (one rounding from fp64, never via fp32) round as the
    exact rational half-to-even rounding does."""
    rng = np.random.default_rng(seed)
    vals = []
    for _ in range(600):
        b = int(rng.integers(0, 0x7F7F)) << 16  # a finite bf16 pattern
        v = float(np.array([b], np.uint32).view(np.float32)[0])
        if v == 0.0:
            continue
        ulp = abs(np.spacing(np.float32(v))) * 2.0 ** 16 if v else 2.0 ** -133
        # just below / at / just above the midpoint to the next bf16, in fp64 resolution
        for off in (0.5 - 2.0 ** -30, 0.5, 0.5 + 2.0 ** -30, 0.25, 0.75):
            vals.append(v + off * ulp)
            vals.append(-(v + off * ulp))
    vals += [2.0 ** -134, 2.0 ** -134 * (1 + 2.0 ** -40), 3 * 2.0 ** -134, 2.0 ** -140,
             (2 - 2.0 ** -8) * 2.0 ** 127, (2 - 2.0 ** -8) * 2.0 ** 127 * (1 - 2.0 ** -40), 1e300]
    x = np.array(vals, dtype=np.float64)
    got = o.bf16_round(x)
    want = np.array([exact_bf16_bits(Fraction(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want), [(x[i], got[i], want[i]) for i in np.flatnonzero(got != want)[:5]]


def pin_bs_brute_force(o, seed=2, M=5, N=260, K=384):
    """Route BS on random codes (with specials), random fp32 scales and a ragged last
    128-row weight-scale block equals the exact brute force."""
    rng = np.random.default_rng(seed)
    A = special_codes(rng, (M, K))
    B = special_codes(rng, (N, K))
    sa = random_fp32_scales(rng, (M, K // 128))
    sb = random_fp32_scales(rng, ((N + 127) // 128, K // 128))
    acc, bits = o.bs_gemm(A, sa, B, sb)
    exact, mag = exact_bs(A, sa, B, sb)
    compare_exact(acc, bits, exact, mag, K // 128)


def pin_bs_tiny_config_exact(o, seed=0):
    """The whole 128x256x512 workload (seeded, quantised as the bench does) equals the exact
    brute force."""
    x = workload.bs_inputs(128, 256, 512, seed)
    acc, bits = o.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    exact, mag = exact_bs(x.A, x.a_scale, x.B, x.b_scale)
    compare_exact(acc, bits, exact, mag, 4)


def pin_mx_brute_force(o, seed=3, M=6, N=40, K=256):
    """Route MX on random codes and random exponent bytes equals the exact brute force."""
    rng = np.random.default_rng(seed)
    A = special_codes(rng, (M, K))
    B = special_codes(rng, (N, K))
    ea = rng.integers(100, 150, size=(M, K // 32), dtype=np.uint8)
    eb = rng.integers(100, 150, size=(N, K // 32), dtype=np.uint8)
    acc, bits = o.mx_gemm(A, ea, B, eb)
    exact, mag = exact_mx(A, ea, B, eb)
    compare_exact(acc, bits, exact, mag, K // 32)


def pin_closed_form_ones(o):
    """All codes 1.0 (0x38) with unit scales: every output equals K."""
    for K in (128, 512, 7168):
        A = np.full((3, K), 0x38, np.uint8)
        B = np.full((130, K), 0x38, np.uint8)
        acc, bits = o.bs_gemm(A, np.ones((3, K // 128), np.float32), B,
                              np.ones((2, K // 128), np.float32))
        assert np.all(acc == K)
        assert np.all(bits == np.float32(K).view(np.uint32) >> 16)


def pin_closed_form_integers(o, seed=4):
    """Integer-valued codes in {-4..4} with unit scales: C is the int64 matmul, rounded to
    bf16 by torch (the products are fp32-exact)."""
    rng = np.random.default_rng(seed)
    ints = rng.integers(-4, 5, size=(24, 256))
    intb = rng.integers(-4, 5, size=(136, 256))
    A = workload.e4m3_encode(ints.astype(np.float32))
    B = workload.e4m3_encode(intb.astype(np.float32))
    acc, bits = o.bs_gemm(A, np.ones((24, 2), np.float32), B, np.ones((2, 2), np.float32))
    ref = ints @ intb.T
    assert np.array_equal(acc, ref.astype(np.float64))
    want = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, want)


def pin_closed_form_one_hot(o, seed=5):
    """One-hot A rows pick single weight values: C[m,n] = bf16(dec(a) dec(B[n,k_m])
    a_s[m,k_m/128] b_s[n/128,k_m/128]) -- pins the operand and scale indexing."""
    rng = np.random.default_rng(seed)
    M, N, K = 8, 384, 512
    A = np.zeros((M, K), np.uint8)
    ks = rng.integers(0, K, size=M)
    av = special_codes(rng, (M,))
    av[av == 0] = 0x40
    A[np.arange(M), ks] = av
    B = special_codes(rng, (N, K))
    sa = random_fp32_scales(rng, (M, K // 128))
    sb = random_fp32_scales(rng, (N // 128, K // 128))
    _, bits = o.bs_gemm(A, sa, B, sb)
    vals = torch_e4m3_values()
    for m in range(M):
        k = ks[m]
        for n in range(0, N, 7):
            v = (Fraction(vals[av[m]]) * Fraction(vals[B[n, k]]) * Fraction(float(sa[m, k // 128]))
                 * Fraction(float(sb[n // 128, k // 128])))
            assert int(bits[m, n]) == exact_bf16_bits(v), (m, n)


def pin_closed_form_pow2_block_scales(o, seed=6):
    """Per-K-block power-of-two scales 2^j constant over rows and columns: C = sum_kb
    2^j_kb P_kb with P_kb the integer block products (exact)."""
    rng = np.random.default_rng(seed)
    M, N, K = 6, 256, 512
    A = special_codes(rng, (M, K))
    B = special_codes(rng, (N, K))
    j = rng.integers(-6, 7, size=K // 128)
    sa = np.tile(np.exp2(j).astype(np.float32), (M, 1))
    sb = np.ones((N // 128, K // 128), np.float32)
    acc, bits = o.bs_gemm(A, sa, B, sb)
    ai, bi = e4m3_int(A), e4m3_int(B)
    for m in range(M):
        for n in range(N):
            v = sum(Fraction(int(ai[m, kb * 128:(kb + 1) * 128] @ bi[n, kb * 128:(kb + 1) * 128]), 2 ** 18)
                    * Fraction(2) ** int(j[kb]) for kb in range(K // 128))
            assert Fraction(float(acc[m, n])) == v
            assert int(bits[m, n]) == exact_bf16_bits(v)


def pin_invariant_scale_doubling(o, seed=7):
    """Doubling every a_scale doubles C bitwise; doubling one a_scale[m,kb] moves row m by
    exactly that block's contribution (and leaves other rows untouched)."""
    x = workload.bs_inputs(16, 256, 512, seed)
    acc, bits = o.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    acc2, bits2 = o.bs_gemm(x.A, x.a_scale * np.float32(2), x.B, x.b_scale)
    assert np.array_equal(acc2, 2 * acc)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f(bits2), 2 * f(bits))
    m, kb = 3, 2
    sa = x.a_scale.copy()
    sa[m, kb] *= 2
    acc3, _ = o.bs_gemm(x.A, sa, x.B, x.b_scale)
    other = np.arange(16) != m
    assert np.array_equal(acc3[other], acc[other])
    ai, bi = e4m3_int(x.A), e4m3_int(x.B)
    p = ai[m, kb * 128:(kb + 1) * 128] @ bi[:, kb * 128:(kb + 1) * 128].T / 2.0 ** 18
    contrib = p * float(x.a_scale[m, kb]) * x.b_scale[np.arange(256) // 128, kb].astype(np.float64)
    scale = np.abs(acc[m]) + np.abs(contrib) + 1e-300
    assert np.all(np.abs(acc3[m] - acc[m] - contrib) <= 1e-14 * scale)


def pin_invariant_permutations(o, seed=8):
    """Permuting rows of A (with their scales) permutes rows of C bitwise; permuting the
    K blocks (A and B columns with the scale columns) leaves C unchanged to fp64 rounding."""
    x = workload.bs_inputs(12, 256, 512, seed)
    acc, bits = o.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    perm = np.random.default_rng(seed).permutation(12)
    accp, bitsp = o.bs_gemm(x.A[perm], x.a_scale[perm], x.B, x.b_scale)
    assert np.array_equal(accp, acc[perm]) and np.array_equal(bitsp, bits[perm])
    kp = np.array([2, 0, 3, 1])
    cols = np.concatenate([np.arange(k * 128, (k + 1) * 128) for k in kp])
    acck, _ = o.bs_gemm(x.A[:, cols], x.a_scale[:, kp], x.B[:, cols], x.b_scale[:, kp])
    ai, bi = e4m3_int(x.A), e4m3_int(x.B)
    mag = sum(np.abs(ai[:, kb * 128:(kb + 1) * 128] @ bi[:, kb * 128:(kb + 1) * 128].T) / 2.0 ** 18
              * x.a_scale[:, kb:kb + 1].astype(np.float64)
              * x.b_scale[np.arange(256) // 128, kb].astype(np.float64) for kb in range(4))
    assert np.all(np.abs(acck - acc) <= 2.0 ** -49 * mag)


def pin_invariant_zero_block(o, seed=9):
    """A zero scale on one K block equals deleting that K block."""
    x = workload.bs_inputs(8, 256, 512, seed)
    sa = x.a_scale.copy()
    sa[:, 1] = 0
    acc, bits = o.bs_gemm(x.A, sa, x.B, x.b_scale)
    keep = np.r_[0:128, 256:512]
    acc2, bits2 = o.bs_gemm(x.A[:, keep], x.a_scale[:, [0, 2, 3]], x.B[:, keep], x.b_scale[:, [0, 2, 3]])
    assert np.array_equal(acc, acc2) and np.array_equal(bits, bits2)


def pin_invariant_cross_route(o, seed=10):
    """BS with power-of-two scales equals MX with the same exponents broadcast over the
    four 32-groups of each block and over the 128 weight rows of each block."""
    rng = np.random.default_rng(seed)
    M, N, K = 10, 256, 384
    A = special_codes(rng, (M, K))
    B = special_codes(rng, (N, K))
    ea = rng.integers(110, 140, size=(M, K // 128))
    eb = rng.integers(110, 140, size=(N // 128, K // 128))
    sa = np.exp2(ea - 127.0).astype(np.float32)
    sb = np.exp2(eb - 127.0).astype(np.float32)
    acc, bits = o.bs_gemm(A, sa, B, sb)
    ea32 = np.repeat(ea, 4, axis=1).astype(np.uint8)
    eb32 = np.repeat(np.repeat(eb, 128, axis=0), 4, axis=1).astype(np.uint8)
    acc2, bits2 = o.mx_gemm(A, ea32, B, eb32)
    ai, bi = e4m3_int(A), e4m3_int(B)
    mag = sum(np.abs(ai[:, g * 32:(g + 1) * 32] @ bi[:, g * 32:(g + 1) * 32].T) / 2.0 ** 18
              * np.exp2(ea[:, g // 4:g // 4 + 1] - 127.0)
              * np.exp2(eb[np.arange(N) // 128, g // 4] - 127.0) for g in range(K // 32))
    assert np.all(np.abs(acc2 - acc) <= 2.0 ** -48 * mag)
    assert np.mean(bits == bits2) > 0.999


def pin_invariant_mx_unit_and_lossless(o, seed=11):
    """MX with every exponent byte 127 is the plain fp8 GEMM (integer matmul times 2^-18);
    adding one to every A exponent doubles C bitwise (power-of-two scaling is lossless)."""
    rng = np.random.default_rng(seed)
    M, N, K = 7, 48, 256
    A = special_codes(rng, (M, K))
    B = special_codes(rng, (N, K))
    ea = np.full((M, K // 32), 127, np.uint8)
    eb = np.full((N, K // 32), 127, np.uint8)
    acc, _ = o.mx_gemm(A, ea, B, eb)
    ref = (e4m3_int(A) @ e4m3_int(B).T).astype(np.float64) / 2.0 ** 18
    assert np.array_equal(acc, ref)
    ea2 = rng.integers(100, 140, size=(M, K // 32), dtype=np.uint8)
    acc1, bits1 = o.mx_gemm(A, ea2, B, eb)
    acc2, bits2 = o.mx_gemm(A, ea2 + 1, B, eb)
    assert np.array_equal(acc2, 2 * acc1)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f(bits2), 2 * f(bits1))


def exact_pt(A, a_scale, B, b_scale):
    """Exact route-PT result as Fractions [M][N] plus |value| (one rounding in the oracle)."""
    ai = e4m3_int(A)
    bi = e4m3_int(B)
    dots = ai @ bi.T  # int64, exact (|dot| < K * 2^36)
    M, N = dots.shape
    two18 = Fraction(1, 2 ** 18)
    sa = [Fraction(float(v)) for v in a_scale]
    sb = [Fraction(float(v)) for v in b_scale]
    out = [[int(dots[m, n]) * two18 * sa[m] * sb[n] for n in range(N)] for m in range(M)]
    mag = [[abs(v) for v in row] for row in out]
    return out, mag


def pin_pt_brute_force(o, seed=12, M=5, N=70, K=384):
    """Route PT on random codes (with specials) and random fp32 row scales equals the exact
    brute force (a single rounding before the bf16 one)."""
    rng = np.random.default_rng(seed)
    A = special_codes(rng, (M, K))
    B = special_codes(rng, (N, K))
    sa = random_fp32_scales(rng, (M,))
    sb = random_fp32_scales(rng, (N,))
    acc, bits = o.pt_gemm(A, sa, B, sb)
    exact, mag = exact_pt(A, sa, B, sb)
    compare_exact(acc, bits, exact, mag, 1)


def pin_pt_inputs_exact(o, seed=0):
    """A seeded per-token / per-channel quantised 64x96x512 problem equals the exact brute
    force."""
    x = workload.pt_inputs(64, 96, 512, seed)
    acc, bits = o.pt_gemm(x.A, x.a_scale, x.B, x.b_scale)
    exact, mag = exact_pt(x.A, x.a_scale, x.B, x.b_scale)
    compare_exact(acc, bits, exact, mag, 1)


def pin_pt_closed_form_integers(o, seed=13):
    """Integer-valued codes with scales 2 (rows of A) and 1/2 (rows of B): C is the int64
    matmul, rounded to bf16 by torch (fp32-exact)."""
    rng = np.random.default_rng(seed)
    ints = rng.integers(-4, 5, size=(9, 384))
    intb = rng.integers(-4, 5, size=(40, 384))
    A = workload.e4m3_encode(ints.astype(np.float32))
    B = workload.e4m3_encode(intb.astype(np.float32))
    acc, bits = o.pt_gemm(A, np.full(9, 2.0, np.float32), B, np.full(40, 0.5, np.float32))
    ref = ints @ intb.T
    assert np.array_equal(acc, ref.astype(np.float64))
    want = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, want)


def pin_pt_cross_route_bs(o, seed=14):
    """PT with power-of-two row scales, the weight scales constant inside each 128-row block,
    equals route BS with those scales broadcast over the K blocks, bit for bit (every term is
    then exact in both)."""
    rng = np.random.default_rng(seed)
    M, N, K = 6, 256, 512
    A = special_codes(rng, (M, K))
    B = special_codes(rng, (N, K))
    ea = rng.integers(110, 140, size=M)
    eb = rng.integers(110, 140, size=N // 128)
    sa = np.exp2(ea - 127.0).astype(np.float32)
    sb_blocks = np.exp2(eb - 127.0).astype(np.float32)
    sb = np.repeat(sb_blocks, 128)
    acc, bits = o.pt_gemm(A, sa, B, sb)
    KB = K // 128
    acc2, bits2 = o.bs_gemm(A, np.repeat(sa[:, None], KB, axis=1), B, np.repeat(sb_blocks[:, None], KB, axis=1))
    assert np.array_equal(acc, acc2) and np.array_equal(bits, bits2)


def pin_pt_scale_linearity(o, seed=15):
    """Scaling a_s[m] or b_s[n] by a power of two scales exactly that row or column of C
    (bitwise, away from overflow); the other outputs are unchanged."""
    rng = np.random.default_rng(seed)
    M, N, K = 6, 50, 256
    A = special_codes(rng, (M, K))
    B = special_codes(rng, (N, K))
    sa = random_fp32_scales(rng, (M,))
    sb = random_fp32_scales(rng, (N,))
    acc, bits = o.pt_gemm(A, sa, B, sb)
    sa2 = sa.copy()
    sa2[2] *= 4
    sb2 = sb.copy()
    sb2[7] *= 0.5
    acc2, bits2 = o.pt_gemm(A, sa2, B, sb2)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    expect = f(bits).copy()
    expect[2, :] *= 4
    expect[:, 7] *= 0.5
    assert np.array_equal(f(bits2), expect)
    assert np.array_equal(acc2[np.ix_([0, 1, 3, 4, 5], [c for c in range(N) if c != 7])],
                          acc[np.ix_([0, 1, 3, 4, 5], [c for c in range(N) if c != 7])])


def _torch_e4m3(x):
    """torch's fp32 -> float8_e4m3fn cast (round to nearest even) of values clipped to +-448."""
    t = torch.from_numpy(np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_encode_vs_torch(o, seed=16):
    """The oracle's e4m3 encoder agrees with torch's cast on random values over the whole
    range, on every e4m3 value, on every midpoint between neighbours (ties) and just off them,
    on the subnormal range and beyond 448 (saturation)."""
    rng = np.random.default_rng(seed)
    vals = torch_e4m3_values()
    fin = np.sort(np.unique(np.abs(vals[np.isfinite(vals)])))
    mids = (fin[1:] + fin[:-1]) / 2
    xs = np.concatenate([
        rng.uniform(-460, 460, 3000), rng.standard_normal(2000) * np.exp2(rng.integers(-12, 9, 2000)),
        fin, -fin, mids, -mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
        np.nextafter(mids.astype(np.float32), np.float32(1000)), [448.0, 449.0, 464.0, 1e6, -1e6, 0.0, -0.0],
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 1000)]).astype(np.float32)
    xs = np.concatenate([xs, np.array([np.nan, -np.nan], np.float32)])
    got = np.array([o.e4m3_encode(v) for v in xs], dtype=np.uint8)
    want = _torch_e4m3(xs)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(xs[i]), int(got[i]), int(want[i])) for i in bad[:5]]


def _quant_input(rng, M, K):
    """Gaussian rows plus rows that stress the quantiser: all zero, one large value, tiny
    values, exact e4m3 values scaled by powers of two."""
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[1] = 0
    x[2] = rng.standard_normal(K).astype(np.float32) * np.float32(2.0 ** -20)
    x[3, 5] = 3.0e5
    vals = torch_e4m3_values()
    fin = vals[np.isfinite(vals)]
    x[4] = (rng.choice(fin, K) * 2.0 ** 7).astype(np.float32)
    x[5, :] = -1.0
    return x


def pin_quantize_bs_vs_recipe(o, seed=17):
    """Route-BS activation quantiser equals the seeded input recipe (an independent numpy /
    torch implementation of the same definition), bit for bit."""
    rng = np.random.default_rng(seed)
    x = _quant_input(rng, 40, 512)
    codes, scale = o.quantize_bs(x)
    c2, s2 = workload.quantize_groups_fp32(x, 1, 128)
    assert np.array_equal(scale.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(codes, c2)


def pin_quantize_mx_vs_recipe(o, seed=18):
    """Route-MX activation quantiser equals the seeded input recipe, bit for bit."""
    rng = np.random.default_rng(seed)
    x = _quant_input(rng, 40, 512)
    codes, e8 = o.quantize_mx(x)
    c2, e2 = workload.quantize_mx(x)
    assert np.array_equal(e8, e2)
    assert np.array_equal(codes, c2)


def pin_quantize_closed_form(o, seed=19):
    """A group holding exact e4m3 values times 2^k with largest magnitude 448 * 2^k has scale
    exactly 2^k (route BS) and exponent k (route MX), and its codes are those values."""
    rng = np.random.default_rng(seed)
    vals = torch_e4m3_values()
    fin_codes = np.array([c for c in range(256) if np.isfinite(vals[c])], dtype=np.uint8)
    M, K = 6, 256
    codes = rng.choice(fin_codes, size=(M, K)).astype(np.uint8)
    codes[:, ::32] = 0x7E  # 448 in every 32-group
    ks = np.array([-5, -1, 0, 2, 7, 12])
    x = (vals[codes] * np.exp2(ks)[:, None]).astype(np.float32)
    c, s = o.quantize_bs(x)
    assert np.array_equal(s, np.repeat(np.exp2(ks)[:, None], K // 128, axis=1).astype(np.float32))
    neg0 = (codes == 0x80)  # -0 and +0 both encode zero; compare values
    assert np.array_equal(np.where(neg0, 0, c), np.where(neg0, 0, codes))
    c, e8 = o.quantize_mx(x)
    assert np.array_equal(e8.astype(int) - 127, np.repeat(ks[:, None], K // 32, axis=1))
    assert np.array_equal(np.where(neg0, 0, c), np.where(neg0, 0, codes))


def pin_quantize_mx_exponent_minimal(o, seed=20):
    """Every MX exponent is the smallest that keeps the group within 448 * 2^e (or the clamp)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((30, 256)) * np.exp2(rng.integers(-30, 30, size=(30, 1)))).astype(np.float32)
    _, e8 = o.quantize_mx(x)
    amax = np.abs(x.reshape(30, 8, 32)).max(axis=2).astype(np.float64)
    e = e8.astype(np.int64) - 127
    assert np.all(amax <= np.ldexp(448.0, e))
    assert np.all((e == -127) | (amax > np.ldexp(448.0, e - 1)))


ALL_PINS = [
    pin_e4m3_decode, pin_e8m0_decode, pin_bf16_round_fp32_exact, pin_bf16_round_exact,
    pin_bs_brute_force, pin_bs_tiny_config_exact, pin_mx_brute_force, pin_closed_form_ones,
    pin_closed_form_integers, pin_closed_form_one_hot, pin_closed_form_pow2_block_scales,
    pin_invariant_scale_doubling, pin_invariant_permutations, pin_invariant_zero_block,
    pin_invariant_cross_route, pin_invariant_mx_unit_and_lossless, pin_pt_brute_force,
    pin_pt_inputs_exact, pin_pt_closed_form_integers, pin_pt_cross_route_bs, pin_pt_scale_linearity,
    pin_e4m3_encode_vs_torch, pin_quantize_bs_vs_recipe, pin_quantize_mx_vs_recipe,
    pin_quantize_closed_form, pin_quantize_mx_exponent_minimal,
]
