"""Seeded synthetic inputs for the fp8 block-scaled GEMM, shared by the tests, the bench
and the smoke check.

This module generates and quantises operands; it holds none of the GEMM's arithmetic and
is imported by both the oracle side and the GPU side so that both consume the same bytes.

Recipe (the workloads of page "Flydsl Fp8 Blockscale Gemm", "When to use" table, with
synthetic values standing in for the model activations and weights measured there):

* ``rng = numpy.random.default_rng(seed)``; ``A = rng.standard_normal((M, K), float32)``,
  then ``B = 0.02 * rng.standard_normal((N, K), float32)``, drawn in that order.
* Route BS: A is quantised per 1x128 group along K and B per 128x128 block, each with the
  fp32 scale ``s = amax / 448`` (``s = 1`` when the group is all zero) and codes
  ``e4m3_rne_saturate(x / s)``.
* Route MX: A and B are quantised per 1x32 group along K with a ue8m0 exponent ``e``, the
  smallest integer with ``amax <= 448 * 2^e`` (clamped to [-127, 127]; byte ``e + 127``;
  byte 127 when the group is all zero), and codes ``e4m3_rne_saturate(x * 2^-e)``.

* Route PT (the promote-free twin): A and B are quantised per whole row with the fp32 scale
  ``s = amax / 448`` of the row.

The e4m3 encoder is torch's fp32 -> float8_e4m3fn conversion (round to nearest even) applied
after clamping to +-448.

Workloads (``CONFIGS``): the four shapes of that table (narrow-N 4096x2048x7168, K-light
16384x7168x768, wide-N 4096x65536x1536 and the page's untuned narrow-N deep-K shape
16384x1536x7168) plus the tiny 128x256x512 case and one eighth of wide-N along N
(4096x8192x1536) (route BS), and the mxfp8 16384x8192x1280 and 16384x5120x2048 cases of page
"aiter PR #6370" (route MX).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

E4M3_MAX = 448.0

# The workloads the bench and the parity tests use, as (M, N, K) and route.
CONFIGS = {
    "tiny": dict(M=128, N=256, K=512, route="bs"),
    "narrow_n": dict(M=4096, N=2048, K=7168, route="bs"),
    "k_light": dict(M=16384, N=7168, K=768, route="bs"),
    "wide_n": dict(M=4096, N=65536, K=1536, route="bs"),
    "mxfp8": dict(M=16384, N=8192, K=1280, route="mx"),
    # a second narrow-N, deep-K shape of the same class as narrow_n, untuned on the pages
    "narrow_n_16k": dict(M=16384, N=1536, K=7168, route="bs"),
    # the mxfp8 shape with the highest throughput on page "aiter PR #6370" (same FLOPs as mxfp8)
    "mxfp8_k2048": dict(M=16384, N=5120, K=2048, route="mx"),
    # one GPU's share of wide_n split eight ways along N (weights sharded, activations replicated)
    "wide_n_shard8": dict(M=4096, N=8192, K=1536, route="bs"),
}


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3 codes (uint8), round to nearest even, saturating at +-448."""
    t = torch.from_numpy(np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def draw(M: int, N: int, K: int, seed: int):
    """The raw fp32 operands: A ~ N(0,1) [M,K], B ~ N(0,0.02^2) [N,K]."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K), dtype=np.float32)
    B = (np.float32(0.02) * rng.standard_normal((N, K), dtype=np.float32)).astype(np.float32)
    return A, B


def quantize_groups_fp32(x: np.ndarray, rows: int, cols: int):
    """Quantise x [R, C] in blocks of rows x cols with fp32 scale amax/448.

    Returns (codes uint8 [R, C], scales fp32 [ceil(R/rows), C/cols])."""
    R, C = x.shape
    if C % cols:
        raise ValueError("columns must divide into groups")
    Rp = -(-R // rows) * rows
    xp = x if Rp == R else np.concatenate([x, np.zeros((Rp - R, C), np.float32)])
    blocks = xp.reshape(Rp // rows, rows, C // cols, cols)
    amax = np.abs(blocks).max(axis=(1, 3)).astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    q = blocks / scale[:, None, :, None]
    codes = e4m3_encode(q.reshape(Rp, C).astype(np.float32))[:R]
    return np.ascontiguousarray(codes), np.ascontiguousarray(scale)


def e8m0_exponents(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e (exact), clamped to [-127, 127];
    0 for all-zero groups."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    # Correct any off-by-one of the floating log2 with exact power-of-two comparisons.
    e = np.where(safe > np.ldexp(E4M3_MAX, e), e + 1, e)
    e = np.where(safe <= np.ldexp(E4M3_MAX, e - 1), e - 1, e)
    e = np.where(amax > 0, e, 0)
    return np.clip(e, -127, 127)


def quantize_mx(x: np.ndarray, group: int = 32):
    """Quantise x [R, C] per 1 x group with ue8m0 scales.

    Returns (codes uint8 [R, C], e8m0 bytes uint8 [R, C/group])."""
    R, C = x.shape
    if C % group:
        raise ValueError("columns must divide into groups")
    g = x.reshape(R, C // group, group)
    e = e8m0_exponents(np.abs(g).max(axis=2))
    q = np.ldexp(g.astype(np.float64), -e[:, :, None]).astype(np.float32)  # exact scaling
    codes = e4m3_encode(q.reshape(R, C))
    return np.ascontiguousarray(codes), np.ascontiguousarray((e + 127).astype(np.uint8))


@dataclass
class BSInputs:
    M: int
    N: int
    K: int
    A: np.ndarray        # uint8 [M, K] e4m3 codes
    a_scale: np.ndarray  # float32 [M, K/128]   logical a_s[m, kb]
    B: np.ndarray        # uint8 [N, K] e4m3 codes
    b_scale: np.ndarray  # float32 [N/128, K/128]

    @property
    def a_scale_kmajor(self) -> np.ndarray:
        """a_scale laid out K-block-major, [K/128, M] contiguous (the library's layout)."""
        return np.ascontiguousarray(self.a_scale.T)


@dataclass
class MXInputs:
    M: int
    N: int
    K: int
    A: np.ndarray        # uint8 [M, K]
    a_e8m0: np.ndarray   # uint8 [M, K/32]
    B: np.ndarray        # uint8 [N, K]
    b_e8m0: np.ndarray   # uint8 [N, K/32]


def bs_inputs(M: int, N: int, K: int, seed: int = 0) -> BSInputs:
    """Route-BS operands: A per-1x128, B per-128x128, fp32 scales amax/448."""
    A, B = draw(M, N, K, seed)
    qa, sa = quantize_groups_fp32(A, 1, 128)
    del A
    qb, sb = quantize_groups_fp32(B, 128, 128)
    return BSInputs(M, N, K, qa, sa, qb, sb)


def mx_inputs(M: int, N: int, K: int, seed: int = 0) -> MXInputs:
    """Route-MX operands: A and B per-1x32 with ue8m0 exponents."""
    A, B = draw(M, N, K, seed)
    qa, ea = quantize_mx(A)
    del A
    qb, eb = quantize_mx(B)
    return MXInputs(M, N, K, qa, ea, qb, eb)


@dataclass
class PTInputs:
    """Route PT: one fp32 scale per row of A (per token) and per row of B (per channel)."""
    A: np.ndarray        # [M, K] uint8 e4m3 codes
    a_scale: np.ndarray  # [M] fp32
    B: np.ndarray        # [N, K] uint8 e4m3 codes
    b_scale: np.ndarray  # [N] fp32


def pt_inputs(M: int, N: int, K: int, seed: int = 0) -> PTInputs:
    """Route-PT operands: A and B quantised per whole row with fp32 scale amax/448."""
    a, b = draw(M, N, K, seed)
    A, sa = quantize_groups_fp32(a, 1, K)
    B, sb = quantize_groups_fp32(b, 1, K)
    return PTInputs(A, np.ascontiguousarray(sa.reshape(M)), B, np.ascontiguousarray(sb.reshape(N)))


def tiled_bs_inputs(M: int, N: int, K: int, seed: int = 0, row_period: int = 8191,
                    block_period: int = 67) -> BSInputs:
    """Route-BS operands at sizes whose fp32 draw would not fit in host memory (M * K or N * K
    near 2^31): the rows of A repeat with period `row_period` and the 128-row weight blocks
    with period `block_period`, each period drawn and quantised as in bs_inputs, with the scales
    repeating along. Both periods are odd, so a read displaced by a power-of-two number of
    bytes lands on different data."""
    rows_a = min(M, row_period)
    blocks_b = min(N // 128, block_period)
    a, b = draw(rows_a, blocks_b * 128, K, seed)
    qa, sa = quantize_groups_fp32(a, 1, 128)
    qb, sb = quantize_groups_fp32(b, 128, 128)
    del a, b
    reps_a = -(-M // rows_a)
    A = np.tile(qa, (reps_a, 1))[:M]
    a_scale = np.tile(sa, (reps_a, 1))[:M]
    reps_b = -(-(N // 128) // blocks_b)
    B = np.tile(qb, (reps_b, 1))[:N]
    b_scale = np.tile(sb, (reps_b, 1))[:N // 128]
    return BSInputs(M, N, K, np.ascontiguousarray(A), np.ascontiguousarray(a_scale), np.ascontiguousarray(B),
                    np.ascontiguousarray(b_scale))


def tiled_mx_inputs(M: int, N: int, K: int, seed: int = 0, row_period: int = 8191) -> MXInputs:
    """Route-MX operands with the rows of A and of B repeating with an odd period (see
    tiled_bs_inputs)."""
    rows_a, rows_b = min(M, row_period), min(N, row_period)
    a, b = draw(rows_a, rows_b, K, seed)
    qa, ea = quantize_mx(a)
    qb, eb = quantize_mx(b)
    del a, b
    ra, rb = -(-M // rows_a), -(-N // rows_b)
    return MXInputs(M, N, K, np.ascontiguousarray(np.tile(qa, (ra, 1))[:M]),
                    np.ascontiguousarray(np.tile(ea, (ra, 1))[:M]),
                    np.ascontiguousarray(np.tile(qb, (rb, 1))[:N]),
                    np.ascontiguousarray(np.tile(eb, (rb, 1))[:N]))


def sample_indices(n_total: int, n_pick: int, seed: int) -> np.ndarray:
    """A seeded, sorted sample of distinct indices that always includes the first and last."""
    if n_pick >= n_total:
        return np.arange(n_total, dtype=np.int32)
    rng = np.random.default_rng(seed + 7919)
    pick = rng.choice(n_total, size=n_pick, replace=False)
    pick[0], pick[-1] = 0, n_total - 1
    return np.unique(pick).astype(np.int32)
