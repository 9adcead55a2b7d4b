"""CPU oracle for the fp8 (OCP e4m3) block-scaled GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package. The product library (``fp8_block_scaled_e4m3_amd``) never loads,
links or calls it, and the two share no code: the oracle is ``oracle.c`` (plain C, fp64,
OpenMP over output rows) plus this ctypes wrapper.

What the oracle computes is the definition of the operation (page "Flydsl Fp8 Blockscale
Gemm", Procedure step 1: fp32 dequantise, matmul, round to bf16; page "aiter PR #6370",
"Why it is faster": 1x32 ue8m0 scales are powers of two applied per 32-wide K group):

    BS:  C[m,n] = bf16( sum_kb a_s[m,kb] * b_s[n//128,kb] * sum_{k in kb} A[m,k] B[n,k] )
    MX:  C[m,n] = bf16( sum_g 2^(ea[m,g]-127) 2^(eb[n,g]-127) sum_{k in g} A[m,k] B[n,k] )
    PT:  C[m,n] = bf16( a_s[m] * b_s[n] * sum_k A[m,k] B[n,k] )   (the promote-free twin,
         page "Flydsl Fp8 Blockscale Gemm", Bottleneck diagnosis item 2)

and the activation quantisers that produce the GEMM's inputs (per 1x128 group fp32 scale
amax/448 for route BS; per 1x32 group ue8m0 exponent for route MX; e4m3 codes nearest, ties
to even, saturating at 448).

with block sums exact in fp64 and one round-to-nearest-even from fp64 to bf16.

Pins (tests/test_oracle_*.py): e4m3 decode against torch's float8_e4m3fn; ue8m0 decode
against torch's float8_e8m0fnu; bf16 rounding against torch's fp32->bf16 conversion and
against exact rational rounding; the whole GEMM against an exact rational brute force, against
integer-matmul closed forms and against scale invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_c_int_p = ctypes.POINTER(ctypes.c_int)


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fp contraction). Returns the path."""
    tmp = output + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c11",
         "-Wall", "-Wextra", "-o", tmp, source, "-lm"],
        check=True,
    )
    os.replace(tmp, output)
    return output


class Oracle:
    """ctypes handle on one compiled copy of the oracle (tests may load a mutated copy)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library not built: {path}")
        self.path = path
        lib = ctypes.CDLL(path)
        for name in ("oracle_bs_gemm", "oracle_mx_gemm", "oracle_pt_gemm"):
            fn = getattr(lib, name)
            fn.restype = None
            fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_int, ctypes.c_int, ctypes.c_int,
                           _c_int_p, ctypes.c_int, _c_int_p, ctypes.c_int,
                           ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        for name in ("oracle_quantize_bs", "oracle_quantize_mx"):
            fn = getattr(lib, name)
            fn.restype = None
            fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_e8m0_decode.restype = ctypes.c_double
        lib.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_bf16_round.argtypes = [ctypes.c_double]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        self.lib = lib

    # -- codecs ------------------------------------------------------------------------
    def e4m3_decode(self, codes) -> np.ndarray:
        codes = np.asarray(codes, dtype=np.uint8)
        return np.array([self.lib.oracle_e4m3_decode(int(c)) for c in codes.ravel()],
                        dtype=np.float64).reshape(codes.shape)

    def e8m0_decode(self, codes) -> np.ndarray:
        codes = np.asarray(codes, dtype=np.uint8)
        return np.array([self.lib.oracle_e8m0_decode(int(c)) for c in codes.ravel()],
                        dtype=np.float64).reshape(codes.shape)

    def bf16_round(self, x) -> np.ndarray:
        """fp64 -> bf16 bit patterns (uint16), round-to-nearest-even, one rounding."""
        x = np.asarray(x, dtype=np.float64)
        return np.array([self.lib.oracle_bf16_round(float(v)) for v in x.ravel()],
                        dtype=np.uint16).reshape(x.shape)

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    # -- GEMMs -------------------------------------------------------------------------
    @staticmethod
    def _grid(n_total: int, idx):
        if idx is None:
            idx = np.arange(n_total, dtype=np.int32)
        idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
        if idx.size and (idx.min() < 0 or idx.max() >= n_total):
            raise IndexError("sample index out of range")
        return idx

    def _run(self, fn, A, sa, B, sb, M, N, K, rows, cols):
        rows = self._grid(M, rows)
        cols = self._grid(N, cols)
        acc = np.empty((rows.size, cols.size), dtype=np.float64)
        bits = np.empty((rows.size, cols.size), dtype=np.uint16)
        fn(A.ctypes.data, sa.ctypes.data, B.ctypes.data, sb.ctypes.data, M, N, K,
           rows.ctypes.data_as(_c_int_p), rows.size, cols.ctypes.data_as(_c_int_p), cols.size,
           acc.ctypes.data, bits.ctypes.data)
        return acc, bits

    def e4m3_encode(self, x: float) -> int:
        return int(self.lib.oracle_e4m3_encode(float(x)))

    def quantize_bs(self, x):
        """Activation quantiser, route BS: x [M,K] fp32 -> (codes uint8 [M,K], scales fp32
        [M,K/128], logical a_s[m,kb])."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        M, K = x.shape
        if K % 128:
            raise ValueError("K must be a multiple of 128")
        codes = np.empty((M, K), np.uint8)
        scale = np.empty((M, K // 128), np.float32)
        self.lib.oracle_quantize_bs(x.ctypes.data, M, K, codes.ctypes.data, scale.ctypes.data)
        return codes, scale

    def quantize_mx(self, x):
        """Activation quantiser, route MX: x [M,K] fp32 -> (codes uint8 [M,K], ue8m0 bytes
        uint8 [M,K/32])."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        M, K = x.shape
        if K % 32:
            raise ValueError("K must be a multiple of 32")
        codes = np.empty((M, K), np.uint8)
        e8 = np.empty((M, K // 32), np.uint8)
        self.lib.oracle_quantize_mx(x.ctypes.data, M, K, codes.ctypes.data, e8.ctypes.data)
        return codes, e8

    def bs_gemm(self, A, a_scale, B, b_scale, rows=None, cols=None):
        """Route BS. A [M,K] and B [N,K] uint8 e4m3 codes; a_scale [M,K/128] fp32 (logical
        a_s[m,kb]); b_scale [ceil(N/128),K/128] fp32. Returns (fp64 sums, bf16 bits) on the
        grid rows x cols (all rows/cols when None)."""
        A = np.ascontiguousarray(A, dtype=np.uint8)
        B = np.ascontiguousarray(B, dtype=np.uint8)
        M, K = A.shape
        N = B.shape[0]
        if B.shape[1] != K or K % 128:
            raise ValueError("bad K")
        KB = K // 128
        a_scale = np.ascontiguousarray(a_scale, dtype=np.float32)
        b_scale = np.ascontiguousarray(b_scale, dtype=np.float32)
        if a_scale.shape != (M, KB) or b_scale.shape != ((N + 127) // 128, KB):
            raise ValueError("bad scale shape")
        return self._run(self.lib.oracle_bs_gemm, A, a_scale, B, b_scale, M, N, K, rows, cols)

    def mx_gemm(self, A, a_e8m0, B, b_e8m0, rows=None, cols=None):
        """Route MX. A [M,K], B [N,K] uint8 e4m3 codes; a_e8m0 [M,K/32], b_e8m0 [N,K/32]
        uint8 biased exponents. Returns (fp64 sums, bf16 bits)."""
        A = np.ascontiguousarray(A, dtype=np.uint8)
        B = np.ascontiguousarray(B, dtype=np.uint8)
        M, K = A.shape
        N = B.shape[0]
        if B.shape[1] != K or K % 32:
            raise ValueError("bad K")
        a_e8m0 = np.ascontiguousarray(a_e8m0, dtype=np.uint8)
        b_e8m0 = np.ascontiguousarray(b_e8m0, dtype=np.uint8)
        if a_e8m0.shape != (M, K // 32) or b_e8m0.shape != (N, K // 32):
            raise ValueError("bad scale shape")
        return self._run(self.lib.oracle_mx_gemm, A, a_e8m0, B, b_e8m0, M, N, K, rows, cols)


    def pt_gemm(self, A, a_scale, B, b_scale, rows=None, cols=None):
        """Route PT (promote-free twin). A [M,K], B [N,K] uint8 e4m3 codes; a_scale [M] and
        b_scale [N] fp32 (one per row of A / of B). Returns (fp64 values, bf16 bits)."""
        A = np.ascontiguousarray(A, dtype=np.uint8)
        B = np.ascontiguousarray(B, dtype=np.uint8)
        M, K = A.shape
        N = B.shape[0]
        if B.shape[1] != K:
            raise ValueError("bad K")
        a_scale = np.ascontiguousarray(a_scale, dtype=np.float32).reshape(-1)
        b_scale = np.ascontiguousarray(b_scale, dtype=np.float32).reshape(-1)
        if a_scale.shape != (M,) or b_scale.shape != (N,):
            raise ValueError("bad scale shape")
        return self._run(self.lib.oracle_pt_gemm, A, a_scale, B, b_scale, M, N, K, rows, cols)


_default: Oracle | None = None


def load(build_if_missing: bool = True) -> Oracle:
    """The oracle built from oracle.c in this directory (compiled first if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            if not build_if_missing:
                raise FileNotFoundError(LIBRARY)
            build()
        _default = Oracle(LIBRARY)
    return _default


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
