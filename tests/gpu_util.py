"""Helpers for the GPU tests: upload seeded inputs, run a route through the C ABI, compare
with the oracle under the parity bar (|gpu - ref| <= 1e-2 + 1e-2 |ref| elementwise, cosine
similarity >= 0.9999, no NaN/Inf)."""
from __future__ import annotations

import numpy as np
import torch

import oracle as oracle_pkg

ATOL = 1e-2
RTOL = 1e-2
MIN_COS = 0.9999


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bits(C: torch.Tensor) -> np.ndarray:
    return C.view(torch.int16).cpu().numpy().view(np.uint16)


def run_bs(fb, x, C=None):
    """Route BS on workload.BSInputs-like x; returns the bf16 bit patterns of C."""
    A = to_dev(x.A)
    sa = to_dev(np.ascontiguousarray(x.a_scale.T))
    B = to_dev(x.B)
    sb = to_dev(x.b_scale)
    if C is None:
        C = torch.empty((x.A.shape[0], x.B.shape[0]), dtype=torch.bfloat16, device=dev())
    fb.fp8bs_gemm(A, sa, fb.prep_weights(B), sb, C)
    torch.cuda.synchronize()
    return bits(C)


def run_mx(fb, y):
    A = to_dev(y.A)
    pa = fb.mx_pack_a_scale(to_dev(y.a_e8m0))
    Bp, pb = fb.mx_prep_weights(to_dev(y.B), to_dev(y.b_e8m0))
    C = torch.empty((y.A.shape[0], y.B.shape[0]), dtype=torch.bfloat16, device=dev())
    fb.fp8mx_gemm(A, pa, Bp, pb, C)
    torch.cuda.synchronize()
    return bits(C)


def run_pt(fb, z, config=None):
    """Route PT on workload.PTInputs-like z (a_scale [M], b_scale [N]); returns bf16 bits."""
    A = to_dev(z.A)
    sa = to_dev(np.ascontiguousarray(z.a_scale, dtype=np.float32))
    sb = to_dev(np.ascontiguousarray(z.b_scale, dtype=np.float32))
    Bp = fb.prep_weights(to_dev(z.B))
    C = torch.empty((z.A.shape[0], z.B.shape[0]), dtype=torch.bfloat16, device=dev())
    if config is None:
        fb.fp8pt_gemm(A, sa, Bp, sb, C)
    else:
        fb.fp8pt_gemm_with_config(A, sa, Bp, sb, C, config)
    torch.cuda.synchronize()
    return bits(C)


def parity(gpu_bits: np.ndarray, ref_bits: np.ndarray, name: str = "") -> dict:
    g = oracle_pkg.bf16_bits_to_f64(gpu_bits)
    r = oracle_pkg.bf16_bits_to_f64(ref_bits)
    assert g.shape == r.shape
    assert np.all(np.isfinite(g)), f"{name}: {int((~np.isfinite(g)).sum())} non-finite outputs"
    diff = np.abs(g - r)
    bad = diff > ATOL + RTOL * np.abs(r)
    denom = np.linalg.norm(g) * np.linalg.norm(r)
    cos = float(np.dot(g.ravel(), r.ravel()) / denom) if denom > 0 else 1.0
    stats = dict(max_abs=float(diff.max()) if diff.size else 0.0, cos=cos,
                 bit_exact=float(np.mean(gpu_bits == ref_bits)) if diff.size else 1.0,
                 n=int(diff.size), n_bad=int(bad.sum()))
    print(f"parity {name}: {stats}", flush=True)
    assert stats["n_bad"] == 0, f"{name}: {stats}"
    assert cos >= MIN_COS, f"{name}: {stats}"
    return stats
