"""Benchmark of the fp8 block-scaled GEMM on one MI355X.

One step = one fp8bs_gemm launch on the narrow-N, deep-K workload (M=4096, N=2048, K=7168,
route BS: fp32 per-1x128 activation scales, fp32 per-128x128 weight scales, bf16 out), with
every input already resident in HBM. Prints ONE JSON line on stdout:

  value      -- TFLOP/s (2*M*N*K per step / wall time per step) of that workload
  roofline   -- the GEMM kernel's achieved TFLOP/s from HIP events on its own stream,
                against the dense fp8 matrix-core peak (5.0 PFLOP/s); traffic from the
                committed rocprofv3 counter summary when it matches the current kernel source
  per_shape  -- the same measurement for all five workloads (tiny, narrow-N, K-light, wide-N,
                mxfp8) with % of peak and algorithmic HBM GB/s
  cpu_baseline -- the CPU oracle (fp64, OpenMP) on a bounded sample of rows of the workload
  parity     -- sampled rows/columns of the timed output against the oracle

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix-core peak (published), TFLOP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth (published), GB/s
METRIC = "fp8 blockscale GEMM TFLOP/s and % of MI355X dense fp8 MFMA peak, per shape"
MAIN = "narrow_n"
KERNEL_SOURCES = ["gemm.hip", "device.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp8_block_scaled_e4m3_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def algorithmic_bytes(route: str, M: int, N: int, K: int) -> int:
    """A, B, scales and C each moved once."""
    if route == "bs":
        scales = 4 * (M * (K // 128) + (N // 128) * (K // 128))
    else:
        scales = M * (K // 32) + N * (K // 32)
    return M * K + N * K + scales + 2 * M * N


class Case:
    """Device-resident operands of one workload plus a launch closure on a given stream."""

    def __init__(self, name: str, cfg: dict, seed: int, stream):
        import torch

        import fp8_block_scaled_e4m3_amd as fb
        import workload

        self.name, self.route = name, cfg["route"]
        self.M, self.N, self.K = cfg["M"], cfg["N"], cfg["K"]
        dev = torch.device("cuda:0")
        t0 = time.time()
        if self.route == "bs":
            x = workload.bs_inputs(self.M, self.N, self.K, seed)
            self.host = x
            self.A = torch.from_numpy(x.A).to(dev)
            self.sa = torch.from_numpy(x.a_scale_kmajor).to(dev)
            self.B = fb.prep_weights(torch.from_numpy(x.B).to(dev), stream)
            self.sb = torch.from_numpy(x.b_scale).to(dev)
        else:
            y = workload.mx_inputs(self.M, self.N, self.K, seed)
            self.host = y
            self.A = torch.from_numpy(y.A).to(dev)
            self.sa = fb.mx_pack_a_scale(torch.from_numpy(y.a_e8m0).to(dev), stream)
            self.B, self.sb = fb.mx_prep_weights(torch.from_numpy(y.B).to(dev),
                                                 torch.from_numpy(y.b_e8m0).to(dev), stream)
        self.C = torch.empty((self.M, self.N), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        log(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s")
        fn = fb.fp8bs_gemm if self.route == "bs" else fb.fp8mx_gemm
        self.launch = lambda: fn(self.A, self.sa, self.B, self.sb, self.C, stream)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def time_launches(self, steps: int, warmup: int, stream):
        """(wall seconds per launch, event seconds per launch) over `steps` launches."""
        import torch
        for _ in range(warmup):
            self.launch()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            self.launch()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        ev = e0.elapsed_time(e1) / 1e3 / steps
        return wall, ev

    def free(self):
        for k in ("A", "sa", "B", "sb", "C"):
            setattr(self, k, None)


def sampled_parity(case: Case, nrows: int = 16, ncols: int = 16) -> dict:
    import numpy as np

    import oracle
    import workload
    o = oracle.load()
    got = case.C.view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    rows = workload.sample_indices(case.M, nrows, 100)
    cols = workload.sample_indices(case.N, ncols, 101)
    h = case.host
    if case.route == "bs":
        _, r1 = o.bs_gemm(h.A, h.a_scale, h.B, h.b_scale, rows=rows)
        _, r2 = o.bs_gemm(h.A, h.a_scale, h.B, h.b_scale, cols=cols)
    else:
        _, r1 = o.mx_gemm(h.A, h.a_e8m0, h.B, h.b_e8m0, rows=rows)
        _, r2 = o.mx_gemm(h.A, h.a_e8m0, h.B, h.b_e8m0, cols=cols)
    g = np.concatenate([oracle.bf16_bits_to_f64(got[rows]).ravel(), oracle.bf16_bits_to_f64(got[:, cols]).ravel()])
    r = np.concatenate([oracle.bf16_bits_to_f64(r1).ravel(), oracle.bf16_bits_to_f64(r2).ravel()])
    bad = int(np.sum(np.abs(g - r) > 1e-2 + 1e-2 * np.abs(r)))
    cos = float(np.dot(g, r) / (np.linalg.norm(g) * np.linalg.norm(r)))
    return dict(sampled_rows=int(rows.size), sampled_cols=int(cols.size), n_bad=bad, cos=round(cos, 8),
                max_abs=float(np.max(np.abs(g - r))), finite=bool(np.all(np.isfinite(g))),
                passed=bool(bad == 0 and cos >= 0.9999 and np.all(np.isfinite(g))))


def cpu_baseline(case: Case, target_s: float = 12.0) -> dict:
    """The oracle as it stands, on a bounded sample of whole output rows of the workload."""
    import numpy as np

    import oracle
    o = oracle.load()
    h = case.host
    run = (lambda rows: o.bs_gemm(h.A, h.a_scale, h.B, h.b_scale, rows=rows)) if case.route == "bs" else \
        (lambda rows: o.mx_gemm(h.A, h.a_e8m0, h.B, h.b_e8m0, rows=rows))
    threads = max(o.num_threads(), 1)
    probe = np.arange(threads, dtype=np.int32)
    t0 = time.perf_counter()
    run(probe)
    dt = time.perf_counter() - t0
    nrows = int(min(case.M, max(threads, threads * round(target_s / max(dt, 1e-3)))))
    rows = np.arange(nrows, dtype=np.int32)
    t0 = time.perf_counter()
    run(rows)
    dt = time.perf_counter() - t0
    flops = 2.0 * nrows * case.N * case.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": o.num_threads(), "kind": "oracle",
            "sample": f"{nrows} full output rows of {case.name} ({case.M}x{case.N}x{case.K}), "
                      f"{flops / 1e9:.1f} GFLOP in {dt:.1f} s, fp64, OpenMP",
            "seconds": round(dt, 2), "host_cpus": os.cpu_count()}


def committed_traffic(workload_name: str):
    """HBM traffic per launch from the committed counter summary, if it was taken on the
    current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    entry = rec.get(workload_name)
    if not entry or entry.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return entry.get("traffic_bytes")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default=None, help="time only this workload (plus the main one)")
    ap.add_argument("--shape-steps", type=int, default=30)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library is a single-GPU kernel and no "
              "multi-GPU path exists (run with --gpus 1).", file=sys.stderr)
        return 2

    import torch

    import workload
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (cuda:0)", file=sys.stderr)
        return 2
    props = torch.cuda.get_device_properties(0)
    stream = torch.cuda.Stream()
    per_shape = {}
    main_row = None
    names = [MAIN] + [n for n in workload.CONFIGS if n != MAIN]
    if args.only:
        names = [MAIN] + ([args.only] if args.only != MAIN else [])
    with torch.cuda.stream(stream):
        for name in names:
            cfg = workload.CONFIGS[name]
            case = Case(name, cfg, 0, stream)
            steps = args.steps if name == MAIN else args.shape_steps
            warm = args.warmup if name == MAIN else max(3, args.warmup // 2)
            wall, ev = case.time_launches(steps, warm, stream)
            tflops = case.flops / ev / 1e12
            nbytes = algorithmic_bytes(case.route, case.M, case.N, case.K)
            row = dict(M=case.M, N=case.N, K=case.K, route=case.route, us=round(ev * 1e6, 2),
                       tflops=round(tflops, 1), pct_peak=round(100 * tflops / PEAK_FP8_TFLOPS, 2),
                       hbm_gbs_algorithmic=round(nbytes / ev / 1e9, 1))
            log(f"[bench] {name}: {row}")
            if name == MAIN:
                row["parity"] = sampled_parity(case)
                log(f"[bench] parity {row['parity']}")
                main_row = dict(wall=wall, ev=ev, case=case, nbytes=nbytes, steps=steps, warmup=warm)
                baseline = None if args.no_cpu else cpu_baseline(case)
                if baseline:
                    log(f"[bench] cpu baseline {baseline}")
                main_row["baseline"] = baseline
            else:
                case.free()
                del case
                torch.cuda.empty_cache()
            per_shape[name] = row

    case = main_row["case"]
    value = case.flops / main_row["wall"] / 1e12
    achieved = case.flops / main_row["ev"] / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": main_row["steps"],
        "warmup": main_row["warmup"],
        "ms_per_step": round(main_row["wall"] * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights, quantised on the host)",
        "config": {"workload": f"{MAIN} blockscale GEMM M={case.M} N={case.N} K={case.K} "
                               "(fp32 1x128 / 128x128 scales, bf16 out)",
                   "M": case.M, "N": case.N, "K": case.K, "route": "bs"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": committed_traffic(MAIN),
                     "kernel": "gemm_kernel (route BS)", "avg_launch_us": round(main_row["ev"] * 1e6, 2),
                     "flop_per_launch": case.flops},
        "cpu_baseline": main_row["baseline"],
        "per_shape": per_shape,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "kernel_source_sha256": kernel_source_hash()[:16]},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
