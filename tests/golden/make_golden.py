"""Writes tests/golden/*.txt: regression fixtures of the oracle's output on the seeded
128x256x512 workloads (route BS, route MX and the promote-free twin, route PT). Calls only the oracle and the input
generator. The pages print no worked numeric example, so these fixtures pin the oracle
against its own earlier, pinned self (they catch accidental changes), nothing more.

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workload  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
PICKS = [(0, 0), (0, 255), (17, 3), (64, 128), (100, 201), (127, 127), (127, 255)]


def write(name, bits, acc, header):
    digest = hashlib.sha256(np.ascontiguousarray(bits).tobytes()).hexdigest()
    lines = [f"# {header}", f"sha256_bf16_bits {digest}"]
    for m, n in PICKS:
        lines.append(f"{m} {n} {int(bits[m, n]):#06x} {float(acc[m, n])!r}")
    open(os.path.join(HERE, name), "w").write("\n".join(lines) + "\n")


def main():
    o = oracle.load()
    x = workload.bs_inputs(128, 256, 512, 0)
    acc, bits = o.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    write("tiny_bs_seed0.txt", bits, acc,
          "oracle route BS, M=128 N=256 K=512 seed 0 (workload.bs_inputs); columns: m n bf16 fp64")
    y = workload.mx_inputs(128, 256, 512, 0)
    acc, bits = o.mx_gemm(y.A, y.a_e8m0, y.B, y.b_e8m0)
    write("tiny_mx_seed0.txt", bits, acc,
          "oracle route MX, M=128 N=256 K=512 seed 0 (workload.mx_inputs); columns: m n bf16 fp64")
    z = workload.pt_inputs(128, 256, 512, 0)
    acc, bits = o.pt_gemm(z.A, z.a_scale, z.B, z.b_scale)
    write("tiny_pt_seed0.txt", bits, acc,
          "oracle route PT, M=128 N=256 K=512 seed 0 (workload.pt_inputs); columns: m n bf16 fp64")


if __name__ == "__main__":
    main()
