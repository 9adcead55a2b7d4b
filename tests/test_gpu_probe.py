"""The diagnostic probes launch and finish on every instantiated configuration (their results
are timings, not values: only the launch status and the FLOP count are checked)."""
import pytest
import torch

import workload
from gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def operands():
    import fp8_block_scaled_e4m3_amd as fb
    x = workload.bs_inputs(512, 512, 1024, 3)
    return fb, to_dev(x.A), fb.prep_weights(to_dev(x.B))


def test_mfma_ceiling_runs(operands):
    fb, A, Bp = operands
    sink = torch.empty(256 * 8, dtype=torch.float32, device=dev())
    flops = fb.fp8bs_mfma_ceiling(A, Bp, 512, 8, sink)
    torch.cuda.synchronize()
    assert flops > 0


@pytest.mark.parametrize("parts", [0, 1, 3, 5, 7, 15, 17, 19, 23, 31])
def test_loop_probe_runs(operands, parts):
    fb, A, Bp = operands
    sink = torch.empty(256 * 8, dtype=torch.float32, device=dev())
    n = fb.lib.fp8bs_loop_probe_out_bytes(parts)
    out = torch.empty(max(n, 16), dtype=torch.uint8, device=dev())
    flops = fb.fp8bs_loop_probe(parts, A, Bp, 512, 12, sink, out)
    torch.cuda.synchronize()
    per_wave = (32 if parts & 16 else 16) * 12 * 2 * 16 * 16 * 128
    assert flops > 0 and flops % per_wave == 0
