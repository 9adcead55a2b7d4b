"""Every instantiated kernel configuration on the GPU: each computes the same per-element
arithmetic (K blocks in order, same instructions), so all configurations must agree bit for
bit with the default one, and the default one must meet the parity bar against the oracle."""
import itertools

import numpy as np
import pytest
import torch

import workload
from gpu_util import bits, dev, parity, to_dev

pytestmark = pytest.mark.gpu


# (block_m, block_n, waves_m, waves_n, stages, pingpong)
TILES = [(128, 128, 2, 2, 3, 0), (256, 256, 4, 2, 2, 0), (256, 256, 2, 4, 2, 0), (128, 256, 2, 2, 3, 0),
         (256, 128, 2, 2, 3, 0), (128, 256, 2, 4, 3, 0), (256, 128, 4, 2, 3, 0), (128, 64, 2, 1, 3, 0),
         (256, 128, 4, 2, 2, 0), (128, 128, 2, 2, 4, 0), (128, 128, 2, 2, 2, 0), (256, 128, 4, 2, 2, 1),
         (128, 256, 2, 4, 2, 1), (256, 128, 4, 2, 3, 2), (128, 256, 2, 4, 3, 2), (256, 128, 2, 2, 3, 2),
         (128, 128, 2, 2, 3, 2)]


@pytest.fixture(scope="module")
def fb():
    import fp8_block_scaled_e4m3_amd as fb
    return fb


def _configs(fb, route, N):
    """Every tile with five tile orders; the C store policy (0, 1, 2) varies with the order, so
    every tile runs each policy."""
    out = []
    for (bm, bn, wm, wn, st, pp), (gm, xcd, pers, cst) in itertools.product(
            TILES, ((1, 0, 0, 0), (3, 1, 1, 2), (2, 0, 1, 1), (2, 2, 1, 2), (1, 2, 0, 1))):
        tm, tn = bm // wm, bn // wn
        ok = (tn <= 128 and 128 % tn == 0) if route == fb.ROUTE_BS else \
            (tm % 64 == 0 and tn % 64 == 0 and st * (bm + bn) * 132 <= 160 * 1024)
        if ok and N % bn == 0:
            out.append(fb.Config(bm, bn, wm, wn, st, gm, xcd, pers, pp, 0, cst))
    return out


# 4160 x 3072 gives more tiles than the persistent grid has workgroups, so workgroups run several
# tiles; K = 128 and 256 are the shallowest depths (one and two K steps per tile)
@pytest.mark.parametrize("M,N,K", [(300, 512, 384), (64, 256, 256), (4160, 3072, 640), (4160, 3072, 256),
                                   (4100, 3072, 128)])
def test_bs_all_configs_bitwise_equal(fb, oracle, M, N, K):
    x = workload.bs_inputs(M, N, K, 7)
    A, sa, sb = to_dev(x.A), to_dev(x.a_scale_kmajor), to_dev(x.b_scale)
    Bp = fb.prep_weights(to_dev(x.B))
    C0 = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8bs_gemm(A, sa, Bp, sb, C0)
    _, ref = oracle.bs_gemm(x.A, x.a_scale, x.B, x.b_scale)
    parity(bits(C0), ref, f"bs default {M}x{N}x{K}")
    # every configuration of the main kernel computes the same thing in the same order (the
    # plain entry point may pick the small-M kernel, which splits K and is checked on its own)
    cfgs = _configs(fb, fb.ROUTE_BS, N)
    assert len(cfgs) >= 8
    C1 = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8bs_gemm_with_config(A, sa, Bp, sb, C1, cfgs[0])
    ref_bits = bits(C1)
    parity(ref_bits, ref, f"bs {cfgs[0]}")
    for cfg in cfgs:
        C = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=dev())
        fb.fp8bs_gemm_with_config(A, sa, Bp, sb, C, cfg)
        got = bits(C)
        assert np.array_equal(got, ref_bits), f"{cfg}: {int((got != ref_bits).sum())} differ"


@pytest.mark.parametrize("M,N,K", [(320, 512, 384), (64, 192, 256), (4160, 3072, 640), (4160, 3072, 256)])
def test_mx_all_configs_bitwise_equal(fb, oracle, M, N, K):
    y = workload.mx_inputs(M, N, K, 8)
    A = to_dev(y.A)
    pa = fb.mx_pack_a_scale(to_dev(y.a_e8m0))
    Bp, pb = fb.mx_prep_weights(to_dev(y.B), to_dev(y.b_e8m0))
    C0 = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fb.fp8mx_gemm(A, pa, Bp, pb, C0)
    ref_bits = bits(C0)
    _, ref = oracle.mx_gemm(y.A, y.a_e8m0, y.B, y.b_e8m0)
    parity(ref_bits, ref, f"mx default {M}x{N}x{K}")
    cfgs = _configs(fb, fb.ROUTE_MX, N)
    assert cfgs
    for cfg in cfgs:
        C = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=dev())
        fb.fp8mx_gemm_with_config(A, pa, Bp, pb, C, cfg)
        got = bits(C)
        assert np.array_equal(got, ref_bits), f"{cfg}: {int((got != ref_bits).sum())} differ"


def test_invalid_configs_rejected(fb):
    x = workload.bs_inputs(128, 256, 256, 1)
    A, sa, sb = to_dev(x.A), to_dev(x.a_scale_kmajor), to_dev(x.b_scale)
    Bp = fb.prep_weights(to_dev(x.B))
    C = torch.full((128, 256), 3.0, dtype=torch.bfloat16, device=dev())
    for cfg in (fb.Config(64, 64, 1, 1, 2, 1, 1, 1), fb.Config(256, 256, 2, 2, 2, 1, 1, 1),  # not instantiated
                fb.Config(256, 256, 4, 2, 3, 1, 1, 1),  # stages not instantiated for this tile
                fb.Config(128, 256, 1, 2, 3, 1, 1, 1), fb.Config(256, 256, 4, 2, 2, 0, 1, 1),  # group_m < 1
                fb.Config(128, 128, 2, 2, 3, 1, 3, 1), fb.Config(128, 128, 2, 2, 3, 1, 1, 5),
                fb.Config(256, 128, 4, 2, 3, 1, 1, 1, 1),  # ping-pong needs two stages
                fb.Config(256, 128, 4, 2, 3, 1, 1, 1, 3),  # no such schedule
                fb.Config(256, 128, 4, 2, 3, 1, 1, 1, 4),  # no such schedule
                fb.Config(256, 128, 4, 2, 2, 1, 1, 1, 2),  # warp-specialised, not with 2 stages
                fb.Config(128, 128, 2, 2, 3, 1, 1, 1, 2, 0, 3),  # no such C store policy
                fb.Config(128, 128, 2, 2, 3, 1, 1, 1, 2, 0, -1)):
        with pytest.raises(fb.Fp8bsError) as e:
            fb.fp8bs_gemm_with_config(A, sa, Bp, sb, C, cfg)
        assert e.value.status == 4
    torch.cuda.synchronize()
    assert torch.all(C == 3.0)
