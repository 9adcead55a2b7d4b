"""The C-ABI library loads and exports every function include/fp8bs.h declares, and the
host-side validation (which runs before any HIP call) returns the documented codes. CPU only:
no call here launches work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(fp8(?:bs|mx)_[a-z0-9_]+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def fb():
    import fp8_block_scaled_e4m3_amd as fb
    return fb


def test_header_declares_the_routes():
    names = _declared()
    for n in ("fp8bs_gemm", "fp8mx_gemm", "fp8bs_prep_weights", "fp8mx_prep_weights", "fp8mx_pack_a_scale"):
        assert n in names


def test_every_declared_symbol_is_exported(fb):
    handle = ctypes.CDLL(fb.LIBRARY)
    for name in _declared():
        assert hasattr(handle, name), name
        assert name in fb.SIGNATURES, f"binding lacks {name}"


def test_version_and_strerror(fb):
    assert fb.fp8bs_version() >= 10200  # fp8bs_config with c_store
    assert ctypes.sizeof(fb.Config) == 11 * 4
    for code in range(6):
        assert fb.fp8bs_strerror(code)
    assert fb.fp8bs_strerror(99) == "unknown status"


def test_sizes(fb):
    assert fb.fp8bs_prep_weight_bytes(256, 512) == 256 * 512
    assert fb.fp8mx_packed_scale_bytes(128, 512) == 128 * 16
    assert fb.fp8bs_prep_weight_bytes(0, 512) == 0


@pytest.mark.parametrize("M,N,K", [(16, 100, 128), (16, 128, 100), (16, 128, 0), (-3, 128, 128), (16, 0, 128)])
def test_bs_shape_rejected_before_any_launch(fb, M, N, K):
    assert fb.lib.fp8bs_gemm(None, None, None, None, None, M, N, K, None) == 2


def test_bs_null_rejected(fb):
    assert fb.lib.fp8bs_gemm(None, None, None, None, None, 16, 128, 128, None) == 1


def test_bs_misaligned_rejected(fb):
    p = 0x1000
    assert fb.lib.fp8bs_gemm(p + 4, p, p, p, p, 16, 128, 128, None) == 3
    assert fb.lib.fp8bs_gemm(p, p + 2, p, p, p, 16, 128, 128, None) == 3


@pytest.mark.parametrize("M,N,K", [(100, 128, 256), (128, 96, 256), (128, 128, 128), (128, 128, 200)])
def test_mx_shape_rejected(fb, M, N, K):
    assert fb.lib.fp8mx_gemm(None, None, None, None, None, M, N, K, None) == 2


def test_mx_null_and_prep_validation(fb):
    assert fb.lib.fp8mx_gemm(None, None, None, None, None, 64, 64, 256, None) == 1
    assert fb.lib.fp8mx_pack_a_scale(None, None, 100, 256, None) == 2
    assert fb.lib.fp8mx_prep_weights(None, None, None, None, 64, 128, None) == 2
    assert fb.lib.fp8bs_prep_weights(None, None, 64, 128, None) == 1


def test_zero_rows_is_accepted_without_pointers(fb):
    assert fb.lib.fp8bs_gemm(None, None, None, None, None, 0, 128, 128, None) == 0


def test_select_config_is_shape_driven(fb):
    """The configuration depends on (M, N, K) only; large shapes take the 256x256 tile (with
    the XCD remap unless the output is very wide), except route BS at K <= 1536, which takes
    the warp-specialised 128x256 tile in 8-row bands; narrow grids a smaller tile that still
    fills the device."""
    big = fb.fp8bs_select_config(fb.ROUTE_BS, 16384, 7168, 768)
    assert (big.block_m, big.block_n, big.pingpong, big.group_m, big.xcd_remap) == (128, 256, 2, 8, 1)
    for route, shape in ((fb.ROUTE_BS, (8192, 8192, 2048)), (fb.ROUTE_BS, (4096, 16384, 7168)),
                         (fb.ROUTE_PT, (16384, 7168, 768)), (fb.ROUTE_MX, (16384, 8192, 1280))):
        c = fb.fp8bs_select_config(route, *shape)
        assert (c.block_m, c.block_n, c.pingpong, c.group_m, c.xcd_remap) == (256, 256, 0, 4, 1), (route, shape)
    nn = fb.fp8bs_select_config(fb.ROUTE_BS, 4096, 2048, 7168)
    assert ((4096 + nn.block_m - 1) // nn.block_m) * (2048 // nn.block_n) >= 256
    # narrow-N: 128x256 tiles, 8 math waves (2x4) plus the four loader waves of schedule 2
    assert (nn.block_m, nn.block_n, nn.waves_m, nn.waves_n, nn.stages, nn.pingpong) == (128, 256, 2, 4, 3, 2)
    nn16 = fb.fp8bs_select_config(fb.ROUTE_BS, 16384, 1536, 7168)
    assert (nn16.block_m, nn16.block_n, nn16.pingpong) == (128, 256, 2)
    # N not a multiple of 256: 256x128 tiles
    nn_odd = fb.fp8bs_select_config(fb.ROUTE_BS, 8192, 1920, 7168)
    assert (nn_odd.block_m, nn_odd.block_n, nn_odd.pingpong) == (256, 128, 2)
    mx = fb.fp8bs_select_config(fb.ROUTE_MX, 4096, 192, 256)  # N % 128 != 0: the 128x64 tile
    assert (mx.small_m, mx.block_n) == (0, 64)
    wide = fb.fp8bs_select_config(fb.ROUTE_BS, 4096, 65536, 1536)  # 2048-tile bands: round-local order
    assert (wide.block_m, wide.block_n, wide.group_m) == (128, 256, 8) and wide.xcd_remap == 2
    wide_pt = fb.fp8bs_select_config(fb.ROUTE_PT, 4096, 65536, 1536)
    assert (wide_pt.block_m, wide_pt.block_n) == (256, 256) and wide_pt.xcd_remap == 2
    # C stores: non-temporal and written through for a C larger than 256 MiB, written through
    # for a C of at most 64 MiB, ordinary stores otherwise
    assert nn.c_store == 1 and wide.c_store == 2 and big.c_store == 0 and nn16.c_store == 1
    for route, shape, policy in ((fb.ROUTE_MX, (16384, 8192, 1280), 0), (fb.ROUTE_MX, (16384, 8192 + 256, 1280), 2),
                                 (fb.ROUTE_BS, (4096, 8192, 1536), 1), (fb.ROUTE_PT, (4096, 2048, 7168), 1),
                                 (fb.ROUTE_BS, (128, 65536, 1536), 1), (fb.ROUTE_BS, (1, 128, 128), 0),
                                 (fb.ROUTE_MX, (16384, 5120, 2048), 0), (fb.ROUTE_BS, (4096, 8192 + 256, 1536), 0),
                                 (fb.ROUTE_BS, (16384, 16384, 1536), 2)):
        assert fb.fp8bs_select_config(route, *shape).c_store == policy, (route, shape)
    for route, shape in ((fb.ROUTE_BS, (4096, 65536, 1536)), (fb.ROUTE_MX, (16384, 8192, 1280)),
                         (fb.ROUTE_BS, (128, 256, 512)), (fb.ROUTE_BS, (1, 128, 128))):
        c = fb.fp8bs_select_config(route, *shape)
        assert c.small_m == 1 or (shape[1] % c.block_n == 0 and c.group_m >= 1)
    # the small-M kernel for M <= 4; up to 16 rows unless one row of 128x256 tiles fills the
    # CUs; from 17 rows while its 16x16x128 products per K block, W = ceil(M/64) * N/16 *
    # ceil(min(M, 64)/16), stay within 3072 (route BS from K = 2048) or 2048 (otherwise)
    for route, shape, small in ((fb.ROUTE_BS, (1, 128, 128), 1), (fb.ROUTE_BS, (4, 65536, 1536), 1),
                                (fb.ROUTE_BS, (16, 65536, 1536), 0), (fb.ROUTE_BS, (16, 32768, 1536), 1),
                                (fb.ROUTE_BS, (17, 32768, 1536), 0), (fb.ROUTE_BS, (64, 16384, 1536), 0),
                                (fb.ROUTE_BS, (64, 2048, 7168), 1), (fb.ROUTE_BS, (64, 65536, 1536), 0),
                                (fb.ROUTE_BS, (65, 128, 7168), 1), (fb.ROUTE_PT, (33, 4096, 512), 1),
                                (fb.ROUTE_BS, (512, 2048, 7168), 0), (fb.ROUTE_PT, (96, 1536, 7168), 1),
                                (fb.ROUTE_BS, (640, 2048, 7168), 0), (fb.ROUTE_BS, (192, 7168, 7168), 0),
                                (fb.ROUTE_BS, (96, 7168, 768), 0), (fb.ROUTE_MX, (128, 2048, 7168), 1),
                                (fb.ROUTE_MX, (128, 7168, 7168), 0), (fb.ROUTE_MX, (64, 32768, 1536), 0),
                                (fb.ROUTE_PT, (0, 4096, 512), 0), (fb.ROUTE_MX, (64, 4096, 512), 1),
                                (fb.ROUTE_BS, (128, 2048, 1024), 1), (fb.ROUTE_BS, (384, 2048, 2048), 1),
                                (fb.ROUTE_BS, (256, 4096, 2048), 0), (fb.ROUTE_PT, (100, 4096, 512), 1),
                                (fb.ROUTE_MX, (128, 4096, 2048), 1), (fb.ROUTE_MX, (192, 4096, 2048), 0),
                                (fb.ROUTE_BS, (48, 7168, 1024), 1), (fb.ROUTE_BS, (48, 16384, 1024), 0),
                                (fb.ROUTE_BS, (200, 2048, 4096), 1), (fb.ROUTE_PT, (192, 4096, 4096), 0)):
        c = fb.fp8bs_select_config(route, *shape)
        assert c.small_m == small, (route, shape)
        if small:
            assert (c.block_m, c.block_n, c.stages) == (0, 0, 0)
    # one row of 128-row tiles covers M and fills the CUs: the 128x256 warp-specialised tile
    for route, shape in ((fb.ROUTE_BS, (16, 65536, 1536)), (fb.ROUTE_BS, (128, 65536, 1536)),
                         (fb.ROUTE_PT, (64, 65536, 7168)), (fb.ROUTE_MX, (64, 65536, 1536))):
        c = fb.fp8bs_select_config(route, *shape)
        assert (c.block_m, c.block_n, c.pingpong) == (128, 256, 2), (route, shape)
    # otherwise 128x128, warp-specialised (one row of 128-row tiles never needs 256-row tiles)
    for route, shape in ((fb.ROUTE_BS, (64, 32768, 1536)), (fb.ROUTE_MX, (128, 32768, 1536)),
                         (fb.ROUTE_BS, (128, 7168, 1024)), (fb.ROUTE_PT, (100, 7168, 512)),
                         (fb.ROUTE_MX, (128, 7168, 7168)), (fb.ROUTE_BS, (64, 16384, 1536))):
        c = fb.fp8bs_select_config(route, *shape)
        assert (c.block_m, c.block_n, c.waves_m, c.waves_n, c.pingpong) == (128, 128, 2, 2, 2), (route, shape)
    c = fb.fp8bs_select_config(fb.ROUTE_BS, 64, 40960 - 128, 1536)  # 319 tiles: two rounds
    assert (c.block_m, c.block_n, c.pingpong) == (128, 128, 2)
    # 256x128 tiles just past one round (257 to 384): 128x128 ones instead; at 256 and from 385
    # the larger tiles, 128x256 where N % 256 == 0
    for route, shape, tile in ((fb.ROUTE_BS, (1280, 7168, 2048), (128, 128)), (fb.ROUTE_MX, (4352, 2048, 7168), (128, 128)),
                               (fb.ROUTE_BS, (4096, 2048, 7168), (128, 256)), (fb.ROUTE_BS, (1664, 7168, 2048), (128, 256)),
                               (fb.ROUTE_BS, (4096, 1920, 7168), (256, 128))):
        c = fb.fp8bs_select_config(route, *shape)
        assert (c.block_m, c.block_n, c.pingpong) == (*tile, 2), (route, shape)
    c = fb.fp8bs_select_config(fb.ROUTE_BS, 129, 65536, 1536)
    assert c.block_m == 256
    # one row of 128-row tiles, where 128x256 tiles need one round of the CUs and 128x128 two
    c = fb.fp8bs_select_config(fb.ROUTE_BS, 64, 36864, 7168)
    assert (c.block_m, c.block_n, c.pingpong) == (128, 256, 2)
    # 256x256 tiles from one round of the CUs for route MX, from two for the others
    assert fb.fp8bs_select_config(fb.ROUTE_MX, 256, 65536, 1536).block_m == 256
    c = fb.fp8bs_select_config(fb.ROUTE_BS, 1024, 24576, 1536)
    assert (c.block_m, c.block_n) == (128, 256)
    # 128x128 tiles only while they need no more rounds of the CUs than 256x128 tiles
    for shape, tile in (((640, 7168, 7168), (256, 128)), ((1024, 7168, 7168), (256, 128)),
                        ((1024, 3072, 7168), (128, 128)), ((1024, 2048, 7168), (128, 128)),
                        ((200, 4096, 512), (128, 128))):
        c = fb.fp8bs_select_config(fb.ROUTE_BS, *shape)
        assert (c.block_m, c.block_n) == tile, shape


def test_select_config_rejects_bad_input(fb):
    import ctypes
    cfg = fb.Config()
    assert fb.lib.fp8bs_select_config(0, 128, 100, 128, ctypes.byref(cfg)) == 2
    assert fb.lib.fp8bs_select_config(1, 100, 128, 256, ctypes.byref(cfg)) == 2
    assert fb.lib.fp8bs_select_config(7, 128, 128, 256, ctypes.byref(cfg)) == 4
    assert fb.lib.fp8bs_select_config(0, 128, 128, 256, None) == 1


def test_small_m_limits_rejected_on_the_host(fb):
    """More than 65535 chunks of 64 rows, and K below the MX minimum, are rejected before
    anything is launched: placeholder pointers are never dereferenced."""
    p = 0x10000
    too_many = 64 * 65535 + 1
    cfg = fb.Config()
    cfg.small_m = 1
    assert fb.lib.fp8bs_gemm_with_config(p, p, p, p, p, too_many, 256, 256, ctypes.byref(cfg), None) == 4
    assert fb.lib.fp8pt_gemm_with_config(p, p, p, p, p, too_many, 256, 256, ctypes.byref(cfg), None) == 4
    assert fb.lib.fp8mx_gemm_small_m(p, p, p, p, p, too_many, 256, 256, None) == 2
    assert fb.lib.fp8mx_gemm_small_m(p, p, p, p, p, 16, 256, 128, None) == 2
    pair = fb.Config()
    pair.small_m = 4  # two weight sub-tiles per workgroup: at most 32 rows per chunk
    assert fb.lib.fp8bs_gemm_with_config(p, p, p, p, p, 33, 256, 256, ctypes.byref(pair), None) == 4
    bad = fb.Config()
    bad.small_m = 5
    assert fb.lib.fp8bs_gemm_with_config(p, p, p, p, p, 8, 256, 256, ctypes.byref(bad), None) == 4


def test_store_policy_out_of_range_rejected(fb):
    """c_store other than 0, 1 or 2 is a configuration error, found before any launch."""
    p = 0x10000
    for policy in (-1, 3):
        for fn in (fb.lib.fp8bs_gemm_with_config, fb.lib.fp8pt_gemm_with_config, fb.lib.fp8mx_gemm_with_config):
            cfg = fb.fp8bs_select_config(fb.ROUTE_BS, 4096, 2048, 7168)
            cfg.c_store = policy
            assert fn(p, p, p, p, p, 4096, 2048, 7168, ctypes.byref(cfg), None) == 4


def test_offsets_past_32_bits_rejected(fb):
    p = 0x10000
    assert fb.lib.fp8bs_gemm(p, p, p, p, p, 1 << 21, 128, 1024, None) == 2  # M*K = 2^31
    assert fb.lib.fp8bs_gemm(p, p, p, p, p, 16, 1 << 21, 1024, None) == 2   # N*K = 2^31


# ---- the Python binding checks every tensor before the library sees it ------------------------

def _cpu_bs(M, N, K):
    import torch
    return (torch.zeros((M, K), dtype=torch.uint8), torch.ones((K // 128, M)), torch.zeros(N * K, dtype=torch.uint8),
            torch.ones((N // 128, K // 128)), torch.zeros((M, N), dtype=torch.bfloat16))


def test_binding_rejects_missized_operands(fb):
    import torch
    M, N, K = 64, 256, 512
    A, sa, Bp, sb, C = _cpu_bs(M, N, K)
    bad = {
        "a_scale in [M, K/128] (the natural layout)": dict(a_scale=torch.ones((M, K // 128))),
        "C with fewer rows": dict(C=torch.zeros((M - 1, N), dtype=torch.bfloat16)),
        "C in fp32": dict(C=torch.zeros((M, N), dtype=torch.float32)),
        "B_prep for fewer weight rows": dict(B_prep=torch.zeros((N - 128) * K, dtype=torch.uint8)),
        "b_scale transposed": dict(b_scale=torch.ones((K // 128, N // 128))),
        "A in bf16": dict(A=torch.zeros((M, K), dtype=torch.bfloat16)),
        "a_scale in fp64": dict(a_scale=torch.ones((K // 128, M), dtype=torch.float64)),
    }
    for what, repl in bad.items():
        args = dict(A=A, a_scale=sa, B_prep=Bp, b_scale=sb, C=C)
        args.update(repl)
        with pytest.raises(ValueError):
            fb.fp8bs_gemm(**args)
        with pytest.raises(ValueError):
            fb.fp8bs_gemm_with_config(config=fb.Config(), **args)
    # every size right, but host memory: refused before any call
    with pytest.raises(ValueError, match="device tensors"):
        fb.fp8bs_gemm(A, sa, Bp, sb, C)


def test_binding_rejects_missized_mx_pt_and_quantiser_operands(fb):
    import torch
    M, N, K = 64, 256, 512
    A = torch.zeros((M, K), dtype=torch.uint8)
    C = torch.zeros((M, N), dtype=torch.bfloat16)
    Bp = torch.zeros(N * K, dtype=torch.uint8)
    pa = torch.zeros(M * K // 32, dtype=torch.uint8)
    pb = torch.zeros(N * K // 32, dtype=torch.uint8)
    with pytest.raises(ValueError, match="b_scale_packed"):
        fb.fp8mx_gemm(A, pa, Bp, pb[:-4], C)
    with pytest.raises(ValueError, match="a_scale_packed"):
        fb.fp8mx_gemm(A, pa[: M * K // 64], Bp, pb, C)
    with pytest.raises(ValueError, match="a_e8m0"):
        fb.fp8mx_gemm_small_m(A, pa, Bp, pb, C)  # the small-M entry takes [M, K/32] bytes
    with pytest.raises(ValueError, match="device tensors"):
        fb.fp8mx_gemm_small_m(A, pa.view(M, K // 32), Bp, pb, C)
    with pytest.raises(ValueError, match="a_scale"):
        fb.fp8pt_gemm(A, torch.ones(M + 1), Bp, torch.ones(N), C)
    with pytest.raises(ValueError, match="b_scale"):
        fb.fp8pt_gemm(A, torch.ones(M), Bp, torch.ones((N // 128, K // 128)), C)
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="a_scale"):
        fb.fp8bs_quantize_act(x, A, torch.ones((M, K // 128)))
    with pytest.raises(ValueError, match="A_codes"):
        fb.fp8mx_quantize_act(x, A[:, : K // 2], torch.zeros((M, K // 32), dtype=torch.uint8))
    with pytest.raises(ValueError, match="dtype"):
        fb.fp8bs_quantize_act(x.to(torch.float16), A, torch.ones((K // 128, M)))
    with pytest.raises(ValueError, match="B_prep"):
        fb.fp8bs_prep_weights(torch.zeros((N, K), dtype=torch.uint8), torch.zeros(N * K // 2, dtype=torch.uint8))
    with pytest.raises(ValueError, match="b_e8m0"):
        fb.fp8mx_prep_weights(torch.zeros((N, K), dtype=torch.uint8), torch.zeros((N, K // 16), dtype=torch.uint8),
                              Bp, pb)


# ---- names the hot-path contract lists, or the recorded name that serves each ------------------

# The survey's boundary names the calls below. Where this library's name differs, the value is
# the exported call that provides it (the difference is recorded in the design notes).
CONTRACT_CALLS = {
    "fp8bs_gemm": "fp8bs_gemm",
    "fp8mx_gemm": "fp8mx_gemm",
    "fp8bs_prep_bytes": "fp8bs_prep_bytes",
    "fp8bs_prep_weights": "fp8bs_prep_weights",
    "fp8mx_prep_weights": "fp8mx_prep_weights",
    "fp8mx_pack_a_scale": "fp8mx_pack_a_scale",
    "fp8mx_scale_bytes": "fp8mx_scale_bytes",
    "fp8bs_select_config": "fp8bs_select_config",
    "fp8bs_gemm_with_config": "fp8bs_gemm_with_config",
    "fp8mx_gemm_with_config": "fp8mx_gemm_with_config",
    "fp8bs_strerror": "fp8bs_strerror",
    "fp8bs_version": "fp8bs_version",
}


def test_contract_calls_are_exported(fb):
    handle = ctypes.CDLL(fb.LIBRARY)
    declared = _declared()
    for want, name in CONTRACT_CALLS.items():
        assert hasattr(handle, name) and name in declared, f"{want}: {name} not exported"
    assert fb.fp8bs_prep_bytes(256, 512) == fb.fp8bs_prep_weight_bytes(256, 512) == 256 * 512
    assert fb.fp8mx_scale_bytes(128, 512) == fb.fp8mx_packed_scale_bytes(128, 512) == 128 * 16


def test_splitk_sizes_and_host_rejections(fb):
    """The library's split choice and its workspace size; rejections before any launch."""
    assert fb.fp8bs_splitk_workspace_bytes(1024, 2048, 7168, 0) == 2 * 1024 * 2048 * 4  # 128 tiles x 2 ranges
    assert fb.fp8bs_splitk_workspace_bytes(1024, 2048, 7168, 1) == 0
    assert fb.fp8bs_splitk_workspace_bytes(1024, 2048, 7168, 4) == 4 * 1024 * 2048 * 4
    assert fb.fp8bs_splitk_workspace_bytes(4096, 2048, 7168, 0) == 0  # 256 tiles fill the CUs
    assert fb.fp8bs_splitk_workspace_bytes(100, 100, 128, 0) == 0     # a shape route BS rejects
    assert fb.fp8bs_splitk_workspace_bytes(256, 4096, 2048, 0) == 0   # too shallow to repay the second pass
    assert fb.fp8bs_splitk_workspace_bytes(128, 7168, 7168, 0) == 4 * 128 * 7168 * 4
    assert fb.fp8bs_splitk_workspace_bytes(512, 2048, 4096, 0) == 0   # K = 4096: splitting does not pay
    p = 0x10000
    L = fb.lib
    assert L.fp8bs_gemm_splitk(p, p, p, p, p, 1024, 2048, 7168, 0, None, 0, None) == 6
    assert L.fp8bs_gemm_splitk(p, p, p, p, p, 1024, 2048, 7168, 0, p + 16, 1 << 30, None) == 6  # misaligned
    assert L.fp8bs_gemm_splitk(p, p, p, p, p, 1024, 2048, 7168, 0, p, 2 * 1024 * 2048 * 4 - 1, None) == 6
    assert L.fp8bs_gemm_splitk(p, p, p, p, p, 1024, 2048, 7168, 3, p, 1 << 30, None) == 4  # 56 % 3
    assert L.fp8bs_gemm_splitk(p, p, p, p, p, 1024, 2048, 7168, 65, p, 1 << 30, None) == 4
    assert L.fp8bs_gemm_splitk(p, p, p, p, p, 1024, 100, 7168, 2, p, 1 << 30, None) == 2
    assert L.fp8bs_gemm_splitk(None, p, p, p, p, 1024, 2048, 7168, 2, p, 1 << 30, None) == 1
    assert L.fp8bs_gemm_splitk(p, p, p, p, p, 0, 2048, 7168, 2, None, 0, None) == 0
    assert fb.fp8bs_strerror(6).startswith("the workspace")


def test_loop_probe_host_rejections(fb):
    """The loop-skeleton probe's host checks: unknown part masks, small operands, NULL or short
    buffers are rejected before anything is launched."""
    L, p = fb.lib, 0x1000
    assert L.fp8bs_loop_probe_out_bytes(2) == 0          # not an instantiated mask
    assert L.fp8bs_loop_probe_out_bytes(7) == 0          # no stores, no output
    assert L.fp8bs_loop_probe_out_bytes(15) > 0 and L.fp8bs_loop_probe_out_bytes(31) == 2 * L.fp8bs_loop_probe_out_bytes(15)
    assert L.fp8bs_loop_probe(2, p, p, 512, 512, 1024, 10, None, 0, p, 4096, None, None) == 4
    assert L.fp8bs_loop_probe(1, p, p, 64, 64, 128, 10, None, 0, p, 4096, None, None) == 2
    assert L.fp8bs_loop_probe(1, None, p, 512, 512, 1024, 10, None, 0, p, 4096, None, None) == 1
    assert L.fp8bs_loop_probe(15, p, p, 512, 512, 1024, 10, None, 0, p, 4096, None, None) == 1
    assert L.fp8bs_loop_probe(15, p, p, 512, 512, 1024, 10, p, 100, p, 4096, None, None) == 6
    assert L.fp8bs_loop_probe(1, p, p, 512, 512, 1024, 10, None, 0, p, 100, None, None) == 6
    assert L.fp8bs_loop_probe(1, p + 4, p, 512, 512, 1024, 10, None, 0, p, 4096, None, None) == 3
