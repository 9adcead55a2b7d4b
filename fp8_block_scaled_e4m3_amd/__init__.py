"""fp8_block_scaled_e4m3_amd -- thin Python binding of libfp8bs, the gfx950 fp8 block-scaled GEMM.

Every function here only marshals arguments (torch tensors -> device pointers, the current
torch stream -> hipStream_t) and calls the C ABI declared in ``include/fp8bs.h`` under the
same name. All computation runs in the HIP library; there is no CPU or PyTorch fallback, and
importing this package fails loudly when the library has not been built.

Routes (see include/fp8bs.h for layouts and constraints):

* ``fp8bs_gemm(A, a_scale, B_prep, b_scale, C)`` -- fp32 per-1x128 activation scales
  (``a_scale`` laid out [K/128, M]) and fp32 per-128x128 weight scales ([N/128, K/128]).
* ``fp8mx_gemm(A, a_scale_packed, B_prep, b_scale_packed, C)`` -- 1x32 ue8m0 scales, packed
  once by ``fp8mx_pack_a_scale`` / ``fp8mx_prep_weights``.
* ``fp8pt_gemm(A, a_scale, B_prep, b_scale, C)`` -- the promote-free twin: fp32 ``a_scale`` [M]
  and ``b_scale`` [N], applied once in the epilogue.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIBRARY", "Fp8bsError", "lib", "fp8bs_version", "fp8bs_strerror",
    "fp8bs_prep_weight_bytes", "fp8bs_prep_bytes", "fp8bs_prep_weights", "fp8bs_gemm",
    "fp8mx_packed_scale_bytes", "fp8mx_scale_bytes", "fp8mx_pack_a_scale", "fp8mx_prep_weights", "fp8mx_gemm",
    "prep_weights", "mx_prep_weights", "mx_pack_a_scale",
    "Config", "ROUTE_BS", "ROUTE_MX", "fp8bs_select_config", "fp8bs_gemm_with_config", "fp8mx_gemm_with_config",
    "fp8bs_mfma_ceiling", "fp8bs_loop_probe", "ROUTE_PT", "fp8pt_gemm", "fp8pt_gemm_with_config",
    "IN_F32", "IN_BF16", "fp8bs_quantize_act", "fp8mx_quantize_act", "quantize_bs", "quantize_mx",
    "fp8mx_gemm_small_m", "fp8bs_splitk_workspace_bytes", "fp8bs_gemm_splitk", "splitk_workspace",
    "fp8bs_gemm_splitk_noalloc", "SPLITK_SCRATCH_BYTES",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libfp8bs.so")

# C ABI symbol table: name -> (restype, argtypes). Mirrors include/fp8bs.h.
_vp, _int, _size = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "fp8bs_version": (_int, []),
    "fp8bs_strerror": (ctypes.c_char_p, [_int]),
    "fp8bs_prep_weight_bytes": (_size, [_int, _int]),
    "fp8bs_prep_bytes": (_size, [_int, _int]),
    "fp8bs_prep_weights": (_int, [_vp, _vp, _int, _int, _vp]),
    "fp8bs_gemm": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _vp]),
    "fp8mx_packed_scale_bytes": (_size, [_int, _int]),
    "fp8mx_scale_bytes": (_size, [_int, _int]),
    "fp8mx_pack_a_scale": (_int, [_vp, _vp, _int, _int, _vp]),
    "fp8mx_prep_weights": (_int, [_vp, _vp, _vp, _vp, _int, _int, _vp]),
    "fp8mx_gemm": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _vp]),
    "fp8bs_select_config": (_int, [_int, _int, _int, _int, _vp]),
    "fp8bs_gemm_with_config": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _vp, _vp]),
    "fp8mx_gemm_with_config": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _vp, _vp]),
    "fp8bs_mfma_ceiling": (_int, [_vp, _vp, _int, _int, _int, _int, _vp, _int, _vp, _vp]),
    "fp8bs_loop_probe_out_bytes": (ctypes.c_size_t, [_int]),
    "fp8bs_loop_probe": (_int, [_int, _vp, _vp, _int, _int, _int, _int, _vp, ctypes.c_size_t, _vp, _int, _vp, _vp]),
    "fp8pt_gemm": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _vp]),
    "fp8bs_quantize_act": (_int, [_vp, _int, _vp, _vp, _int, _int, _vp]),
    "fp8mx_gemm_small_m": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _vp]),
    "fp8mx_quantize_act": (_int, [_vp, _int, _vp, _vp, _int, _int, _vp]),
    "fp8pt_gemm_with_config": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _vp, _vp]),
    "fp8bs_splitk_workspace_bytes": (_size, [_int, _int, _int, _int]),
    "fp8bs_gemm_splitk": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp, _size, _vp]),
    "fp8bs_gemm_splitk_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp]),
}

ROUTE_BS, ROUTE_MX, ROUTE_PT = 0, 1, 2
IN_F32, IN_BF16 = 0, 1
_IN_DTYPE = {torch.float32: IN_F32, torch.bfloat16: IN_BF16}


class Config(ctypes.Structure):
    """fp8bs_config of include/fp8bs.h."""
    _fields_ = [(n, ctypes.c_int) for n in
                ("block_m", "block_n", "waves_m", "waves_n", "stages", "group_m", "xcd_remap", "persistent",
                 "pingpong", "small_m", "c_store")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}

    def __repr__(self) -> str:
        return f"Config({self.as_dict()})"


class Fp8bsError(RuntimeError):
    """A libfp8bs call returned a non-zero status."""

    def __init__(self, name: str, status: int):
        self.status = status
        super().__init__(f"{name} failed with status {status}: {fp8bs_strerror(status)}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIBRARY):
        raise ImportError(
            f"libfp8bs is not built ({LIBRARY} missing); build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` from the repository root")
    handle = ctypes.CDLL(LIBRARY)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libfp8bs takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libfp8bs takes contiguous tensors only")
    return t.data_ptr()


# fp8 e4m3 codes may come as raw bytes or as torch's own e4m3 type (same bytes)
_CODE_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _expect(fn: str, arg: str, t: torch.Tensor, dtypes, shape=None, numel=None) -> None:
    """Raise ValueError unless t has one of `dtypes` and exactly `shape` (or `numel` elements,
    for the opaque prepared buffers). Checked before anything reaches the library, so a buffer
    of the wrong size or layout never becomes an out-of-bounds access on the device."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{fn}: {arg} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{fn}: {arg} has dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{fn}: {arg} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{fn}: {arg} has {t.numel()} elements, expected {numel}")


def _matrix(fn: str, arg: str, t: torch.Tensor, dtypes) -> tuple[int, int]:
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{fn}: {arg} must be a 2-D tensor")
    _expect(fn, arg, t, dtypes)
    return tuple(t.shape)


def _same_device(fn: str, *ts) -> None:
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"{fn}: tensors are on different devices {sorted(map(str, devs))}")


def _gemm_operands(fn: str, route: str, A, a_scale, B_prep, b_scale, C, packed_a: bool = True):
    """(M, N, K) after checking every operand of a GEMM entry point against A [M, K] and C [M, N]."""
    M, K = _matrix(fn, "A", A, _CODE_DTYPES)
    Mc, N = _matrix(fn, "C", C, (torch.bfloat16,))
    if Mc != M:
        raise ValueError(f"{fn}: C has {Mc} rows, A has {M}")
    _expect(fn, "B_prep", B_prep, _CODE_DTYPES, numel=N * K)
    # a shape the route rejects never reaches a kernel: the library returns FP8BS_E_SHAPE for it,
    # so the scale buffers are sized only for shapes it accepts
    if route == "bs":
        if K % 128 == 0 and N % 128 == 0:
            _expect(fn, "a_scale", a_scale, (torch.float32,), shape=(K // 128, M))
            _expect(fn, "b_scale", b_scale, (torch.float32,), shape=(N // 128, K // 128))
    elif route == "pt":
        _expect(fn, "a_scale", a_scale, (torch.float32,), shape=(M,))
        _expect(fn, "b_scale", b_scale, (torch.float32,), shape=(N,))
    elif K % 32 == 0:
        if packed_a:
            _expect(fn, "a_scale_packed", a_scale, (torch.uint8,), numel=M * (K // 32))
        else:
            _expect(fn, "a_e8m0", a_scale, (torch.uint8,), shape=(M, K // 32))
        _expect(fn, "b_scale_packed", b_scale, (torch.uint8,), numel=N * (K // 32))
    _same_device(fn, A, a_scale, B_prep, b_scale, C)
    return M, N, K


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(name: str, status: int) -> None:
    if status != 0:
        raise Fp8bsError(name, status)


# ---- raw ABI, same names as include/fp8bs.h --------------------------------------------------

def fp8bs_version() -> int:
    return lib.fp8bs_version()


def fp8bs_strerror(status: int) -> str:
    return lib.fp8bs_strerror(status).decode()


def fp8bs_prep_weight_bytes(N: int, K: int) -> int:
    return lib.fp8bs_prep_weight_bytes(N, K)


def fp8mx_packed_scale_bytes(rows: int, K: int) -> int:
    return lib.fp8mx_packed_scale_bytes(rows, K)


def fp8bs_prep_bytes(N: int, K: int) -> int:
    return lib.fp8bs_prep_bytes(N, K)


def fp8mx_scale_bytes(rows: int, K: int) -> int:
    return lib.fp8mx_scale_bytes(rows, K)


def fp8bs_prep_weights(B: torch.Tensor, B_prep: torch.Tensor, stream=None) -> None:
    N, K = _matrix("fp8bs_prep_weights", "B", B, _CODE_DTYPES)
    _expect("fp8bs_prep_weights", "B_prep", B_prep, _CODE_DTYPES, numel=N * K)
    _same_device("fp8bs_prep_weights", B, B_prep)
    _check("fp8bs_prep_weights", lib.fp8bs_prep_weights(_ptr(B), _ptr(B_prep), N, K, _stream(stream)))


def fp8bs_gemm(A: torch.Tensor, a_scale: torch.Tensor, B_prep: torch.Tensor, b_scale: torch.Tensor,
               C: torch.Tensor, stream=None) -> torch.Tensor:
    """C[M,N] (bf16) from A [M,K] (uint8 e4m3 codes), a_scale [K/128, M] fp32, B_prep from
    fp8bs_prep_weights of B [N,K], b_scale [N/128, K/128] fp32."""
    M, N, K = _gemm_operands("fp8bs_gemm", "bs", A, a_scale, B_prep, b_scale, C)
    _check("fp8bs_gemm", lib.fp8bs_gemm(_ptr(A), _ptr(a_scale), _ptr(B_prep), _ptr(b_scale), _ptr(C),
                                        M, N, K, _stream(stream)))
    return C


def fp8mx_pack_a_scale(a_e8m0: torch.Tensor, a_scale_packed: torch.Tensor, stream=None) -> None:
    M, G = _matrix("fp8mx_pack_a_scale", "a_e8m0", a_e8m0, (torch.uint8,))
    _expect("fp8mx_pack_a_scale", "a_scale_packed", a_scale_packed, (torch.uint8,), numel=M * G)
    _same_device("fp8mx_pack_a_scale", a_e8m0, a_scale_packed)
    _check("fp8mx_pack_a_scale", lib.fp8mx_pack_a_scale(_ptr(a_e8m0), _ptr(a_scale_packed), M, G * 32,
                                                        _stream(stream)))


def fp8mx_prep_weights(B: torch.Tensor, b_e8m0: torch.Tensor, B_prep: torch.Tensor,
                       b_scale_packed: torch.Tensor, stream=None) -> None:
    fn = "fp8mx_prep_weights"
    N, K = _matrix(fn, "B", B, _CODE_DTYPES)
    if K % 32:
        raise ValueError(f"{fn}: K ({K}) must be a multiple of 32")
    _expect(fn, "b_e8m0", b_e8m0, (torch.uint8,), shape=(N, K // 32))
    _expect(fn, "B_prep", B_prep, _CODE_DTYPES, numel=N * K)
    _expect(fn, "b_scale_packed", b_scale_packed, (torch.uint8,), numel=N * (K // 32))
    _same_device(fn, B, b_e8m0, B_prep, b_scale_packed)
    _check("fp8mx_prep_weights", lib.fp8mx_prep_weights(_ptr(B), _ptr(b_e8m0), _ptr(B_prep),
                                                        _ptr(b_scale_packed), N, K, _stream(stream)))


def fp8mx_gemm(A: torch.Tensor, a_scale_packed: torch.Tensor, B_prep: torch.Tensor,
               b_scale_packed: torch.Tensor, C: torch.Tensor, stream=None) -> torch.Tensor:
    M, N, K = _gemm_operands("fp8mx_gemm", "mx", A, a_scale_packed, B_prep, b_scale_packed, C)
    _check("fp8mx_gemm", lib.fp8mx_gemm(_ptr(A), _ptr(a_scale_packed), _ptr(B_prep), _ptr(b_scale_packed),
                                        _ptr(C), M, N, K, _stream(stream)))
    return C


def fp8pt_gemm(A: torch.Tensor, a_scale: torch.Tensor, B_prep: torch.Tensor, b_scale: torch.Tensor,
               C: torch.Tensor, stream=None) -> torch.Tensor:
    """Route PT (promote-free twin): C[M,N] (bf16) = a_scale[m] * b_scale[n] * (A B^T)[m,n] with
    A [M,K] uint8 e4m3 codes, a_scale [M] fp32, B_prep from fp8bs_prep_weights, b_scale [N] fp32."""
    M, N, K = _gemm_operands("fp8pt_gemm", "pt", A, a_scale, B_prep, b_scale, C)
    _check("fp8pt_gemm", lib.fp8pt_gemm(_ptr(A), _ptr(a_scale), _ptr(B_prep), _ptr(b_scale), _ptr(C),
                                        M, N, K, _stream(stream)))
    return C


def fp8pt_gemm_with_config(A, a_scale, B_prep, b_scale, C, config: Config, stream=None):
    M, N, K = _gemm_operands("fp8pt_gemm_with_config", "pt", A, a_scale, B_prep, b_scale, C)
    _check("fp8pt_gemm_with_config",
           lib.fp8pt_gemm_with_config(_ptr(A), _ptr(a_scale), _ptr(B_prep), _ptr(b_scale), _ptr(C), M, N, K,
                                      ctypes.byref(config), _stream(stream)))
    return C


def fp8bs_quantize_act(x: torch.Tensor, A_codes: torch.Tensor, a_scale: torch.Tensor, stream=None) -> None:
    """x [M,K] bf16/fp32 -> A_codes [M,K] uint8 e4m3, a_scale [K/128, M] fp32 (route BS)."""
    fn = "fp8bs_quantize_act"
    M, K = _matrix(fn, "x", x, tuple(_IN_DTYPE))
    if K % 128:
        raise ValueError(f"{fn}: K ({K}) must be a multiple of 128")
    _expect(fn, "A_codes", A_codes, _CODE_DTYPES, shape=(M, K))
    _expect(fn, "a_scale", a_scale, (torch.float32,), shape=(K // 128, M))
    _same_device(fn, x, A_codes, a_scale)
    _check("fp8bs_quantize_act", lib.fp8bs_quantize_act(_ptr(x), _IN_DTYPE.get(x.dtype, -1), _ptr(A_codes),
                                                        _ptr(a_scale), M, K, _stream(stream)))


def fp8mx_quantize_act(x: torch.Tensor, A_codes: torch.Tensor, a_e8m0: torch.Tensor, stream=None) -> None:
    """x [M,K] bf16/fp32 -> A_codes [M,K] uint8 e4m3, a_e8m0 [M, K/32] uint8 (route MX)."""
    fn = "fp8mx_quantize_act"
    M, K = _matrix(fn, "x", x, tuple(_IN_DTYPE))
    if K % 32:
        raise ValueError(f"{fn}: K ({K}) must be a multiple of 32")
    _expect(fn, "A_codes", A_codes, _CODE_DTYPES, shape=(M, K))
    _expect(fn, "a_e8m0", a_e8m0, (torch.uint8,), shape=(M, K // 32))
    _same_device(fn, x, A_codes, a_e8m0)
    _check("fp8mx_quantize_act", lib.fp8mx_quantize_act(_ptr(x), _IN_DTYPE.get(x.dtype, -1), _ptr(A_codes),
                                                        _ptr(a_e8m0), M, K, _stream(stream)))


def fp8mx_gemm_small_m(A: torch.Tensor, a_e8m0: torch.Tensor, B_prep: torch.Tensor, b_scale_packed: torch.Tensor,
                       C: torch.Tensor, stream=None) -> torch.Tensor:
    """Route MX through the small-M kernel (meant for few rows; any M): a_e8m0 [M, K/32] uint8
    row-major (not packed)."""
    M, N, K = _gemm_operands("fp8mx_gemm_small_m", "mx", A, a_e8m0, B_prep, b_scale_packed, C, packed_a=False)
    _check("fp8mx_gemm_small_m", lib.fp8mx_gemm_small_m(_ptr(A), _ptr(a_e8m0), _ptr(B_prep), _ptr(b_scale_packed),
                                                        _ptr(C), M, N, K, _stream(stream)))
    return C


def fp8bs_splitk_workspace_bytes(M: int, N: int, K: int, splits: int = 0) -> int:
    return lib.fp8bs_splitk_workspace_bytes(M, N, K, splits)


def fp8bs_gemm_splitk(A, a_scale, B_prep, b_scale, C, workspace: torch.Tensor | None, splits: int = 0,
                      stream=None) -> torch.Tensor:
    """Route BS with K split over `splits` workgroups per output tile (0: the library's choice);
    workspace: a device tensor of at least fp8bs_splitk_workspace_bytes(M, N, K, splits) bytes
    (None when the call does not split)."""
    M, N, K = _gemm_operands("fp8bs_gemm_splitk", "bs", A, a_scale, B_prep, b_scale, C)
    ws, nbytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
    _check("fp8bs_gemm_splitk", lib.fp8bs_gemm_splitk(_ptr(A), _ptr(a_scale), _ptr(B_prep), _ptr(b_scale), _ptr(C),
                                                      M, N, K, splits, ws, nbytes, _stream(stream)))
    return C


SPLITK_SCRATCH_BYTES = 32 << 20  # FP8BS_SPLITK_SCRATCH_BYTES of include/fp8bs.h


def fp8bs_gemm_splitk_noalloc(A, a_scale, B_prep, b_scale, C, splits: int = 0, stream=None) -> torch.Tensor:
    """fp8bs_gemm_splitk with the library's static scratch instead of a workspace (nothing is
    allocated; calls that overlap on one GPU race)."""
    M, N, K = _gemm_operands("fp8bs_gemm_splitk_noalloc", "bs", A, a_scale, B_prep, b_scale, C)
    _check("fp8bs_gemm_splitk_noalloc",
           lib.fp8bs_gemm_splitk_noalloc(_ptr(A), _ptr(a_scale), _ptr(B_prep), _ptr(b_scale), _ptr(C), M, N, K,
                                         splits, _stream(stream)))
    return C


def splitk_workspace(M: int, N: int, K: int, splits: int = 0, device="cuda") -> torch.Tensor | None:
    """A workspace tensor for fp8bs_gemm_splitk (None when the shape does not split)."""
    n = fp8bs_splitk_workspace_bytes(M, N, K, splits)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def fp8bs_select_config(route: int, M: int, N: int, K: int) -> Config:
    cfg = Config()
    _check("fp8bs_select_config", lib.fp8bs_select_config(route, M, N, K, ctypes.byref(cfg)))
    return cfg


def fp8bs_gemm_with_config(A, a_scale, B_prep, b_scale, C, config: Config, stream=None):
    M, N, K = _gemm_operands("fp8bs_gemm_with_config", "bs", A, a_scale, B_prep, b_scale, C)
    _check("fp8bs_gemm_with_config",
           lib.fp8bs_gemm_with_config(_ptr(A), _ptr(a_scale), _ptr(B_prep), _ptr(b_scale), _ptr(C), M, N, K,
                                      ctypes.byref(config), _stream(stream)))
    return C


def fp8mx_gemm_with_config(A, a_scale_packed, B_prep, b_scale_packed, C, config: Config, stream=None):
    M, N, K = _gemm_operands("fp8mx_gemm_with_config", "mx", A, a_scale_packed, B_prep, b_scale_packed, C)
    _check("fp8mx_gemm_with_config",
           lib.fp8mx_gemm_with_config(_ptr(A), _ptr(a_scale_packed), _ptr(B_prep), _ptr(b_scale_packed), _ptr(C),
                                      M, N, K, ctypes.byref(config), _stream(stream)))
    return C


def fp8bs_mfma_ceiling(A: torch.Tensor, B_prep: torch.Tensor, N: int, iters: int, sink: torch.Tensor,
                       stream=None) -> int:
    """Launch the matrix-core ceiling probe on A [M,K] and prepared weights of N rows; returns the
    FLOP count of the launch (time it with events on the stream)."""
    fn = "fp8bs_mfma_ceiling"
    M, K = _matrix(fn, "A", A, _CODE_DTYPES)
    _expect(fn, "B_prep", B_prep, _CODE_DTYPES)
    if B_prep.numel() < N * K:
        raise ValueError(f"{fn}: B_prep holds {B_prep.numel()} bytes, {N} weight rows need {N * K}")
    _expect(fn, "sink", sink, (torch.float32,))
    _same_device(fn, A, B_prep, sink)
    flops = ctypes.c_longlong(0)
    _check("fp8bs_mfma_ceiling", lib.fp8bs_mfma_ceiling(_ptr(A), _ptr(B_prep), M, N, K, iters, _ptr(sink),
                                                        sink.numel(), ctypes.byref(flops), _stream(stream)))
    return flops.value


LP_READS, LP_LOADS, LP_PROMOTE, LP_STORES, LP_BIG = 1, 2, 4, 8, 16


def fp8bs_loop_probe(parts: int, A: torch.Tensor, B_prep: torch.Tensor, N: int, steps: int, sink: torch.Tensor,
                     out: torch.Tensor | None = None, stream=None) -> int:
    """Launch the loop-skeleton probe (parts: a mask of the LP_* parts) on A [M,K] and prepared
    weights of N rows; returns the launch's matrix FLOP count (time it with events)."""
    fn = "fp8bs_loop_probe"
    M, K = _matrix(fn, "A", A, _CODE_DTYPES)
    _expect(fn, "B_prep", B_prep, _CODE_DTYPES)
    _expect(fn, "sink", sink, (torch.float32,))
    if out is not None:
        _same_device(fn, A, B_prep, sink, out)
    else:
        _same_device(fn, A, B_prep, sink)
    flops = ctypes.c_longlong(0)
    _check(fn, lib.fp8bs_loop_probe(parts, _ptr(A), _ptr(B_prep), M, N, K, steps,
                                    _ptr(out) if out is not None else None, out.numel() * out.element_size() if out is not None else 0,
                                    _ptr(sink), sink.numel(), ctypes.byref(flops), _stream(stream)))
    return flops.value


# ---- allocation helpers (torch owns the memory; the library never allocates) ----------------

def prep_weights(B: torch.Tensor, stream=None) -> torch.Tensor:
    """Prepared weight buffer for B [N,K] uint8 e4m3 codes (route BS)."""
    N, K = B.shape
    out = torch.empty(fp8bs_prep_weight_bytes(N, K), dtype=torch.uint8, device=B.device)
    fp8bs_prep_weights(B, out, stream)
    return out


def mx_prep_weights(B: torch.Tensor, b_e8m0: torch.Tensor, stream=None):
    """(prepared weights, packed weight scales) for route MX."""
    N, K = B.shape
    B_prep = torch.empty(fp8bs_prep_weight_bytes(N, K), dtype=torch.uint8, device=B.device)
    packed = torch.empty(fp8mx_packed_scale_bytes(N, K), dtype=torch.uint8, device=B.device)
    fp8mx_prep_weights(B, b_e8m0, B_prep, packed, stream)
    return B_prep, packed


def quantize_bs(x: torch.Tensor, stream=None):
    """(A codes [M,K] uint8, a_scale [K/128, M] fp32) for route BS from activations x."""
    M, K = x.shape
    A = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    sa = torch.empty((K // 128, M), dtype=torch.float32, device=x.device)
    fp8bs_quantize_act(x, A, sa, stream)
    return A, sa


def quantize_mx(x: torch.Tensor, stream=None):
    """(A codes [M,K] uint8, a_e8m0 [M, K/32] uint8) for route MX from activations x."""
    M, K = x.shape
    A = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    e8 = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    fp8mx_quantize_act(x, A, e8, stream)
    return A, e8


def mx_pack_a_scale(a_e8m0: torch.Tensor, stream=None) -> torch.Tensor:
    M, G = a_e8m0.shape
    packed = torch.empty(fp8mx_packed_scale_bytes(M, G * 32), dtype=torch.uint8, device=a_e8m0.device)
    fp8mx_pack_a_scale(a_e8m0, packed, stream)
    return packed
