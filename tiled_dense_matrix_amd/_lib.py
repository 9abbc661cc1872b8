"""ctypes binding of libtdm.so (the C ABI declared in include/tdm.h).

Argument marshalling only: every step of the product runs in the HIP
kernels behind the C ABI. Torch tensors supply device memory and the
current stream. There is no CPU fallback; if libtdm.so cannot be loaded the
calls raise.
"""
from __future__ import annotations

import ctypes
import enum
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtdm.so")

# The C ABI, as (name, restype, argtypes). Tests check that libtdm.so exports
# every function declared in include/tdm.h and nothing is missing here.
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


class Roofline(ctypes.Structure):
    _fields_ = [("flops", ctypes.c_double), ("bytes", ctypes.c_double),
                ("intensity", ctypes.c_double)]


SIGNATURES = {
    "gemm_f32": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _i64, _p]),
    "gemm_bf16_f32acc": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _i64, _p]),
    "gemm_roofline": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, ctypes.POINTER(Roofline)]),
    "tdm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tdm_gemm_f32_path": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _i64, ctypes.c_int, _p]),
    "gemm_f32_ex": (ctypes.c_int, [_p, _p, ctypes.c_int, _p, _i64, _i64, _i64, _p]),
    "tdm_gemm_f32_ex_path": (ctypes.c_int, [_p, _p, ctypes.c_int, _p, _i64, _i64, _i64,
                                            ctypes.c_int, _p]),
    "tdm_gemm_bf16_f32acc_path": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _i64, ctypes.c_int, _p]),
    "tdm_path_supports": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "tdm_select_path": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64]),
    "tdm_path_name": (ctypes.c_char_p, [ctypes.c_int]),
    "tdm_version": (ctypes.c_int, []),
    "gemm_bf16_epilogue": (ctypes.c_int, [_p, _p, _p, ctypes.c_int, _p, _p, ctypes.c_int,
                                          _i64, _i64, _i64, _p]),
    "tdm_gemm_bf16_epilogue_path": (ctypes.c_int, [_p, _p, _p, ctypes.c_int, _p, _p,
                                                   ctypes.c_int, _i64, _i64, _i64,
                                                   ctypes.c_int, _p]),
    "gemm_bf16_ex": (ctypes.c_int, [_p, _p, ctypes.c_int, _p, ctypes.c_int, _p, _p,
                                    ctypes.c_int, _i64, _i64, _i64, _p]),
    "tdm_gemm_bf16_ex_path": (ctypes.c_int, [_p, _p, ctypes.c_int, _p, ctypes.c_int, _p, _p,
                                             ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, _p]),
    "gemm_bf16_ex_noalloc": (ctypes.c_int, [_p, _p, ctypes.c_int, _p, ctypes.c_int, _p, _p,
                                            ctypes.c_int, _i64, _i64, _i64, _p]),
    "tdm_path_supports_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64,
                                            _i64, _i64, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int]),
    "tdm_select_path_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64]),
    "gemm_fp8": (ctypes.c_int, [_p, ctypes.c_int, _p, _p, ctypes.c_int, _p, _p, ctypes.c_int,
                                _p, _p, ctypes.c_int, _i64, _i64, _i64, _p]),
    "tdm_fp8_supports": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int]),
    "attention_fwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, ctypes.c_float,
                                     ctypes.c_int, _p]),
}


class Status(enum.IntEnum):
    SUCCESS = 0
    ERROR_INVALID_VALUE = 1
    ERROR_NOT_SUPPORTED = 2
    ERROR_NO_DEVICE = 3
    ERROR_LAUNCH = 4


class Kind(enum.IntEnum):
    F32 = 0
    BF16_F32ACC = 1


class Path(enum.IntEnum):
    AUTO = 0
    EDGE = 1
    VALU = 2
    MFMA = 3
    SKINNY = 4


class Layout(enum.IntEnum):
    """How A and B are stored (bit 0: B is N x K; bit 1: A is K x M)."""
    KN = 0     # A M x K, B K x N: C = A @ B
    NK = 1     # B N x K (a torch Linear weight): C = A @ B.T
    KM_KN = 2  # A K x M: C = A.T @ B
    KM_NK = 3  # A K x M, B N x K: C = A.T @ B.T


class DType(enum.IntEnum):
    F32 = 0
    BF16 = 1


class Fp8Format(enum.IntEnum):
    """FP8 element formats: E4M3 (range +-448) and E5M2 (range +-57344)."""
    E4M3 = 0
    E5M2 = 1


class TdmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = Status(status) if status in Status._value2member_map_ else status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lock = threading.Lock()
_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libtdm.so (building it first if it has never been built)."""
    global _lib
    with _lock:
        if _lib is None:
            lib_path = path or LIB_PATH
            if not os.path.exists(lib_path):
                from . import build as _build
                _build.build(verbose=False)
            lib = ctypes.CDLL(lib_path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().tdm_status_string(int(status)).decode()


def path_name(path: int) -> str:
    return load().tdm_path_name(int(path)).decode()


def version() -> int:
    return load().tdm_version()


def gemm_roofline(kind: int, M: int, N: int, K: int) -> Roofline:
    out = Roofline()
    st = load().gemm_roofline(int(kind), M, N, K, ctypes.byref(out))
    if st != Status.SUCCESS:
        raise TdmError(st, "gemm_roofline")
    return out


def tdm_select_path(kind: int, M: int, N: int, K: int) -> Path:
    return Path(load().tdm_select_path(int(kind), M, N, K))


def tdm_path_supports(kind: int, path: int, M: int, N: int, K: int,
                      misalign_a: int = 0, misalign_b: int = 0, misalign_c: int = 0) -> bool:
    return bool(load().tdm_path_supports(int(kind), int(path), M, N, K,
                                         misalign_a, misalign_b, misalign_c))


# ---------------------------------------------------------------------------
# Torch-facing wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(stream) -> int | None:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _check_matrix(name: str, t, dtypes, rows: int | None = None, cols: int | None = None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major); call .contiguous()")
    if rows is not None and t.shape[0] != rows:
        raise ValueError(f"{name} has {t.shape[0]} rows, expected {rows}")
    if cols is not None and t.shape[1] != cols:
        raise ValueError(f"{name} has {t.shape[1]} columns, expected {cols}")


def _prep(A, B, C, in_dtypes):
    torch = _torch()
    _check_matrix("A", A, in_dtypes)
    M, K = A.shape
    _check_matrix("B", B, in_dtypes, rows=K)
    N = B.shape[1]
    if A.device != B.device:
        raise ValueError("A and B are on different devices")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    else:
        _check_matrix("C", C, (torch.float32,), rows=M, cols=N)
        if C.device != A.device:
            raise ValueError("C is on another device than A and B")
    return M, N, K, C


def _call(fname: str, A, B, C, M, N, K, stream, path=None):
    torch = _torch()
    lib = load()
    fn = getattr(lib, fname)
    with torch.cuda.device(A.device):
        args = [A.data_ptr() or None, B.data_ptr() or None, C.data_ptr() or None, M, N, K]
        if path is not None:
            args.append(int(path))
        args.append(_stream_handle(stream))
        st = fn(*args)
    if st != Status.SUCCESS:
        raise TdmError(st, fname)
    return C


def gemm_f32(A, B, C=None, stream=None):
    """C = A @ B for fp32 A[M,K], B[K,N] (row-major CUDA tensors). Returns C."""
    torch = _torch()
    M, N, K, C = _prep(A, B, C, (torch.float32,))
    return _call("gemm_f32", A, B, C, M, N, K, stream)


def gemm_bf16_f32acc(A, B, C=None, stream=None):
    """C = A @ B for bf16 A, B (torch.bfloat16 or raw int16/uint16 bits); fp32 C."""
    torch = _torch()
    M, N, K, C = _prep(A, B, C, _bf16_dtypes())
    return _call("gemm_bf16_f32acc", A, B, C, M, N, K, stream)


def tdm_gemm_f32_path(A, B, C=None, path=Path.AUTO, stream=None):
    torch = _torch()
    M, N, K, C = _prep(A, B, C, (torch.float32,))
    return _call("tdm_gemm_f32_path", A, B, C, M, N, K, stream, path)


def _prep_layout(A, B, C, layout, in_dtypes):
    """Shapes of op(A) @ op(B) for A, B stored as `layout` says; returns
    (M, N, K, C)."""
    torch = _torch()
    layout = Layout(layout)
    _check_matrix("A", A, in_dtypes)
    K, M = A.shape if layout & Layout.KM_KN else A.shape[::-1]
    if layout & Layout.NK:
        _check_matrix("B", B, in_dtypes, cols=K)
        N = B.shape[0]
    else:
        _check_matrix("B", B, in_dtypes, rows=K)
        N = B.shape[1]
    if A.device != B.device:
        raise ValueError("A and B are on different devices")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    else:
        _check_matrix("C", C, (torch.float32,), rows=M, cols=N)
        if C.device != A.device:
            raise ValueError("C is on another device than A and B")
    return M, N, K, C


def _call_layout(fname: str, A, B, layout, C, M, N, K, stream, path=None):
    torch = _torch()
    fn = getattr(load(), fname)
    with torch.cuda.device(A.device):
        args = [A.data_ptr() or None, B.data_ptr() or None, int(layout), C.data_ptr() or None,
                M, N, K]
        if path is not None:
            args.append(int(path))
        args.append(_stream_handle(stream))
        st = fn(*args)
    if st != Status.SUCCESS:
        raise TdmError(st, fname)
    return C


def gemm_f32_ex(A, B, layout=Layout.KN, C=None, stream=None):
    """C = op(A) @ op(B) for fp32 A, B: op(A) = A.T when A is stored K x M
    (Layout.KM_KN, Layout.KM_NK), op(B) = B.T when B is stored N x K
    (Layout.NK, Layout.KM_NK). Returns C (M x N, fp32)."""
    torch = _torch()
    M, N, K, C = _prep_layout(A, B, C, layout, (torch.float32,))
    return _call_layout("gemm_f32_ex", A, B, layout, C, M, N, K, stream)


def tdm_gemm_f32_ex_path(A, B, layout=Layout.KN, C=None, path=Path.AUTO, stream=None):
    torch = _torch()
    M, N, K, C = _prep_layout(A, B, C, layout, (torch.float32,))
    return _call_layout("tdm_gemm_f32_ex_path", A, B, layout, C, M, N, K, stream, path)


def tdm_gemm_bf16_f32acc_path(A, B, C=None, path=Path.AUTO, stream=None):
    M, N, K, C = _prep(A, B, C, _bf16_dtypes())
    return _call("tdm_gemm_bf16_f32acc_path", A, B, C, M, N, K, stream, path)


def _epilogue_args(A, B, D, out_dtype, bias, residual, layout=Layout.KN):
    """Check the epilogue operands; returns (M, N, K, D, DType)."""
    torch = _torch()
    bf16 = _bf16_dtypes()
    _check_matrix("A", A, bf16)
    layout = Layout(layout)
    K, M = A.shape if layout & Layout.KM_KN else A.shape[::-1]
    if layout & Layout.NK:
        _check_matrix("B", B, bf16, cols=K)
        N = B.shape[0]
    else:
        _check_matrix("B", B, bf16, rows=K)
        N = B.shape[1]
    if A.device != B.device:
        raise ValueError("A and B are on different devices")
    if D is None:
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
        D = torch.empty((M, N), dtype=out_dtype, device=A.device)
    dt = DType.F32 if D.dtype == torch.float32 else DType.BF16
    same = (torch.float32,) if dt == DType.F32 else bf16
    _check_matrix("D", D, same, rows=M, cols=N)
    if D.device != A.device:
        raise ValueError("D is on another device than A and B")
    if bias is not None:
        if not isinstance(bias, torch.Tensor) or bias.dim() != 1 or bias.shape[0] != N:
            raise ValueError(f"bias must be a 1-D tensor of {N} elements")
        if bias.dtype not in same or not bias.is_cuda or not bias.is_contiguous() \
                or bias.device != A.device:
            raise ValueError("bias must be a contiguous tensor of D's element type on A's device")
    if residual is not None:
        _check_matrix("residual", residual, same, rows=M, cols=N)
        if residual.device != A.device:
            raise ValueError("residual is on another device than A and B")
    return M, N, K, D, dt


def _call_epilogue(fname, A, B, D, dt, bias, residual, gelu, M, N, K, stream, path=None):
    torch = _torch()
    fn = getattr(load(), fname)
    with torch.cuda.device(A.device):
        args = [A.data_ptr() or None, B.data_ptr() or None, D.data_ptr() or None, int(dt),
                None if bias is None else bias.data_ptr(),
                None if residual is None else residual.data_ptr(),
                1 if gelu else 0, M, N, K]
        if path is not None:
            args.append(int(path))
        args.append(_stream_handle(stream))
        st = fn(*args)
    if st != Status.SUCCESS:
        raise TdmError(st, fname)
    return D


def gemm_bf16_epilogue(A, B, D=None, out_dtype=None, bias=None, residual=None, gelu=False,
                       stream=None):
    """D = epilogue(A @ B) for bf16 A, B: + bias[j], then GELU (exact, erf), then
    + residual[i, j], stored as D's dtype (torch.float32 or bf16). Without D, a
    new tensor of out_dtype (default torch.bfloat16) is returned."""
    torch = _torch()
    M, N, K, D, dt = _epilogue_args(A, B, D, out_dtype or torch.bfloat16, bias, residual)
    return _call_epilogue("gemm_bf16_epilogue", A, B, D, dt, bias, residual, gelu, M, N, K, stream)


def tdm_gemm_bf16_epilogue_path(A, B, D=None, out_dtype=None, bias=None, residual=None,
                                gelu=False, path=Path.AUTO, stream=None):
    torch = _torch()
    M, N, K, D, dt = _epilogue_args(A, B, D, out_dtype or torch.bfloat16, bias, residual)
    return _call_epilogue("tdm_gemm_bf16_epilogue_path", A, B, D, dt, bias, residual, gelu,
                          M, N, K, stream, path)


def gemm_bf16_ex(A, B, layout=Layout.KN, D=None, out_dtype=None, bias=None, residual=None,
                 gelu=False, stream=None):
    """D = epilogue(op(A) @ op(B)) for bf16 A, B: op(B) = B.T when B is
    stored N x K (Layout.NK, Layout.KM_NK; like a torch Linear weight), op(A)
    = A.T when A is stored K x M (Layout.KM_KN, Layout.KM_NK). The epilogue
    is gemm_bf16_epilogue's; without D a new tensor of out_dtype (default
    torch.bfloat16) is returned."""
    torch = _torch()
    M, N, K, D, dt = _epilogue_args(A, B, D, out_dtype or torch.bfloat16, bias, residual, layout)
    return _call_ex("gemm_bf16_ex", A, B, layout, D, dt, bias, residual, gelu, M, N, K, stream)


def gemm_bf16_ex_noalloc(A, B, layout=Layout.KN, D=None, out_dtype=None, bias=None,
                         residual=None, gelu=False, stream=None):
    """gemm_bf16_ex through the entry point that allocates nothing: the
    small-M K x N partial sums use the library's one static buffer per GPU
    (calls that overlap in time on one GPU race). Pass D to keep the call
    itself free of allocation; without D a new tensor is returned."""
    torch = _torch()
    M, N, K, D, dt = _epilogue_args(A, B, D, out_dtype or torch.bfloat16, bias, residual, layout)
    return _call_ex("gemm_bf16_ex_noalloc", A, B, layout, D, dt, bias, residual, gelu, M, N, K,
                    stream)


def tdm_gemm_bf16_ex_path(A, B, layout=Layout.KN, D=None, out_dtype=None, bias=None,
                          residual=None, gelu=False, path=Path.AUTO, stream=None):
    torch = _torch()
    M, N, K, D, dt = _epilogue_args(A, B, D, out_dtype or torch.bfloat16, bias, residual, layout)
    return _call_ex("tdm_gemm_bf16_ex_path", A, B, layout, D, dt, bias, residual, gelu, M, N, K,
                    stream, path)


def _call_ex(fname, A, B, layout, D, dt, bias, residual, gelu, M, N, K, stream, path=None):
    torch = _torch()
    fn = getattr(load(), fname)
    with torch.cuda.device(A.device):
        args = [A.data_ptr() or None, B.data_ptr() or None, int(layout), D.data_ptr() or None,
                int(dt), None if bias is None else bias.data_ptr(),
                None if residual is None else residual.data_ptr(), 1 if gelu else 0, M, N, K]
        if path is not None:
            args.append(int(path))
        args.append(_stream_handle(stream))
        st = fn(*args)
    if st != Status.SUCCESS:
        raise TdmError(st, fname)
    return D


def tdm_path_supports_ex(kind: int, layout: int, path: int, M: int, N: int, K: int,
                         misalign_a: int = 0, misalign_b: int = 0, misalign_c: int = 0) -> bool:
    return bool(load().tdm_path_supports_ex(int(kind), int(layout), int(path), M, N, K,
                                            misalign_a, misalign_b, misalign_c))


def tdm_select_path_ex(kind: int, layout: int, M: int, N: int, K: int) -> Path:
    return Path(load().tdm_select_path_ex(int(kind), int(layout), M, N, K))


def _bf16_dtypes():
    torch = _torch()
    dts = [torch.bfloat16, torch.int16]
    if hasattr(torch, "uint16"):
        dts.append(torch.uint16)
    return tuple(dts)


# ---------------------------------------------------------------------------
# FP8
# ---------------------------------------------------------------------------

def _fp8_format(name: str, t, fmt):
    """The format of an FP8 operand: given, or taken from a torch float8 dtype
    (raw uint8 codes default to E4M3)."""
    torch = _torch()
    from_dtype = {getattr(torch, "float8_e4m3fn", None): Fp8Format.E4M3,
                  getattr(torch, "float8_e5m2", None): Fp8Format.E5M2}.get(t.dtype)
    if fmt is None:
        return from_dtype if from_dtype is not None else Fp8Format.E4M3
    fmt = Fp8Format(fmt)
    if from_dtype is not None and from_dtype != fmt:
        raise ValueError(f"{name} has dtype {t.dtype} but format {fmt.name} was given")
    return fmt


def _fp8_dtypes():
    torch = _torch()
    dts = [torch.uint8]
    for n in ("float8_e4m3fn", "float8_e5m2"):
        if hasattr(torch, n):
            dts.append(getattr(torch, n))
    return tuple(dts)


def gemm_fp8(A, B, a_format=None, b_format=None, a_scale=None, b_scale=None, D=None,
             out_dtype=None, bias=None, residual=None, gelu=False, stream=None):
    """D = epilogue(A @ B.T) for FP8 A [M, K] and B [N, K] (uint8 codes or torch
    float8 tensors; a uint8 operand is E4M3 unless its format is given).
    a_scale [M, K/32] and b_scale [N, K/32] (uint8 exponents e, factor
    2^(e-127) per 32 k of a row) come together or not at all. The epilogue
    and D are as in gemm_bf16_epilogue; without D a new tensor of out_dtype
    (default torch.bfloat16) is returned."""
    torch = _torch()
    fp8 = _fp8_dtypes()
    _check_matrix("A", A, fp8)
    M, K = A.shape
    _check_matrix("B", B, fp8, cols=K)
    N = B.shape[0]
    fa, fb = _fp8_format("A", A, a_format), _fp8_format("B", B, b_format)
    if A.device != B.device:
        raise ValueError("A and B are on different devices")
    if (a_scale is None) != (b_scale is None):
        raise ValueError("a_scale and b_scale come together")
    if a_scale is not None:
        if K % 32:
            raise ValueError("block scales need K a multiple of 32")
        _check_matrix("a_scale", a_scale, (torch.uint8,), rows=M, cols=K // 32)
        _check_matrix("b_scale", b_scale, (torch.uint8,), rows=N, cols=K // 32)
        if a_scale.device != A.device or b_scale.device != A.device:
            raise ValueError("scales are on another device than A and B")
    bf16 = _bf16_dtypes()
    if D is None:
        out_dtype = out_dtype or torch.bfloat16
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
        D = torch.empty((M, N), dtype=out_dtype, device=A.device)
    dt = DType.F32 if D.dtype == torch.float32 else DType.BF16
    same = (torch.float32,) if dt == DType.F32 else bf16
    _check_matrix("D", D, same, rows=M, cols=N)
    if D.device != A.device:
        raise ValueError("D is on another device than A and B")
    if bias is not None:
        if not isinstance(bias, torch.Tensor) or bias.dim() != 1 or bias.shape[0] != N:
            raise ValueError(f"bias must be a 1-D tensor of {N} elements")
        if bias.dtype not in same or not bias.is_cuda or not bias.is_contiguous() \
                or bias.device != A.device:
            raise ValueError("bias must be a contiguous tensor of D's element type on A's device")
    if residual is not None:
        _check_matrix("residual", residual, same, rows=M, cols=N)
        if residual.device != A.device:
            raise ValueError("residual is on another device than A and B")
    fn = load().gemm_fp8
    with torch.cuda.device(A.device):
        st = fn(A.data_ptr() or None, int(fa), None if a_scale is None else a_scale.data_ptr(),
                B.data_ptr() or None, int(fb), None if b_scale is None else b_scale.data_ptr(),
                D.data_ptr() or None, int(dt), None if bias is None else bias.data_ptr(),
                None if residual is None else residual.data_ptr(), 1 if gelu else 0, M, N, K,
                _stream_handle(stream))
    if st != Status.SUCCESS:
        raise TdmError(st, "gemm_fp8")
    return D


def tdm_fp8_supports(M: int, N: int, K: int, misalign_a: int = 0, misalign_b: int = 0) -> bool:
    return bool(load().tdm_fp8_supports(M, N, K, misalign_a, misalign_b))


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def attention_fwd(Q, K, V, causal=False, scale=None, O=None, return_lse=False, stream=None):
    """O = softmax(Q K^T * scale) V per (batch, head) for bf16 tensors
    Q [..., n_q, d], K and V [..., n_kv, d] (same leading dimensions,
    contiguous); scale defaults to 1/sqrt(d). Returns O (bf16, Q's shape), or
    (O, lse) with the fp32 row logsumexp [..., n_q] when return_lse."""
    torch = _torch()
    bf16 = _bf16_dtypes()
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if not isinstance(t, torch.Tensor) or t.dim() < 2:
            raise ValueError(f"{name} must be a tensor of at least 2 dimensions")
        if t.dtype not in bf16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor on a GPU")
    lead, (n_q, d) = Q.shape[:-2], Q.shape[-2:]
    if K.shape[:-2] != lead or V.shape != K.shape or K.shape[-1] != d:
        raise ValueError(f"shapes do not match: Q {tuple(Q.shape)}, K {tuple(K.shape)}, "
                         f"V {tuple(V.shape)}")
    if K.device != Q.device or V.device != Q.device:
        raise ValueError("Q, K and V are on different devices")
    n_kv = K.shape[-2]
    bh = 1
    for x in lead:
        bh *= x
    if O is None:
        O = torch.empty(Q.shape, dtype=torch.bfloat16, device=Q.device)
    elif O.shape != Q.shape or O.dtype not in bf16 or not O.is_contiguous() or O.device != Q.device:
        raise ValueError("O must be a contiguous bf16 tensor shaped like Q, on Q's device")
    lse = torch.empty(tuple(lead) + (n_q,), dtype=torch.float32, device=Q.device) \
        if return_lse else None
    sc = float(d) ** -0.5 if scale is None else float(scale)
    fn = load().attention_fwd
    with torch.cuda.device(Q.device):
        st = fn(Q.data_ptr() or None, K.data_ptr() or None, V.data_ptr() or None,
                O.data_ptr() or None, None if lse is None else lse.data_ptr(), bh, n_q, n_kv, d,
                sc, 1 if causal else 0, _stream_handle(stream))
    if st != Status.SUCCESS:
        raise TdmError(st, "attention_fwd")
    return (O, lse) if return_lse else O
