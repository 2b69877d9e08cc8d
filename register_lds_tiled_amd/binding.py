"""ctypes binding of libsgemm_mi355x.so (the C ABI in include/sgemm.h).

Argument marshalling only: every arithmetic step runs in the library's HIP
kernels.  Functions keep the C names and argument order.  Matrix arguments
may be integer device addresses or torch CUDA tensors (their ``data_ptr()``
is passed); ``stream`` may be an integer hipStream_t, a ``torch.cuda.Stream``
or None (torch's current stream on the current device).

If the library has not been built, the first call raises ``RuntimeError``
naming the build command; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsgemm_mi355x.so")
LDSPOISON_LIB_PATH = os.path.join(HERE, "libsgemm_mi355x_ldspoison.so")

SGEMM_OK = 0
SGEMM_EINVAL_DIM = -1
SGEMM_EINVAL_LD = -2
SGEMM_EINVAL_PTR = -3
SGEMM_EALIAS = -4
SGEMM_EHIP = -5
SGEMM_EINVAL_PATH = -6
SGEMM_EINVAL_ACT = -7

ACT_NONE = 0
ACT_RELU = 1
ACTS = {"none": ACT_NONE, "relu": ACT_RELU}

PATH_AUTO = 0
PATH_VALU = 1
PATH_MFMA = 2
PATH_VALU_PAGE = 3
PATHS = {"auto": PATH_AUTO, "valu": PATH_VALU, "mfma": PATH_MFMA, "valu_page": PATH_VALU_PAGE}

EXPORTS = ("sgemm_f32", "sgemm_f32_path", "sgemm_f32_ex", "gemm_bf16_f32", "gemm_f16_f32",
           "sgemm_micro4x4_f32", "sgemm_f32_valu_tile", "sgemm_valu_tile_count",
           "sgemm_valu_tile_name", "sgemm_status_string", "sgemm_last_error",
           "sgemm_abi_version")

_lib = None
_lib_poison = None


class SgemmError(RuntimeError):
    def __init__(self, status: int, detail: str = ""):
        self.status = status
        msg = status_string(status)
        if detail:
            msg += f" [{detail}]"
        super().__init__(msg)


def _load(path: str):
    """ctypes handle of one build of the library, with the C signatures."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m register_lds_tiled_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    i, p = ctypes.c_int, ctypes.c_void_p
    gemm = [i, i, i, p, i, p, i, p, i, p]
    lib.sgemm_f32.argtypes = gemm
    lib.sgemm_f32.restype = i
    lib.sgemm_f32_path.argtypes = gemm + [i]
    lib.sgemm_f32_path.restype = i
    f = ctypes.c_float
    lib.sgemm_f32_ex.argtypes = [i, i, i, p, i, p, i, p, i, f, f, p, i, p]
    lib.sgemm_f32_ex.restype = i
    lib.gemm_bf16_f32.argtypes = gemm
    lib.gemm_bf16_f32.restype = i
    lib.gemm_f16_f32.argtypes = gemm
    lib.gemm_f16_f32.restype = i
    lib.sgemm_micro4x4_f32.argtypes = [i, p, p, p, p]
    lib.sgemm_micro4x4_f32.restype = i
    lib.sgemm_f32_valu_tile.argtypes = gemm + [i]
    lib.sgemm_f32_valu_tile.restype = i
    lib.sgemm_valu_tile_count.argtypes = []
    lib.sgemm_valu_tile_count.restype = i
    lib.sgemm_valu_tile_name.argtypes = [i]
    lib.sgemm_valu_tile_name.restype = ctypes.c_char_p
    lib.sgemm_status_string.argtypes = [i]
    lib.sgemm_status_string.restype = ctypes.c_char_p
    lib.sgemm_last_error.argtypes = []
    lib.sgemm_last_error.restype = ctypes.c_char_p
    lib.sgemm_abi_version.argtypes = []
    lib.sgemm_abi_version.restype = i
    return lib


def library():
    """Load (once) and return the ctypes handle of the HIP library."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def ldspoison_library():
    """Load (once) and return the handle of the debug build whose kernels
    poison every retired LDS stage with NaN before refilling it
    (libsgemm_mi355x_ldspoison.so, same C ABI).  For tests and debugging: a
    correct schedule gives results bit-identical to ``library()``'s."""
    global _lib_poison
    if _lib_poison is None:
        _lib_poison = _load(LDSPOISON_LIB_PATH)
    return _lib_poison


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    if hasattr(x, "data_ptr"):
        import torch
        if not x.is_cuda:
            raise ValueError("matrix tensors must live on the GPU")
        if x.dtype != torch.float32:
            raise TypeError("matrix tensors must be float32")
        return x.data_ptr() or None
    raise TypeError(f"cannot take a device address from {type(x).__name__}")


def _ptr16(x, fmt):
    """Device address of 16-bit storage: an int, or a CUDA tensor of dtype
    bfloat16 (fmt "bf16"), float16 (fmt "f16"), int16 or uint16."""
    if x is None or isinstance(x, int):
        return _ptr(x)
    if hasattr(x, "data_ptr"):
        import torch
        if not x.is_cuda:
            raise ValueError("matrix tensors must live on the GPU")
        ok = {"bf16": torch.bfloat16, "f16": torch.float16}[fmt]
        if x.dtype not in (ok, torch.int16, getattr(torch, "uint16", torch.int16)):
            raise TypeError(f"a {fmt} operand must be a {ok} (or 16-bit integer) tensor")
        return x.data_ptr() or None
    raise TypeError(f"cannot take a device address from {type(x).__name__}")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(s, int):
        return s or None
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream or None
    raise TypeError(f"cannot take a stream handle from {type(s).__name__}")


def _check(status: int) -> int:
    if status != SGEMM_OK:
        detail = library().sgemm_last_error().decode() if status == SGEMM_EHIP else ""
        raise SgemmError(status, detail)
    return status


def status_string(status: int) -> str:
    return library().sgemm_status_string(int(status)).decode()


def sgemm_status_string(status: int) -> str:
    return status_string(status)


def sgemm_last_error() -> str:
    return library().sgemm_last_error().decode()


def sgemm_abi_version() -> int:
    return library().sgemm_abi_version()


def sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None, *, check=True) -> int:
    """C = A.B (row-major fp32) on the library's default path."""
    st = library().sgemm_f32(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _stream(stream))
    return _check(st) if check else st


def sgemm_f32_path(M, N, K, A, lda, B, ldb, C, ldc, stream=None, path=PATH_AUTO, *,
                   check=True) -> int:
    """C = A.B (row-major fp32) on an explicit path (int or name in PATHS)."""
    path = PATHS[path] if isinstance(path, str) else int(path)
    st = library().sgemm_f32_path(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                                  _stream(stream), path)
    return _check(st) if check else st


def sgemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, alpha=1.0, beta=0.0, bias=None,
                 act=ACT_NONE, stream=None, *, check=True) -> int:
    """C = act(alpha * A.B + beta * C + bias[col]) (row-major fp32), fused into
    the matrix-core kernels' store; act is an int or a name in ACTS."""
    act = ACTS[act] if isinstance(act, str) else int(act)
    st = library().sgemm_f32_ex(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                                float(alpha), float(beta), _ptr(bias), act, _stream(stream))
    return _check(st) if check else st


def gemm_bf16_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None, *, check=True) -> int:
    """C = A.B with bfloat16 A and B (16-bit storage), fp32 accumulate and C."""
    st = library().gemm_bf16_f32(M, N, K, _ptr16(A, "bf16"), lda, _ptr16(B, "bf16"), ldb,
                                 _ptr(C), ldc, _stream(stream))
    return _check(st) if check else st


def gemm_f16_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None, *, check=True) -> int:
    """C = A.B with IEEE binary16 A and B, fp32 accumulate and C."""
    st = library().gemm_f16_f32(M, N, K, _ptr16(A, "f16"), lda, _ptr16(B, "f16"), ldb,
                                _ptr(C), ldc, _stream(stream))
    return _check(st) if check else st


def sgemm_micro4x4_f32(K, A, B, C, stream=None, *, check=True) -> int:
    """The one-thread 4x4 micro-GEMM: A 4xK (ld K), B Kx4 (ld 4), C 4x4."""
    st = library().sgemm_micro4x4_f32(K, _ptr(A), _ptr(B), _ptr(C), _stream(stream))
    return _check(st) if check else st


def sgemm_f32_valu_tile(M, N, K, A, lda, B, ldb, C, ldc, stream=None, tile=0, *,
                        check=True) -> int:
    """C = A.B (row-major fp32) on the VALU path at one built tile configuration."""
    st = library().sgemm_f32_valu_tile(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc,
                                       _stream(stream), int(tile))
    return _check(st) if check else st


def sgemm_valu_tile_count() -> int:
    return library().sgemm_valu_tile_count()


def sgemm_valu_tile_name(tile: int):
    r = library().sgemm_valu_tile_name(int(tile))
    return None if r is None else r.decode()


def valu_tiles():
    """{index: description} of the VALU path's built tile configurations."""
    return {t: sgemm_valu_tile_name(t) for t in range(sgemm_valu_tile_count())}


def matmul(A, B, out=None, path=PATH_AUTO, stream=None):
    """Tensor convenience over sgemm_f32_path: A (MxK) and B (KxN) float32
    CUDA tensors with unit column stride; returns (or fills) C (MxN)."""
    import torch
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"bad shapes {tuple(A.shape)} @ {tuple(B.shape)}")
    M, K = A.shape
    N = B.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    for name, X in (("A", A), ("B", B), ("out", out)):
        if X.numel() and X.shape[1] > 1 and X.stride(1) != 1:
            raise ValueError(f"{name} must have unit stride along its rows")
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    ld = lambda X: max(X.stride(0), X.shape[1], 1)  # noqa: E731
    sgemm_f32_path(M, N, K, A, ld(A), B, ld(B), out, ld(out), stream, path)
    return out
