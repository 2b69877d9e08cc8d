"""CPU oracle for row-major single-precision GEMM -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library in
``register_lds_tiled_amd``) never imports, links or calls it, and the two share
no code: the only module both sides use is the seeded input generator
``register_lds_tiled_amd.workloads``, which holds none of the method's
arithmetic.

The arithmetic lives in ``sgemm_ref.c`` (plain C, built by gcc with
``-O2 -ffp-contract=off -fopenmp``, no fast-math):

* ``sgemm_ref_f64``         C[i,j] = sum_k A[i,k] B[k,j] in double, ascending k
  -- the product's definition ("Micro Kernel 입문하기",
  teach-meaning.tistory.com/1544, walkthrough section 2; row-major layouts from
  its sections 3-1, 3-2 and 4; ``ldc`` from "누산 개념을 Grid-Block-Warp-Thread
  계층에 끼워넣기", teach-meaning.tistory.com/1518, section 2).
* ``sgemm_ref_f64_entries`` the same sum for chosen (i, j) only.
* ``micro4x4_seq_fma_f32``  the first page's one-thread 4x4 micro-GEMM in fp32
  with one fused multiply-add per k (page 1 section 2; the fused form is the
  ``fmaf`` of "gemm_tiled_test", teach-meaning.tistory.com/1542, section 5).
* ``sgemm_ex_ref_f64``      the product followed by the fused epilogue
  act(alpha * S + beta * C_in + bias[j]) that the tiled page's original
  kernel carries (its opening paragraph; reading in the C source).
* ``sgemm_ex_ref_f64_entries``  selected entries of the same, one by one.
* ``decode16_f32``, ``gemm_lowp_ref_f64``  16-bit inputs (bfloat16 or IEEE
  binary16) decoded to their exact values, then the same ascending-k double
  sum.

Pins (tests/test_oracle.py): the first page's printed worked-example output,
exact rational sums on tiny shapes, integer-valued inputs against exact integer
products, identity / zero / ones / transpose invariants and a float64 library
product; the epilogue against exact integer arithmetic, exact power-of-two
scaling and its special cases (K = 0, beta = 0 with NaN in C_in, NaN through
ReLU); the 16-bit decoders exhaustively against numpy's binary16 and the
bfloat16 bit definition, and the 16-bit product against exact integer
arithmetic and the float32 oracle on the decoded values.  No function here is
"parity unpinned".

``parity`` applies the acceptance rule max|C - C_ref| <= 1e-4 * max|C_ref|
(NaN anywhere fails; an all-zero reference demands an exact zero result).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgemm_ref.c")
_LIB = os.path.join(_HERE, "libsgemm_ref.so")

REL_TOL = 1e-4
_default = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle library (always recompiles)."""
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    "-Wall", "-Wextra", src, "-o", out, "-lm"], check=True)
    return out


def _rowmajor_f32(X: np.ndarray, name: str):
    """Return (array, leading dimension in elements) for a 2-D float32 array
    whose rows are unit-stride (a row slice of a larger matrix is fine)."""
    if not isinstance(X, np.ndarray) or X.dtype != np.float32 or X.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 numpy array")
    rows, cols = X.shape
    if ((cols > 1 and X.strides[1] != 4) or
            (rows > 1 and (X.strides[0] % 4 or X.strides[0] // 4 < cols))):
        X = np.ascontiguousarray(X)
    ld = X.strides[0] // 4 if rows > 1 else cols
    return X, max(ld, 1)


class OracleLib:
    """ctypes wrapper around one build of ``sgemm_ref.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i, ll, p = ctypes.c_int, ctypes.c_longlong, ctypes.c_void_p
        lib.sgemm_ref_f64.argtypes = [i, i, i, p, ll, p, ll, p, ll]
        lib.sgemm_ref_f64.restype = None
        lib.sgemm_ref_f64_entries.argtypes = [i, p, ll, p, ll, ll, p, p, p]
        lib.sgemm_ref_f64_entries.restype = None
        lib.micro4x4_seq_fma_f32.argtypes = [i, p, p, p]
        lib.micro4x4_seq_fma_f32.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i
        d = ctypes.c_double
        lib.sgemm_ex_ref_f64.argtypes = [i, i, i, p, ll, p, ll, p, ll, d, d, p, i, p, ll]
        lib.sgemm_ex_ref_f64.restype = None
        lib.sgemm_ex_ref_f64_entries.argtypes = [i, p, ll, p, ll, p, ll, d, d, p, i, ll, p, p, p]
        lib.sgemm_ex_ref_f64_entries.restype = None
        lib.decode16_f32.argtypes = [i, ll, p, p]
        lib.decode16_f32.restype = None
        lib.gemm_lowp_ref_f64.argtypes = [i, i, i, p, ll, p, ll, i, p, ll]
        lib.gemm_lowp_ref_f64.restype = i
        self._lib = lib
        self.path = path

    def num_threads(self) -> int:
        return self._lib.oracle_num_threads()

    def sgemm_ref_f64(self, A: np.ndarray, B: np.ndarray) -> np.ndarray:
        """C = A @ B in float64 by the ascending-k definition."""
        A, lda = _rowmajor_f32(A, "A")
        B, ldb = _rowmajor_f32(B, "B")
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ")
        C = np.empty((M, N), dtype=np.float64)
        if M and N:
            self._lib.sgemm_ref_f64(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                    C.ctypes.data, N)
        return C

    def sgemm_ref_f64_entries(self, A: np.ndarray, B: np.ndarray, rows, cols) -> np.ndarray:
        """C[rows[t], cols[t]] of A @ B, each by the ascending-k double sum."""
        A, lda = _rowmajor_f32(A, "A")
        B, ldb = _rowmajor_f32(B, "B")
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ")
        rows, cols = _entry_indices(rows, cols, M, N)
        out = np.empty(rows.size, dtype=np.float64)
        if rows.size:
            self._lib.sgemm_ref_f64_entries(K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                            rows.size, rows.ctypes.data, cols.ctypes.data,
                                            out.ctypes.data)
        return out

    @staticmethod
    def _epilogue_operands(M, N, C_in, beta, bias, act):
        """Checked (C_in, ldc, bias) for the epilogue functions; C_in is
        passed only when beta != 0, as the C code reads it only then."""
        if act not in (0, 1):
            raise ValueError("act must be 0 (identity) or 1 (ReLU)")
        ldc = max(N, 1)
        if beta != 0.0:
            if C_in is None or C_in.shape != (M, N):
                raise ValueError("beta != 0 needs C_in of shape (M, N)")
            C_in, ldc = _rowmajor_f32(C_in, "C_in")
        else:
            C_in = None
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32)
            if bias.shape != (N,):
                raise ValueError("bias must have shape (N,)")
        return C_in, ldc, bias

    def sgemm_ex_ref_f64(self, A: np.ndarray, B: np.ndarray, C_in=None, alpha: float = 1.0,
                         beta: float = 0.0, bias=None, act: int = 0) -> np.ndarray:
        """act(alpha * A @ B + beta * C_in + bias[j]) in float64 (see the C
        source for the epilogue reading).  C_in is read only if beta != 0;
        bias is a length-N float32 vector or None; act 0 = identity, 1 = ReLU."""
        A, lda = _rowmajor_f32(A, "A")
        B, ldb = _rowmajor_f32(B, "B")
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ")
        C_in, ldc, bias = self._epilogue_operands(M, N, C_in, beta, bias, act)
        out = np.empty((M, N), dtype=np.float64)
        if M and N:
            self._lib.sgemm_ex_ref_f64(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                       _addr(C_in), ldc, float(alpha), float(beta), _addr(bias),
                                       act, out.ctypes.data, N)
        return out

    def sgemm_ex_ref_f64_entries(self, A: np.ndarray, B: np.ndarray, rows, cols, C_in=None,
                                 alpha: float = 1.0, beta: float = 0.0, bias=None,
                                 act: int = 0) -> np.ndarray:
        """Entries (rows[t], cols[t]) of ``sgemm_ex_ref_f64``'s result, each
        computed on its own (for products too large to form whole)."""
        A, lda = _rowmajor_f32(A, "A")
        B, ldb = _rowmajor_f32(B, "B")
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ")
        rows, cols = _entry_indices(rows, cols, M, N)
        C_in, ldc, bias = self._epilogue_operands(M, N, C_in, beta, bias, act)
        out = np.empty(rows.size, dtype=np.float64)
        if rows.size:
            self._lib.sgemm_ex_ref_f64_entries(K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                               _addr(C_in), ldc, float(alpha), float(beta),
                                               _addr(bias), act, rows.size, rows.ctypes.data,
                                               cols.ctypes.data, out.ctypes.data)
        return out

    def decode16_f32(self, X: np.ndarray, fmt: str) -> np.ndarray:
        """Exact float32 values of 16-bit storage X (uint16) in format fmt
        ("bf16" or "f16")."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        out = np.empty(X.shape, dtype=np.float32)
        if X.size:
            self._lib.decode16_f32(LOWP_FORMATS[fmt], X.size, X.ctypes.data, out.ctypes.data)
        return out

    def gemm_lowp_ref_f64(self, A: np.ndarray, B: np.ndarray, fmt: str) -> np.ndarray:
        """C = A @ B in float64 for 16-bit A (MxK) and B (KxN) given as uint16
        storage in format fmt, by the ascending-k definition over the decoded
        values."""
        A, lda = _rowmajor_u16(A, "A")
        B, ldb = _rowmajor_u16(B, "B")
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ")
        C = np.empty((M, N), dtype=np.float64)
        if M and N:
            if self._lib.gemm_lowp_ref_f64(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                           LOWP_FORMATS[fmt], C.ctypes.data, N) != 0:
                raise MemoryError("oracle could not allocate its decoded copies")
        return C

    def micro4x4_seq_fma_f32(self, A: np.ndarray, B: np.ndarray) -> np.ndarray:
        """The first page's one-thread 4x4 micro-GEMM in fp32 fused arithmetic."""
        A = np.ascontiguousarray(A, dtype=np.float32)
        B = np.ascontiguousarray(B, dtype=np.float32)
        if (A.ndim != 2 or A.shape[0] != 4 or B.ndim != 2 or B.shape[1] != 4
                or A.shape[1] != B.shape[0]):
            raise ValueError("micro-GEMM takes A of shape (4, K) and B of shape (K, 4)")
        C = np.empty((4, 4), dtype=np.float32)
        self._lib.micro4x4_seq_fma_f32(A.shape[1], A.ctypes.data, B.ctypes.data, C.ctypes.data)
        return C


LOWP_FORMATS = {"bf16": 1, "f16": 2}


def _rowmajor_u16(X: np.ndarray, name: str):
    """As _rowmajor_f32, for 2-D uint16 arrays of 16-bit storage."""
    if not isinstance(X, np.ndarray) or X.dtype != np.uint16 or X.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint16 numpy array of 16-bit storage")
    rows, cols = X.shape
    if ((cols > 1 and X.strides[1] != 2) or
            (rows > 1 and (X.strides[0] % 2 or X.strides[0] // 2 < cols))):
        X = np.ascontiguousarray(X)
    ld = X.strides[0] // 2 if rows > 1 else cols
    return X, max(ld, 1)


def _addr(x):
    return None if x is None else x.ctypes.data


def _entry_indices(rows, cols, M, N):
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise IndexError("entry index out of range")
    return rows, cols


def default() -> OracleLib:
    """The oracle built from ``sgemm_ref.c`` in this directory (built on
    first use if missing or older than its source)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _default = OracleLib(_LIB)
    return _default


def num_threads() -> int:
    return default().num_threads()


def sgemm_ref_f64(A, B):
    return default().sgemm_ref_f64(A, B)


def sgemm_ref_f64_entries(A, B, rows, cols):
    return default().sgemm_ref_f64_entries(A, B, rows, cols)


def micro4x4_seq_fma_f32(A, B):
    return default().micro4x4_seq_fma_f32(A, B)


def decode16_f32(X, fmt):
    return default().decode16_f32(X, fmt)


def gemm_lowp_ref_f64(A, B, fmt):
    return default().gemm_lowp_ref_f64(A, B, fmt)


def sgemm_ex_ref_f64_entries(A, B, rows, cols, C_in=None, alpha=1.0, beta=0.0, bias=None, act=0):
    return default().sgemm_ex_ref_f64_entries(A, B, rows, cols, C_in, alpha, beta, bias, act)


def sgemm_ex_ref_f64(A, B, C_in=None, alpha=1.0, beta=0.0, bias=None, act=0):
    return default().sgemm_ex_ref_f64(A, B, C_in, alpha, beta, bias, act)


def parity(C_test, C_ref, rel_tol: float = REL_TOL):
    """Acceptance rule: err = max|C_test - C_ref|, ref = max|C_ref|;
    pass iff err <= rel_tol * ref, with no NaN/Inf in C_test; when ref == 0
    the result must be exactly zero.  Returns (ok, err, ref, tol)."""
    C_test = np.asarray(C_test, dtype=np.float64)
    C_ref = np.asarray(C_ref, dtype=np.float64)
    if C_test.shape != C_ref.shape:
        raise ValueError(f"shape mismatch {C_test.shape} vs {C_ref.shape}")
    if C_ref.size == 0:
        return True, 0.0, 0.0, 0.0
    if not np.all(np.isfinite(C_test)):
        return False, float("inf"), float(np.max(np.abs(C_ref))), 0.0
    err = float(np.max(np.abs(C_test - C_ref)))
    ref = float(np.max(np.abs(C_ref)))
    tol = rel_tol * ref
    return (err <= tol), err, ref, tol


def timed_rows(A: np.ndarray, B: np.ndarray, rows: int):
    """Time the full-product oracle on the first ``rows`` rows of A @ B.
    Returns (seconds, flops) with flops = 2 * rows * N * K."""
    sub = A[:rows]
    t0 = time.perf_counter()
    sgemm_ref_f64(sub, B)
    dt = time.perf_counter() - t0
    return dt, 2.0 * sub.shape[0] * B.shape[1] * A.shape[1]
