"""MI355X (gfx950) single-precision row-major GEMM by register/LDS tiling.

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/sgemm.h``); ``binding`` marshals arguments to
it with ctypes and raises if the library is missing.  ``workloads`` draws the
seeded synthetic inputs.  Importing this package loads nothing; the library is
opened on the first call.
"""
from .binding import (  # noqa: F401
    PATH_AUTO, PATH_MFMA, PATH_VALU, PATH_VALU_PAGE, PATHS, SgemmError, matmul,
    sgemm_abi_version, sgemm_f32, sgemm_f32_path, sgemm_last_error,
    sgemm_micro4x4_f32, sgemm_status_string,
)
