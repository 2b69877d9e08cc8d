"""MI355X (gfx950) single-precision row-major GEMM by register/LDS tiling.

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/sgemm.h``); ``binding`` marshals arguments to
it with ctypes.  ``workloads`` draws the seeded synthetic inputs.
"""
