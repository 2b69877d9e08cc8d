"""Host builds under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only; the toolchain has no device-side race detector to rely on):

* the oracle (oracle/sgemm_ref.c), built by gcc with the sanitizers and
  driven by tests/sanitize/oracle_driver.c over small and degenerate shapes
  with heap buffers of exactly each matrix's extent, every 16-bit pattern
  and the micro-GEMM;
* the C ABI layer of the library (csrc/sgemm_api.hip: argument validation,
  extents, overlap checks), compiled for the host only with the sanitizers
  and linked with stand-ins for the kernel launchers
  (tests/sanitize/launch_stubs.cpp); tests/sanitize/api_driver.c checks
  every documented return code, extreme dimensions and pointers near the top
  of the address space included.  No call reaches a GPU.

Any out-of-bounds access, overflow or other undefined behaviour aborts the
driver (-fno-sanitize-recover), which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "register_lds_tiled_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-ffp-contract=off", "-fopenmp",
         os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "sgemm_ref.c"),
         "-o", str(exe), "-lm"])
    run([str(exe)], env={**os.environ, "OMP_NUM_THREADS": "2", "ASAN_OPTIONS": "detect_leaks=1"})


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain missing")
def test_abi_validation_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    host = ["--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-fPIC",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
    api, stubs, drv, exe = (tmp_path / n for n in ("api.o", "stubs.o", "drv.o", "api_driver"))
    run([HIPCC, *host, *inc, "-c", os.path.join(CSRC, "sgemm_api.hip"), "-o", str(api)])
    run([HIPCC, *host, *inc, "-x", "hip", "-c", os.path.join(SAN, "launch_stubs.cpp"), "-o", str(stubs)])
    run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-I", os.path.join(ROOT, "include"), "-c", os.path.join(SAN, "api_driver.c"), "-o", str(drv)])
    run([CLANG + "++", "-fsanitize=address,undefined", str(drv), str(api), str(stubs),
         "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)])
    run([str(exe)], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
