"""CPU tests of the C-ABI library: it loads, exports exactly what
include/sgemm.h declares, and rejects invalid arguments with the documented
codes before any HIP call (so these run without a GPU; no compute call is
made).  Device addresses passed here are fake and never dereferenced."""
import ctypes
import os
import re
import subprocess

import pytest

from register_lds_tiled_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")

F = 0x10000000  # fake, 16-byte aligned "device" addresses, never dereferenced


def header_functions():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"SGEMM_API\s+[\w\s\*]*?\b((?:s?gemm)_\w+)\s*\(", text)))


def header_constants():
    text = open(HEADER, encoding="utf-8").read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(SGEMM_\w+)\s+(-?\d+)", text)}


@pytest.fixture(scope="module")
def lib():
    return b.library()


def test_library_exports_every_declared_symbol(lib):
    fns = header_functions()
    assert fns == sorted(b.EXPORTS)
    for f in fns:
        assert hasattr(lib, f), f
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == fns, f"library exports {exported}, header declares {fns}"


def test_debug_build_exports_the_same_abi():
    """The LDS-poison debug build is the same C ABI: the same exported
    functions and the same ABI version."""
    fns = header_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", b.LDSPOISON_LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == fns, f"debug library exports {exported}, header declares {fns}"
    assert b.ldspoison_library().sgemm_abi_version() == b.sgemm_abi_version()


def test_constants_match_header():
    c = header_constants()
    for name in ("OK", "EINVAL_DIM", "EINVAL_LD", "EINVAL_PTR", "EALIAS", "EHIP", "EINVAL_PATH",
                 "EINVAL_ACT"):
        assert getattr(b, "SGEMM_" + name) == c["SGEMM_" + name]
    for name in ("NONE", "RELU"):
        assert getattr(b, "ACT_" + name) == c["SGEMM_ACT_" + name]
    for name in ("AUTO", "VALU", "MFMA", "VALU_PAGE"):
        assert getattr(b, "PATH_" + name) == c["SGEMM_PATH_" + name]


def test_abi_version_and_strings(lib):
    assert b.sgemm_abi_version() == 4
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        s = b.sgemm_status_string(code)
        assert s.startswith("SGEMM_")
    assert b.sgemm_status_string(12345) == "unknown sgemm status"
    assert b.sgemm_last_error() == ""


def call(M, N, K, A, lda, B, ldb, C, ldc, path=0):
    return b.sgemm_f32_path(M, N, K, A, lda, B, ldb, C, ldc, 0, path, check=False)


@pytest.mark.parametrize("path", [0, 1, 2, 3])
def test_validation_codes(path):
    A, B, C = F, F + (1 << 24), F + (1 << 26)
    assert call(-1, 4, 4, A, 4, B, 4, C, 4, path) == b.SGEMM_EINVAL_DIM
    assert call(4, -1, 4, A, 4, B, 4, C, 4, path) == b.SGEMM_EINVAL_DIM
    assert call(4, 4, -1, A, 4, B, 4, C, 4, path) == b.SGEMM_EINVAL_DIM
    assert call(4, 4, 8, A, 7, B, 4, C, 4, path) == b.SGEMM_EINVAL_LD
    assert call(4, 8, 4, A, 4, B, 7, C, 8, path) == b.SGEMM_EINVAL_LD
    assert call(4, 8, 4, A, 4, B, 8, C, 7, path) == b.SGEMM_EINVAL_LD
    assert call(4, 4, 0, A, 0, B, 4, C, 4, path) == b.SGEMM_EINVAL_LD  # ld >= 1
    assert call(4, 4, 4, 0, 4, B, 4, C, 4, path) == b.SGEMM_EINVAL_PTR
    assert call(4, 4, 4, A, 4, 0, 4, C, 4, path) == b.SGEMM_EINVAL_PTR
    assert call(4, 4, 4, A, 4, B, 4, 0, 4, path) == b.SGEMM_EINVAL_PTR
    # C overlapping A (last byte) or B (first byte); A overlapping B is fine
    assert call(4, 4, 4, A, 4, B, 4, A + 60, 4, path) == b.SGEMM_EALIAS
    assert call(4, 4, 4, A, 4, B, 4, B - 60, 4, path) == b.SGEMM_EALIAS
    # empty C: success without touching anything (NULL pointers allowed)
    assert call(0, 4, 4, 0, 4, 0, 4, 0, 4, path) == b.SGEMM_OK
    assert call(4, 0, 4, 0, 4, 0, 1, 0, 1, path) == b.SGEMM_OK


def test_invalid_path():
    assert call(4, 4, 4, F, 4, F + 4096, 4, F + 8192, 4, path=4) == b.SGEMM_EINVAL_PATH
    assert call(4, 4, 4, F, 4, F + 4096, 4, F + 8192, 4, path=-1) == b.SGEMM_EINVAL_PATH


def test_valu_tile_table_and_validation():
    """The VALU tile table: every configuration named (block, waves, lane
    tile), NULL past the end; the tile index and then the plain product's
    argument checks are applied before any HIP call."""
    n = b.sgemm_valu_tile_count()
    assert n >= 6
    names = [b.sgemm_valu_tile_name(t) for t in range(n)]
    assert all(nm and "waves" in nm and "lanes" in nm for nm in names)
    assert len(set(names)) == n
    assert b.sgemm_valu_tile_name(n) is None and b.sgemm_valu_tile_name(-1) is None
    # the register tiles compared on the micro-kernel page, and the tiled page's 16x4
    for lane_tile in ("4x4", "8x4", "16x4", "8x8", "16x8"):
        assert any(f" of {lane_tile} stages" in nm for nm in names), lane_tile
    v = lambda *a, tile=0: b.sgemm_f32_valu_tile(*a, 0, tile, check=False)  # noqa: E731
    A, B, C = F, F + (1 << 24), F + (1 << 26)
    assert v(4, 4, 4, A, 4, B, 4, C, 4, tile=n) == b.SGEMM_EINVAL_PATH
    assert v(4, 4, 4, A, 4, B, 4, C, 4, tile=-1) == b.SGEMM_EINVAL_PATH
    for t in range(n):
        assert v(-1, 4, 4, A, 4, B, 4, C, 4, tile=t) == b.SGEMM_EINVAL_DIM
        assert v(4, 8, 4, A, 4, B, 8, C, 7, tile=t) == b.SGEMM_EINVAL_LD
        assert v(4, 4, 4, 0, 4, B, 4, C, 4, tile=t) == b.SGEMM_EINVAL_PTR
        assert v(4, 4, 4, A, 4, B, 4, A + 60, 4, tile=t) == b.SGEMM_EALIAS
        assert v(0, 4, 4, 0, 4, 0, 4, 0, 4, tile=t) == b.SGEMM_OK


def ex(M, N, K, A, lda, B, ldb, C, ldc, alpha=1.0, beta=0.0, bias=0, act=0):
    return b.sgemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, bias, act, 0, check=False)


def test_ex_validation_codes():
    A, B, C = F, F + (1 << 24), F + (1 << 26)
    # an unknown activation is refused before anything else is looked at
    assert ex(4, 4, 4, A, 4, B, 4, C, 4, act=2) == b.SGEMM_EINVAL_ACT
    assert ex(4, 4, 4, A, 4, B, 4, C, 4, act=-1) == b.SGEMM_EINVAL_ACT
    assert ex(-1, 4, 4, A, 4, B, 4, C, 4, act=7) == b.SGEMM_EINVAL_ACT
    # the plain product's checks apply unchanged
    assert ex(-1, 4, 4, A, 4, B, 4, C, 4) == b.SGEMM_EINVAL_DIM
    assert ex(4, 8, 4, A, 4, B, 8, C, 7) == b.SGEMM_EINVAL_LD
    assert ex(4, 4, 4, A, 4, B, 4, 0, 4, beta=1.0) == b.SGEMM_EINVAL_PTR
    assert ex(4, 4, 4, A, 4, B, 4, A + 60, 4, bias=F + (1 << 28)) == b.SGEMM_EALIAS
    # bias (N floats) overlapping C: its last float on C's first, or inside C
    assert ex(4, 4, 4, A, 4, B, 4, C, 4, bias=C - 12) == b.SGEMM_EALIAS
    assert ex(4, 4, 4, A, 4, B, 4, C, 4, bias=C + 60) == b.SGEMM_EALIAS
    assert ex(4, 4, 4, A, 4, B, 4, C, 8, bias=C + 16) == b.SGEMM_EALIAS   # in ldc padding
    # empty C: success without a launch, whatever the epilogue
    assert ex(0, 4, 4, 0, 4, 0, 4, 0, 4, 2.0, 1.0, C, 1) == b.SGEMM_OK
    assert ex(4, 0, 4, 0, 4, 0, 1, 0, 1, 2.0, 1.0, C, 1) == b.SGEMM_OK


@pytest.mark.parametrize("fn", ["gemm_bf16_f32", "gemm_f16_f32"])
def test_lowp_validation_codes(fn):
    f = lambda *a: getattr(b, fn)(*a, 0, check=False)  # noqa: E731
    A, B, C = F, F + (1 << 24), F + (1 << 26)
    assert f(-1, 4, 4, A, 4, B, 4, C, 4) == b.SGEMM_EINVAL_DIM
    assert f(4, 4, 8, A, 7, B, 4, C, 4) == b.SGEMM_EINVAL_LD
    assert f(4, 8, 4, A, 4, B, 8, C, 7) == b.SGEMM_EINVAL_LD
    assert f(4, 4, 4, 0, 4, B, 4, C, 4) == b.SGEMM_EINVAL_PTR
    assert f(4, 4, 4, A, 4, B, 4, 0, 4) == b.SGEMM_EINVAL_PTR
    # overlap uses 2-byte extents for A and B: A spans 4*4*2 = 32 bytes
    assert f(4, 4, 4, A, 4, B, 4, A + 28, 4) == b.SGEMM_EALIAS
    assert f(4, 4, 4, A, 4, B, 4, B - 60, 4) == b.SGEMM_EALIAS
    assert f(0, 4, 4, 0, 4, 0, 4, 0, 4) == b.SGEMM_OK


def test_micro_validation():
    m = lambda K, A, B, C: b.sgemm_micro4x4_f32(K, A, B, C, 0, check=False)  # noqa: E731
    assert m(-1, F, F + 65536, F + 131072) == b.SGEMM_EINVAL_DIM
    assert m(8, 0, F + 65536, F + 131072) == b.SGEMM_EINVAL_PTR
    assert m(8, F, 0, F + 131072) == b.SGEMM_EINVAL_PTR
    assert m(8, F, F + 65536, 0) == b.SGEMM_EINVAL_PTR
    assert m(8, F, F + 65536, F + 16) == b.SGEMM_EALIAS     # C inside A (4x8 floats)
    assert m(8, F, F + 65536, F + 65536 + 64) == b.SGEMM_EALIAS


def test_errors_raise_with_message():
    with pytest.raises(b.SgemmError) as e:
        b.sgemm_f32_path(-1, 1, 1, F, 1, F, 1, F, 1, 0, 0)
    assert e.value.status == b.SGEMM_EINVAL_DIM
    assert "EINVAL_DIM" in str(e.value)


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "sgemm.h"\nint main(void){return sgemm_abi_version()==4?0:1;}\n')
    exe = tmp_path / "use"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                    str(src), b.LIB_PATH, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], env={**os.environ, "LD_LIBRARY_PATH": os.path.dirname(b.LIB_PATH)})
    assert r.returncode == 0
