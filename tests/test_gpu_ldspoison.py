"""GPU checks of the LDS stage schedules with the debug build
libsgemm_mi355x_ldspoison.so: its kernels write NaN over every LDS location
between the barrier (or wave-level fence) that retires it and its refill, so
a read of a stage outside its lifetime turns into NaN in C.  Each case runs
one entry point through both builds of the C ABI on the same device inputs
and requires C -- written outputs and the NaN-filled padding alike -- to be
bit-identical, and the release result to be finite.  The cases reach every
kernel that reuses an LDS stage: the large wave-tile kernels (each tile
size, odd and even stage counts, stages shifted below k = 0 with lanes
switched off, 16- and 4-byte DMA forms), the direct-to-LDS and
register-staged matrix-core kernels, every vector-ALU tile configuration
and the page's geometry, the fused epilogue with its C prefetch, the 16-bit
kernels (shifted first stages included, with and without the in-loop
lane mask), the few-row and few-column streaming kernels and the 4x4
micro-GEMM.  Correctness against the oracle is the parity tests' business;
here a difference between the builds means a schedule that reads a stage
while it is being refilled ("Register/Shared Memory Tiling", operating
principle, double buffering: the barrier placement that keeps the stages
apart).
"""
import numpy as np
import pytest

from register_lds_tiled_amd import binding as b
from register_lds_tiled_amd import workloads as W
from tests.test_gpu_parity import ALIGN_CASES, CLASS_SHAPES, DEV, EDGE_SHAPES

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    return b.library(), b.ldspoison_library()


def dev(X: np.ndarray, ld: int, offset: int = 0, dtype=torch.float32, fill=float("nan")):
    """X (rows x cols) in a fresh device buffer, leading dimension ld,
    `offset` elements in, the rest filled; returns (buffer, address)."""
    rows, cols = X.shape
    buf = torch.full((offset + max(rows * ld, 1),), fill, dtype=dtype, device=DEV)
    if rows and cols:
        buf[offset:offset + rows * ld].view(rows, ld)[:, :cols].copy_(torch.from_numpy(np.ascontiguousarray(X)))
    return buf, buf.data_ptr() + buf.element_size() * offset


def same_in_both(libs, M, N, ldc, call, what, off_c=0, init=None):
    """call(lib, c_address, stream) in each build on its own C buffer (NaN,
    or the device tensor `init` where the call reads C); the two buffers must
    hold the same bits afterwards, and the outputs be finite."""
    stream = torch.cuda.current_stream()
    outs = []
    for lib in libs:
        if init is None:
            bufC = torch.full((off_c + max(M * ldc, 1),), float("nan"), device=DEV)
        else:
            bufC = init.clone()
        st = call(lib, bufC.data_ptr() + 4 * off_c, stream.cuda_stream)
        assert st == 0, f"{what}: status {st} {lib.sgemm_last_error()}"
        outs.append(bufC)
    torch.cuda.synchronize()
    rel, dbg = outs
    if M and N:
        C = rel[off_c:off_c + M * ldc].view(M, ldc)[:, :N]
        assert bool(torch.isfinite(C).all()), f"{what}: release output not finite"
    diff = rel.view(torch.int32) != dbg.view(torch.int32)
    n = int(diff.sum())
    if n:
        first = int(torch.nonzero(diff)[0]) - off_c
        raise AssertionError(f"{what}: {n} words differ between the release and the LDS-poison "
                             f"build (first at C[{first // ldc}][{first % ldc}]: "
                             f"{float(rel[first + off_c])} vs {float(dbg[first + off_c])})")


def f32_case(libs, M, N, K, path=b.PATH_AUTO, pad=(0, 0, 0), off=(0, 0, 0), seed=0, tile=None):
    A, B = W.random_inputs(M, N, K, seed=seed or (M + 3 * N + 5 * K))
    lda, ldb, ldc = max(K + pad[0], 1), max(N + pad[1], 1), max(N + pad[2], 1)
    bufA, pA = dev(A, lda, off[0])
    bufB, pB = dev(B, ldb, off[1])
    if tile is None:
        call = lambda lib, pC, s: lib.sgemm_f32_path(M, N, K, pA, lda, pB, ldb, pC, ldc, s, path)
    else:
        call = lambda lib, pC, s: lib.sgemm_f32_valu_tile(M, N, K, pA, lda, pB, ldb, pC, ldc, s, tile)
    same_in_both(libs, M, N, ldc, call, f"{M}x{N}x{K} path {path} tile {tile} pad {pad} off {off}",
                 off_c=off[2])
    del bufA, bufB


@pytest.mark.parametrize("shape", CLASS_SHAPES + [(2048, 2048, 2048), (4096, 4096, 1024), (1024, 1024, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_matrix_core_tile_classes(libs, shape):
    f32_case(libs, *shape)


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_large_wave_tile_edges(libs, shape):
    M, N, K, extra = shape
    f32_case(libs, M, N, K, pad=(extra, 0, 0))


@pytest.mark.parametrize("case", ALIGN_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-pad{c[3]}-off{c[4]}")
def test_large_wave_tile_alignments(libs, case):
    M, N, K, pad, off = case
    f32_case(libs, M, N, K, pad=pad, off=off)


@pytest.mark.parametrize("tile", range(15))
def test_vector_alu_tiles(libs, tile):
    assert b.sgemm_valu_tile_count() == 15
    for M, N, K in [(517, 389, 300), (1024, 1024, 256), (130, 70, 17)]:
        f32_case(libs, M, N, K, tile=tile)


@pytest.mark.parametrize("shape", [(300, 260, 100), (1000, 1000, 777), (2048, 2048, 512)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("path", [b.PATH_VALU, b.PATH_VALU_PAGE], ids=["valu", "valu_page"])
def test_vector_alu_paths(libs, path, shape):
    f32_case(libs, *shape, path=path)


@pytest.mark.parametrize("shape", [(2048, 2048, 512), (1000, 1500, 777), (1024, 1024, 1024), (3900, 3900, 272)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fused_epilogue(libs, shape):
    """C = relu(0.75 A.B + 0.5 C + bias): the large wave tiles prefetch C's
    previous values during the last stage."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M + N + K)
    C0, bias = W.epilogue_inputs(M, N, seed=K)
    bufA, pA = dev(A, K)
    bufB, pB = dev(B, N)
    bufBias, pBias = dev(bias.reshape(1, N), N)
    init = torch.from_numpy(np.ascontiguousarray(C0, dtype=np.float32)).to(DEV).reshape(-1)
    same_in_both(libs, M, N, N,
                 lambda lib, pC, s: lib.sgemm_f32_ex(M, N, K, pA, K, pB, N, pC, N, 0.75, 0.5, pBias,
                                                     b.ACT_RELU, s),
                 f"ex {shape}", init=init)
    del bufA, bufB, bufBias


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(2048, 2048, 2048), (1000, 1500, 777), (3000, 3072, 256), (4100, 4000, 72),
                                   (1024, 1001, 512), (2048, 2048, 104), (130, 70, 17), (256, 128, 4096),
                                   (1024, 1024, 1000), (3072, 3072, 392)],
                         ids=lambda s: "x".join(map(str, s)))
def test_sixteen_bit_inputs(libs, fmt, shape):
    M, N, K = shape
    A16, B16 = W.lowp_inputs(M, N, K, seed=M + 2 * N + K, fmt=fmt)
    bufA, pA = dev(A16.view(np.int16), K, dtype=torch.int16, fill=0)
    bufB, pB = dev(B16.view(np.int16), N, dtype=torch.int16, fill=0)
    entry = "gemm_bf16_f32" if fmt == "bf16" else "gemm_f16_f32"
    same_in_both(libs, M, N, N, lambda lib, pC, s: getattr(lib, entry)(M, N, K, pA, K, pB, N, pC, N, s),
                 f"{fmt} {shape}")
    del bufA, bufB


# few rows: the 16-row corner kernel, the split narrow-grid form, the
# scalar-row kernel; few columns: the LDS-shared and 16-byte-load kernels
@pytest.mark.parametrize("shape", [(16, 2048, 4099), (13, 4099, 1000), (8, 4099, 1000), (5, 2048, 4099),
                                   (4, 3000, 2500), (12, 16000, 77), (1, 8192, 8192),
                                   (1000, 8, 1000), (4099, 16, 2570), (300, 12, 1000), (4097, 8, 4096),
                                   (32769, 8, 1100), (1000, 4, 1000), (70001, 4, 1024), (4099, 3, 2500)],
                         ids=lambda s: "x".join(map(str, s)))
def test_streaming_kernels(libs, shape):
    f32_case(libs, *shape)


@pytest.mark.parametrize("K", [1024, 5000])
def test_micro_gemm(libs, K):
    A, B = W.random_inputs(4, 4, K, seed=K)
    bufA, pA = dev(A, K)
    bufB, pB = dev(B, 4)
    same_in_both(libs, 4, 4, 4, lambda lib, pC, s: lib.sgemm_micro4x4_f32(K, pA, pB, pC, s), f"micro K={K}")
    del bufA, bufB
