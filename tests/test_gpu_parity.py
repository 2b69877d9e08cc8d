"""GPU parity tests: every path of the HIP library, called through the C ABI,
against the CPU oracle on the same seeded inputs.

Acceptance rule (oracle.parity): max|C - C_ref| <= 1e-4 * max|C_ref| over the
compared outputs, no NaN/Inf where the reference is finite.  Integer-valued
inputs must match bit for bit (every partial sum is exact in fp32).  C is
pre-filled with NaN before every call so an unwritten output fails.
Workloads the oracle finishes in seconds (up to 2048^3) are compared in full.
At 8192^3 every output is checked to have been written (C starts as NaN), and
the oracle's values are compared on samples that touch every tile of C: one
whole row in each 128-row band and one whole column in each 128-column band
(at an offset inside the band that changes from band to band) and one entry
in each 64 x 64 tile.
"""
import math

import numpy as np
import pytest

import oracle
from register_lds_tiled_amd import binding as b
from register_lds_tiled_amd import workloads as W
from tests import pins

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ALL_PATHS = ["auto", "mfma", "valu", "valu_page"]
DEV = "cuda:0"


# ------------------------------------------------------------------ helpers --
def to_device(X: np.ndarray, ld: int, offset: int = 0, fill=float("nan")):
    """Place row-major X (rows x cols) in a fresh device buffer with leading
    dimension ld, starting `offset` floats into the buffer.  Returns
    (buffer, address of X[0,0])."""
    rows, cols = X.shape
    n = offset + max(rows * ld, 1)
    buf = torch.full((n,), fill, dtype=torch.float32, device=DEV)
    if rows and cols:
        view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
        view.copy_(torch.from_numpy(np.ascontiguousarray(X)))
    return buf, buf.data_ptr() + 4 * offset


def gemm(A: np.ndarray, B: np.ndarray, path="auto", *, pad=(0, 0, 0), off=(0, 0, 0),
         stream=None):
    """Run C = A.B on the GPU through sgemm_f32_path (or sgemm_f32 for
    path=None) with padded leading dimensions / offset base addresses and a
    NaN-filled C; return C as a numpy array."""
    M, K = A.shape
    N = B.shape[1]
    lda, ldb, ldc = max(K + pad[0], 1), max(N + pad[1], 1), max(N + pad[2], 1)
    bufA, pA = to_device(A, lda, off[0])
    bufB, pB = to_device(B, ldb, off[1])
    bufC, pC = to_device(np.full((M, N), np.nan, np.float32), ldc, off[2])
    s = stream if stream is not None else torch.cuda.current_stream()
    if path is None:
        b.sgemm_f32(M, N, K, pA, lda, pB, ldb, pC, ldc, s)
    else:
        b.sgemm_f32_path(M, N, K, pA, lda, pB, ldb, pC, ldc, s, path)
    torch.cuda.synchronize()
    if M == 0 or N == 0:
        return np.zeros((M, N), np.float32)
    C = bufC[off[2]:off[2] + M * ldc].view(M, ldc)[:, :N].cpu().numpy()
    del bufA, bufB, bufC
    return C


def assert_parity(C, R, what):
    ok, err, ref, tol = oracle.parity(C, R)
    assert ok, f"{what}: max|C-C_ref| = {err:.3e} > tol {tol:.3e} (max|C_ref| = {ref:.3e})"


# Largest M*N*K compared in full against the oracle (2048^3 included).
FULL_LIMIT = 1.3e10


tile_samples = W.tile_samples


def sampled_ref(A, B, samples):
    """The oracle on tile_samples' rows, columns and entries."""
    rows, cols, er, ec = samples
    return ("sampled", dict(
        rows=rows, R_rows=oracle.sgemm_ref_f64(A[rows], B),
        cols=cols, R_cols=oracle.sgemm_ref_f64(A, np.ascontiguousarray(B[:, cols])),
        er=er, ec=ec, R_e=oracle.sgemm_ref_f64_entries(A, B, er, ec)))


def sampled_values(C, R):
    """(GPU, oracle) values at the sampled outputs of a sampled reference."""
    got = np.concatenate([C[R["rows"]].ravel(), C[:, R["cols"]].ravel(), C[R["er"], R["ec"]]])
    exp = np.concatenate([R["R_rows"].ravel(), R["R_cols"].ravel(), R["R_e"]])
    return got, exp


_cache = {}


def workload_case(name):
    """Inputs and (full or tile-sampled) oracle reference for a named workload."""
    if name in _cache:
        return _cache[name]
    w = W.WORKLOADS[name]
    A, B = W.inputs_for(w)
    if w.M * w.N * w.K <= FULL_LIMIT:
        ref = ("full", oracle.sgemm_ref_f64(A, B))
    else:
        ref = sampled_ref(A, B, tile_samples(w.M, w.N, seed=4242))
    _cache[name] = (w, A, B, ref)
    return _cache[name]


def check_against(C, ref, what):
    """Full comparison, or (sampled reference) every output written and the
    sampled outputs within tolerance.  C must have been NaN-filled before
    the call, and the reference must be finite everywhere."""
    kind, R = ref
    if kind == "full":
        assert_parity(C, R, what)
        return
    unwritten = int(np.isnan(C).sum())
    assert unwritten == 0, f"{what}: {unwritten} outputs still NaN (never written)"
    assert np.isfinite(C).all(), f"{what}: non-finite output"
    got, exp = sampled_values(C, R)
    assert_parity(got, exp, what + " (a row and a column per 128 band, an entry per 64x64 tile)")


# --------------------------------------------------------------- micro-GEMM --
def micro_gpu(A, B):
    K = A.shape[1]
    dA = torch.from_numpy(np.ascontiguousarray(A)).to(DEV)
    dB = torch.from_numpy(np.ascontiguousarray(B)).to(DEV)
    dC = torch.full((4, 4), float("nan"), dtype=torch.float32, device=DEV)
    b.sgemm_micro4x4_f32(K, dA if K else 0, dB if K else 0, dC)
    torch.cuda.synchronize()
    return dC.cpu().numpy()


def test_micro_worked_example_bit_exact():
    K, printed = pins.read_golden()
    A, B = W.worked_example(K)
    C = micro_gpu(A, B)
    R = oracle.micro4x4_seq_fma_f32(A, B)
    assert np.array_equal(C.view(np.uint32), R.view(np.uint32)), (C, R)
    assert ["%f" % float(v) for v in C[0]] == printed
    assert_parity(C, oracle.sgemm_ref_f64(A, B), "micro vs f64 oracle")


@pytest.mark.parametrize("K", [0, 1, 2, 7, 8, 9, 1000, 4099])
def test_micro_random_bit_exact(K):
    rng = np.random.Generator(np.random.PCG64(31 + K))
    A = rng.uniform(-1, 1, (4, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, 4)).astype(np.float32)
    C = micro_gpu(A, B)
    R = oracle.micro4x4_seq_fma_f32(A, B)
    assert np.array_equal(C.view(np.uint32), R.view(np.uint32))


# ------------------------------------------------------------ tiled paths --
@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("shape", [(1, 1, 1), (7, 5, 3), (64, 64, 16), (128, 128, 16),
                                   (127, 129, 17), (255, 257, 31), (300, 260, 100),
                                   (129, 257, 33), (520, 390, 300), (33, 1000, 7),
                                   (1000, 40, 2000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_small_shapes(path, shape):
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M * 7919 + N * 31 + K)
    assert_parity(gemm(A, B, path), oracle.sgemm_ref_f64(A, B), f"{path} {shape}")


@pytest.mark.parametrize("path", ALL_PATHS)
def test_tiny_sweep(path):
    rng = np.random.Generator(np.random.PCG64(77))
    for _ in range(60):
        M, N, K = (int(x) for x in rng.integers(1, 10, 3))
        A, B = W.random_inputs(M, N, K, seed=int(rng.integers(1 << 30)))
        assert_parity(gemm(A, B, path), oracle.sgemm_ref_f64(A, B), f"{path} {M}x{N}x{K}")


@pytest.mark.parametrize("path", ALL_PATHS)
def test_tile_edges(path):
    for M in (63, 65, 128, 129, 257):
        for N in (63, 65, 128, 129, 257):
            for K in (15, 16, 17, 33):
                A, B = W.integer_inputs(M, N, K, seed=M * 1000 + N * 10 + K)
                C = gemm(A, B, path)
                R = oracle.sgemm_ref_f64(A, B)
                assert np.array_equal(C.astype(np.float64), R), f"{path} {M}x{N}x{K}"


# Shapes that reach every kernel instance of the matrix-core path:
#   256x256 tiles, last round full, whole tiles, K a multiple of 32 (the
#   shortest pipeline, two stages, and six)
#                                  -> large wave-tile kernel, 256x256
#   3/4 to 1 tile of 128x128 per CU, whole, K a multiple of 64
#                                  -> large wave-tile kernel, 128x128
#   whole 64x64 tiles, K a multiple of 64 (small grids; 2304^2, whose
#   128x128 grid fills its rounds poorly; K = 4096: 64-k stages)
#                                  -> large wave-tile kernel, 64x64
# and, with ragged K (a partial last slab):
#   256x256 tiles, last round full (ragged M and N, or whole)
#                                  -> register kernel, 256x256 tiles
#   many 128x128 tiles that fill their rounds (ragged or whole; 6000x5900:
#   576 tiles of 256x256 leave a last round a quarter full)
#                                  -> register kernel, 128x128 tiles
#   many 128x128 tiles with a half-empty last round (2000x3000, 2048x3072:
#   384 of them; 2560x1664 with lda = 77: 260) -> register kernel, 64x64
#   3/4 to 1 tile of 128x128 per CU, whole tiles -> direct-to-LDS, 128x128
#   the same with unaligned rows (lda = 77)   -> register kernel, 128x128
#   1 to 1.5 tiles of 128x128 per CU, whole tiles -> direct-to-LDS, 128x64
#   small grid, ragged M and N, or rows not 16-byte aligned (lda = 45)
#                                         -> register kernel, 64x64 tiles
#   the same where 64x96 tiles fill the CUs better (700x2000: 231 tiles
#   against 352)                          -> register kernel, 64x96 tiles
#   small grid, whole 64x64 tiles, aligned -> direct-to-LDS kernel, 64x64
#   small grid, <= 256 whole tiles, K >= 512, lda >= 2^22 (too long for
#   the large wave-tile kernel's 32-bit offsets)
#                                         -> the same with K split four ways
#                                            inside the workgroup (see
#                                            test_ksplit_class_with_long_rows)
CLASS_SHAPES = [(4096, 4096, 32), (4096, 4096, 96), (2048, 2048, 64), (2048, 2048, 192),
                (1024, 1024, 128), (1536, 1536, 64), (2304, 2304, 64), (256, 512, 4096),
                (4090, 4090, 33), (4096, 4096, 48), (6000, 5900, 33), (2000, 3000, 77),
                (2048, 3072, 40), (2560, 1664, 77), (2048, 2048, 100), (2048, 2048, 77),
                (2304, 2304, 104), (500, 700, 45), (512, 768, 45), (700, 2000, 100),
                (512, 768, 48), (1536, 1536, 100), (1024, 64, 1000), (768, 512, 1200),
                (1024, 1024, 520), (1024, 1024, 1536), (512, 1000, 2000),
                (1024, 1024, 300), (512, 512, 300), (4096, 4096, 150)]


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("shape", CLASS_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_tile_classes_ragged(path, shape):
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M + 3 * N + 7 * K)
    assert_parity(gemm(A, B, path), oracle.sgemm_ref_f64(A, B), f"{path} {shape}")
    Ai, Bi = W.integer_inputs(M, N, K, seed=M + N + K)
    assert np.array_equal(gemm(Ai, Bi, path).astype(np.float64), oracle.sgemm_ref_f64(Ai, Bi))


@pytest.mark.parametrize("shape", [(128, 256, 520), (64, 1024, 1000), (256, 64, 1200)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ksplit_class_with_long_rows(shape):
    """Whole 64x64 tiles, at most one per CU, K >= 512, A rows 2^22 floats
    apart (beyond the large wave-tile kernel's 32-bit DMA offsets) and C
    one float off 16 bytes: the direct-to-LDS kernel with K split four ways
    inside the workgroup.  A's buffer is 0.25-1 GB of NaN padding."""
    M, N, K = shape
    pad = ((1 << 22) - K, 0, 0)
    A, B = W.random_inputs(M, N, K, seed=M + K)
    assert_parity(gemm(A, B, None, pad=pad, off=(0, 0, 1)), oracle.sgemm_ref_f64(A, B), f"{shape}")
    Ai, Bi = W.integer_inputs(M, N, K, seed=N + K)
    C = gemm(Ai, Bi, None, pad=pad, off=(0, 0, 1)).astype(np.float64)
    assert np.array_equal(C, oracle.sgemm_ref_f64(Ai, Bi))


# The large wave-tile kernels at any alignment: B rows not 16-byte aligned
# or N % 4 != 0 (the 4-byte B DMA form), C rows not 16-byte aligned (C
# stored one float at a time), with the 4-byte A form where lda or K is odd.
# (M, N, K, pad, off)
ALIGN_CASES = [(1000, 1001, 777, (0, 0, 0), (0, 0, 0)),
               (2048, 2001, 2048, (0, 0, 0), (0, 0, 0)),
               (2047, 2047, 2047, (0, 0, 0), (0, 0, 0)),
               (1024, 1024, 520, (0, 0, 0), (0, 0, 1)),
               (1024, 1024, 1536, (0, 0, 0), (0, 3, 0)),
               (3000, 3004, 1024, (0, 1, 2), (0, 0, 0)),
               (4100, 4101, 512, (0, 0, 0), (1, 1, 1))]


@pytest.mark.parametrize("case", ALIGN_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-pad{c[3]}-off{c[4]}")
def test_large_wave_tile_any_alignment(case):
    M, N, K, pad, off = case
    A, B = W.random_inputs(M, N, K, seed=M + 2 * N + K)
    assert_parity(gemm(A, B, None, pad=pad, off=off), oracle.sgemm_ref_f64(A, B), f"{case}")
    Ai, Bi = W.integer_inputs(M, N, K, seed=M + N + 3 * K)
    C = gemm(Ai, Bi, None, pad=pad, off=off).astype(np.float64)
    assert np.array_equal(C, oracle.sgemm_ref_f64(Ai, Bi)), f"{case} integer"


# Shapes that reach the large wave-tile kernels with ragged M and N, a K
# that is not a multiple of two stages (the first two stages reach below
# k = 0 and are zero-filled), and A rows that are not 16-byte aligned (the
# 4-byte DMA form).  (M, N, K, extra lda)
EDGE_SHAPES = [(3900, 3900, 272, 0),    # 256x256, ragged, shift 16
               (4096, 4096, 301, 0),    # 256x256, K % 4 != 0: 4-byte A, shift 19
               (2000, 2000, 600, 0),    # 128x128, ragged, shift 40
               (1000, 1500, 777, 0),    # 64x96, lda 777, shift 23: 25 stages (the ragged workload)
               (1000, 1500, 776, 3),    # 64x96, lda 779: 4-byte A, shift 24: 25 stages
               (1000, 1500, 330, 0),    # 64x96, shift 22: 11 stages
               (1000, 1000, 330, 0),    # 64x64, shift 22: 11 stages
               (1000, 1000, 331, 0),    # 64x64, K % 4 != 0: 4-byte A, shift 21: 11 stages
               (512, 768, 200, 0),      # 64x64, 96 tiles, shift 24: 7 stages
               (1000, 1000, 352, 0),    # 64x64, no shift: 11 stages
               (3000, 500, 4100, 0)]    # 64x64 with 64-k stages, shift 124


def edge_samples(M, N, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = np.unique(np.array([0, 1, M // 2, M - 2, M - 1]))
    cols = np.unique(np.array([0, 3, N // 2, N - 5, N - 4, N - 1]))
    er, ec = rng.integers(0, M, 2048), rng.integers(0, N, 2048)
    return rows, cols, er, ec


def sampled(C, A, B, rows, cols, er, ec):
    got = np.concatenate([C[rows].ravel(), C[:, cols].ravel(), C[er, ec]])
    exp = np.concatenate([oracle.sgemm_ref_f64(A[rows], B).ravel(),
                          oracle.sgemm_ref_f64(A, np.ascontiguousarray(B[:, cols])).ravel(),
                          oracle.sgemm_ref_f64_entries(A, B, er, ec)])
    return got, exp


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_large_wave_tile_edges(shape):
    M, N, K, pad = shape
    rows, cols, er, ec = edge_samples(M, N, M + K)
    A, B = W.random_inputs(M, N, K, seed=M + 2 * N + K)
    C = gemm(A, B, None, pad=(pad, 0, 0))
    got, exp = sampled(C, A, B, rows, cols, er, ec)
    assert_parity(got, exp, f"{shape} random (sampled rows, columns and entries)")
    Ai, Bi = W.integer_inputs(M, N, K, seed=M + N + 3 * K)
    Ci = gemm(Ai, Bi, None, pad=(pad, 0, 0))
    got, exp = sampled(Ci, Ai, Bi, rows, cols, er, ec)
    assert np.array_equal(got.astype(np.float64), exp), f"{shape} integer"


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("name", ["sq1024", "ragged", "sq2048", "sq8192"])
def test_workloads(path, name):
    w, A, B, ref = workload_case(name)
    C = gemm(A, B, path)
    check_against(C, ref, f"{path} {w.describe()}")


_int_cache = {}


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("name", ["sq1024", "ragged", "sq2048", "sq8192"])
def test_integer_inputs_bit_exact(path, name):
    """Integer inputs on {-3..3} at the workload sizes: every partial sum is
    an integer below 9K <= 73,728 < 2^24, exact in fp32 in any order, so C
    must equal the oracle bit for bit -- in full up to 2048^3, at 8192^3 on
    every output's being written and on the tile samples."""
    w = W.WORKLOADS[name]
    if name not in _int_cache:
        A, B = W.integer_inputs(w.M, w.N, w.K, seed=9000 + w.M + w.K)
        if w.M * w.N * w.K <= FULL_LIMIT:
            ref = ("full", oracle.sgemm_ref_f64(A, B))
        else:
            ref = sampled_ref(A, B, tile_samples(w.M, w.N, seed=5))
        _int_cache[name] = (A, B, ref)
    A, B, (kind, R) = _int_cache[name]
    C = gemm(A, B, path)
    if kind == "full":
        assert np.array_equal(C.astype(np.float64), R)
        return
    assert not np.isnan(C).any(), f"{path} {name}: outputs never written"
    got, exp = sampled_values(C, R)
    assert np.array_equal(got.astype(np.float64), exp), f"{path} {name} integer samples"


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("pad,off", [((3, 0, 0), (0, 0, 0)), ((0, 5, 0), (0, 1, 0)),
                                     ((1, 1, 1), (1, 3, 2)), ((4, 4, 4), (4, 4, 4)),
                                     ((0, 0, 7), (0, 0, 1))],
                         ids=["lda+3", "ldb+5,B+1", "all+1,offsets", "aligned-pads", "ldc+7,C+1"])
def test_leading_dims_and_alignment(path, pad, off):
    for (M, N, K) in ((200, 300, 150), (17, 23, 9)):
        A, B = W.random_inputs(M, N, K, seed=M + N + K + sum(pad))
        C = gemm(A, B, path, pad=pad, off=off)
        assert_parity(C, oracle.sgemm_ref_f64(A, B), f"{path} {M}x{N}x{K} pad={pad} off={off}")


@pytest.mark.parametrize("path", ALL_PATHS)
def test_k_zero_gives_zeros(path):
    C = gemm(np.zeros((70, 0), np.float32), np.zeros((0, 130), np.float32), path)
    assert np.array_equal(C, np.zeros((70, 130), np.float32))


@pytest.mark.parametrize("path", ALL_PATHS)
def test_empty_c_is_untouched(path):
    bufC = torch.full((64,), float("nan"), dtype=torch.float32, device=DEV)
    A = torch.ones(64, dtype=torch.float32, device=DEV)
    b.sgemm_f32_path(0, 8, 8, A, 8, A, 8, bufC, 8, None, path)
    b.sgemm_f32_path(8, 0, 8, A, 8, A, 1, bufC, 1, None, path)
    torch.cuda.synchronize()
    assert torch.isnan(bufC).all()


@pytest.mark.parametrize("path", ALL_PATHS)
def test_nan_inf_propagate(path):
    M, N, K = 150, 140, 70
    A, B = W.random_inputs(M, N, K, seed=11)
    B = np.abs(B) + np.float32(0.5)
    A[3, 5] = np.nan
    A[100, 7] = np.inf
    C = gemm(A, B, path)
    R = oracle.sgemm_ref_f64(A, B)
    assert np.array_equal(np.isnan(C), np.isnan(R))
    assert np.array_equal(np.isposinf(C), np.isposinf(R))
    fin = np.isfinite(R)
    assert fin.sum() == (M - 2) * N
    assert_parity(C[fin], R[fin], f"{path} finite part")


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("shape", [(130, 70, 17), (1000, 1500, 777), (4090, 4090, 33),
                                   (2000, 3000, 77), (500, 700, 45)],
                         ids=lambda s: "x".join(map(str, s)))
def test_nan_in_last_row_and_column_stays_there(path, shape):
    """Lanes of an edge tile whose A row lies past M, or whose B columns lie
    past N, may re-read A's last row and B's first columns of the tile; the
    NaN and Inf planted in A's last row and B's last column must reach C's
    last row and column only, and the rest must match the oracle."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M + N)
    B = np.abs(B) + np.float32(0.5)
    A[M - 1, K // 2] = np.nan
    A[M - 1, 0] = np.inf
    B[K - 1, N - 1] = np.nan
    C = gemm(A, B, path)
    R = oracle.sgemm_ref_f64(A, B)
    assert np.isnan(C[M - 1]).all() and np.isnan(C[:, N - 1]).all()
    assert np.isfinite(C[:M - 1, :N - 1]).all()
    assert_parity(C[:M - 1, :N - 1], R[:M - 1, :N - 1], f"{path} {shape} finite part")


@pytest.mark.parametrize("path", ALL_PATHS)
def test_deterministic_repeats(path):
    w, A, B, ref = workload_case("ragged")
    dA = torch.from_numpy(A).to(DEV)
    dB = torch.from_numpy(B).to(DEV)
    dC = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    first = None
    for _ in range(10):
        dC.fill_(float("nan"))
        b.sgemm_f32_path(w.M, w.N, w.K, dA, w.K, dB, w.N, dC, w.N, None, path)
        torch.cuda.synchronize()
        cur = dC.cpu().numpy()
        if first is None:
            first = cur
            check_against(first, ref, f"{path} ragged")
        assert np.array_equal(cur.view(np.uint32), first.view(np.uint32))


def test_default_entry_point_and_side_stream():
    A, B = W.random_inputs(333, 444, 555, seed=3)
    R = oracle.sgemm_ref_f64(A, B)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C = gemm(A, B, None, stream=s)
    assert_parity(C, R, "sgemm_f32 on a side stream")


def test_alias_rejected_on_device():
    buf = torch.zeros(4096, dtype=torch.float32, device=DEV)
    st = b.sgemm_f32(32, 32, 32, buf, 32, buf[2048:], 32, buf[1000:], 32, None, check=False)
    assert st == b.SGEMM_EALIAS
    assert math.isclose(float(buf.abs().sum()), 0.0)


@pytest.mark.parametrize("lda", [(1 << 22) - 4, 1 << 22])
def test_leading_dimension_at_the_offset_limit(lda):
    """The large wave-tile kernels address a DMA lane's element as a 32-bit
    byte offset from its tile's first row.  With lda = 2^22 - 4 floats the
    128 rows of a tile reach 2.1 GB past it (beyond 2^31: the offsets must
    be unsigned); at lda = 2^22 the library takes a kernel with 64-bit
    addresses instead.  A is 2 GB of mostly NaN padding on the device."""
    M, N, K = 128, 32768, 64
    A, B = W.random_inputs(M, N, K, seed=4242)
    C = gemm(A, B, pad=(lda - K, 0, 0))
    assert_parity(C, oracle.sgemm_ref_f64(A, B), f"lda={lda}")


@pytest.mark.parametrize("path", ["auto", "valu", "bf16"])
def test_output_past_2_31_elements(path):
    """C with more than 2^31 elements (65,600 x 32,768 fp32, 8.6 GB; 2,099
    tiles of rows past the 32-bit element offset): rows on both sides of
    2^16 (row x ldc = 2^31) and the last row, whole, each against the
    oracle on that row alone; fp32 (default and VALU paths) and bfloat16
    inputs.  C is filled with NaN first, so an unwritten or misplaced row
    fails."""
    M, N, K = 65600, 32768, 16
    if path == "bf16":
        A, B = W.lowp_inputs(M, N, K, seed=2031, fmt="bf16")
        dA, dB = (torch.from_numpy(X.view(np.int16)).to(DEV) for X in (A, B))
    else:
        A, B = W.random_inputs(M, N, K, seed=2031)
        dA, dB = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    s = torch.cuda.current_stream()
    if path == "bf16":
        b.gemm_bf16_f32(M, N, K, dA, K, dB, N, C, N, s)
    else:
        b.sgemm_f32_path(M, N, K, dA, K, dB, N, C, N, s, path)
    torch.cuda.synchronize()
    rows = [0, 1, 65535, 65536, 65537, 65599] + [int(r) for r in np.random.default_rng(7).integers(0, M, 4)]
    for r in rows:
        got = C[r].cpu().numpy()[None, :]
        ref = (oracle.gemm_lowp_ref_f64(A[r:r + 1], B, "bf16") if path == "bf16"
               else oracle.sgemm_ref_f64(A[r:r + 1], B))
        assert_parity(got, ref, f"{path} row {r}")
    del C, dA, dB
    torch.cuda.empty_cache()


FEW_ROWS = [(1, 1, 1), (1, 8192, 8192), (2, 63, 17), (3, 64, 16), (5, 65, 15), (8, 1000, 100),
            (13, 4099, 1000), (16, 2048, 4099), (16, 129, 0), (4, 70000, 33), (8, 65536, 8192),
            # narrow grids: 32- or 16-column workgroups, K split between lane groups
            (8, 4099, 1000), (5, 2048, 4099), (4, 3000, 2500), (6, 6000, 1100), (8, 8192, 8192),
            (12, 16000, 77),
            # 9 to 16 rows on the matrix cores (aligned; the padded run takes
            # the vector-ALU kernels): 64-, 32- and 16-column workgroups,
            # columns wholly past N, short slices of K with a tail, K = 0
            (16, 16384, 1000), (9, 20000, 64), (16, 8192, 8192), (15, 8192, 100), (12, 4096, 1000),
            (10, 1000, 4096), (13, 2050, 520), (11, 512, 33), (16, 128, 0), (9, 64, 16)]


@pytest.mark.parametrize("shape", FEW_ROWS, ids=lambda s: "x".join(map(str, s)))
def test_few_rows_of_a(shape):
    """A with at most 16 rows (the default path streams B once, 16 waves
    splitting K, their sums added in order; 9 to 16 rows with aligned rows
    on the matrix cores, everything else on the vector ALU): random inputs
    to the tolerance, integer inputs bit for bit, with padded leading
    dimensions and bases off 16-byte boundaries (the vector-ALU kernels),
    and K = 0."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M * 31 + N + K)
    R = oracle.sgemm_ref_f64(A, B)
    assert_parity(gemm(A, B), R, f"{shape}")
    assert_parity(gemm(A, B, pad=(3, 5, 1), off=(1, 2, 3)), R, f"{shape} padded")
    Ai, Bi = W.integer_inputs(M, N, K, seed=M + N + 7 * K)
    assert np.array_equal(gemm(Ai, Bi).astype(np.float64), oracle.sgemm_ref_f64(Ai, Bi)), f"{shape} integer"


@pytest.mark.parametrize("shape", [(16, 16384, 1000), (12, 8192, 800), (9, 4096, 2049)],
                         ids=lambda s: "x".join(map(str, s)))
def test_few_rows_matrix_cores_unaligned_a(shape):
    """9 to 16 rows with A's rows off 16-byte boundaries (lda = K + 1) and
    B aligned: the matrix-core kernel reading A one float at a time, with
    64-, 32- and 16-column workgroups; to the tolerance and bit for bit on
    integers."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M + 5 * N + K)
    assert_parity(gemm(A, B, pad=(1, 0, 0)), oracle.sgemm_ref_f64(A, B), f"{shape}")
    Ai, Bi = W.integer_inputs(M, N, K, seed=M + N + 11 * K)
    got = gemm(Ai, Bi, pad=(1, 0, 0)).astype(np.float64)
    assert np.array_equal(got, oracle.sgemm_ref_f64(Ai, Bi)), f"{shape} integer"


@pytest.mark.parametrize("shape", [(16, 16000, 500), (12, 8191, 2048), (9, 4100, 1000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_few_rows_matrix_cores_unaligned_b(shape):
    """9 to 16 rows with B's rows not aligned to a lane's group of columns
    (ldb = N + 1) and B within the last-level cache: the matrix-core kernel
    reading B one float per column, with 64- and 32-column workgroups and
    columns past N; to the tolerance and bit for bit on integers."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M + 7 * N + K)
    assert_parity(gemm(A, B, pad=(0, 1, 0)), oracle.sgemm_ref_f64(A, B), f"{shape}")
    Ai, Bi = W.integer_inputs(M, N, K, seed=M + N + 13 * K)
    got = gemm(Ai, Bi, pad=(0, 1, 0)).astype(np.float64)
    assert np.array_equal(got, oracle.sgemm_ref_f64(Ai, Bi)), f"{shape} integer"


@pytest.mark.parametrize("name", list(W.SKINNY))
def test_skinny_workloads(name):
    """The HBM-bound shapes the benchmark times (1x8192x8192, 8192x1x8192,
    8x65536x8192, 65536x4x8192, 16x65536x8192), at their sizes and seeds on
    the default path: every output against the oracle."""
    w = W.SKINNY[name]
    A, B = W.inputs_for(w)
    assert_parity(gemm(A, B, None), oracle.sgemm_ref_f64(A, B), w.describe())


FEW_COLS = [(17, 1, 1), (65, 3, 300), (1000, 4, 1000), (4099, 4, 257), (300, 2, 0),
            (100, 3, 4097), (70001, 2, 64), (129, 1, 256), (1000, 8, 1000), (4099, 16, 257),
            (8192, 1, 8192), (65536, 4, 8192), (77, 7, 300), (300, 12, 1000), (65536, 16, 8192),
            (4099, 4, 2500), (333, 6, 1028), (70001, 4, 1024), (4097, 8, 4096), (32769, 8, 1100),
            (40000, 6, 512),
            # one or two columns at 16, 8 and 4 rows per wave
            (5000, 1, 3000), (8192, 2, 2000), (2000, 2, 700)]


@pytest.mark.parametrize("shape", FEW_COLS, ids=lambda s: "x".join(map(str, s)))
def test_few_columns_of_b(shape):
    """B with at most 16 columns and A with more than 16 rows (the default
    path streams A once: a wave's lanes split each 256-k step and their sums
    meet in a butterfly; with 5 to 16 columns the step's rows of B are shared
    through LDS): random inputs to the tolerance, integer inputs bit
    for bit, padded leading dimensions and offset bases, a K tail shorter
    than a step, and K = 0."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M + 17 * N + K)
    R = oracle.sgemm_ref_f64(A, B)
    assert_parity(gemm(A, B), R, f"{shape}")
    assert_parity(gemm(A, B, pad=(5, 3, 2), off=(3, 1, 2)), R, f"{shape} padded")
    Ai, Bi = W.integer_inputs(M, N, K, seed=M + 3 * N + K)
    assert np.array_equal(gemm(Ai, Bi).astype(np.float64), oracle.sgemm_ref_f64(Ai, Bi)), f"{shape} integer"


@pytest.mark.parametrize("shape", [(1000, 4, 1000), (4099, 3, 2500), (70001, 4, 1024), (333, 6, 1028),
                                   (4097, 8, 4096), (32771, 7, 1028), (32768, 8, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_few_columns_aligned_padded(shape):
    """3 to 8 columns with A's rows on 16-byte boundaries but a leading
    dimension past K and an offset base (the 16-byte-load kernel with
    lda != K): full steps, a ragged last step and rows past the last whole
    wave, to the tolerance and bit for bit on integers."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M + 19 * N + K)
    R = oracle.sgemm_ref_f64(A, B)
    assert_parity(gemm(A, B, pad=(8 - K % 4, 1, 3), off=(4, 1, 2)), R, f"{shape} aligned, padded")
    Ai, Bi = W.integer_inputs(M, N, K, seed=M + 5 * N + K)
    got = gemm(Ai, Bi, pad=(8 - K % 4, 1, 3), off=(4, 1, 2))
    assert np.array_equal(got.astype(np.float64), oracle.sgemm_ref_f64(Ai, Bi)), f"{shape} integer"


SHORT_K = [(17, 17, 1), (100, 300, 16), (1000, 1001, 7), (4099, 257, 16), (64, 65, 3),
           (8192, 8192, 8)]


@pytest.mark.parametrize("shape", SHORT_K, ids=lambda s: "x".join(map(str, s)))
def test_short_k(shape):
    """K of at most 16 with A and B larger than 16 (short stages of the
    matrix-core kernels, C-write bound): random inputs to the tolerance,
    integer inputs bit for bit, padded leading dimensions and offset bases,
    ragged N."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=5 * M + N + K)
    R = oracle.sgemm_ref_f64(A, B)
    assert_parity(gemm(A, B), R, f"{shape}")
    assert_parity(gemm(A, B, pad=(2, 3, 1), off=(1, 2, 1)), R, f"{shape} padded")
    Ai, Bi = W.integer_inputs(M, N, K, seed=M + 2 * N + K)
    assert np.array_equal(gemm(Ai, Bi).astype(np.float64), oracle.sgemm_ref_f64(Ai, Bi)), f"{shape} integer"


def test_tall_single_column_past_2_26_rows():
    """B with one column and A with 2^26 + 1 rows (256 MB each for A and C):
    the A-streaming kernel's grid (one wave per 16 rows) fits the launch
    limit here, and every output is checked against the oracle."""
    M, N, K = (1 << 26) + 1, 1, 1
    rng = np.random.Generator(np.random.PCG64(2026))
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = np.array([[0.75]], np.float32)
    C = gemm(A, B)
    assert_parity(C, oracle.sgemm_ref_f64(A, B), f"{M}x{N}x{K}")


def test_tall_sixteen_columns_past_the_streaming_grid():
    """B with 16 columns and A with 2^28 + 64 rows: one wave per 4 rows would
    need more than 2^32 - 1 threads, so the library hands the shape to the
    matrix-core path.  C is 17 GB of NaN on the device; rows around the
    2^28 mark, the last rows and random rows are read back and compared,
    and a NaN count over all of C shows every output was written."""
    M, N, K = (1 << 28) + 64, 16, 1
    rng = np.random.Generator(np.random.PCG64(2028))
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    dA, dB = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    b.sgemm_f32(M, N, K, dA, K, dB, N, dC, N, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert int(torch.isnan(dC).sum()) == 0
    rows = np.unique(np.concatenate([[0, 1, (1 << 28) - 1, 1 << 28, M - 2, M - 1],
                                     rng.integers(0, M, 4096)]))
    got = dC[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert_parity(got, oracle.sgemm_ref_f64(A[rows], B), f"{M}x{N}x{K} sampled rows")
    del dA, dB, dC
    torch.cuda.empty_cache()
