"""GPU parity tests of the fused epilogue entry point sgemm_f32_ex,
C = act(alpha * A.B + beta * C + bias[col]), called through the C ABI and
compared with the oracle's sgemm_ex_ref_f64 on the same seeded inputs.

Acceptance rule as for the plain product (oracle.parity): max|C - C_ref| <=
1e-4 * max|C_ref| over the compared outputs.  The epilogue operands are drawn
on the scale of the dot products so that the largest output is not far below
the terms that make it up.  Integer-valued operands with integer alpha, beta
and bias must match bit for bit.  Every tile class of the matrix-core path
(register-staged 256/128/64 and direct-to-LDS 128/64) and the streaming
kernels of the few-row and few-column shapes are covered.
"""
import numpy as np
import pytest

import oracle
from register_lds_tiled_amd import binding as b
from register_lds_tiled_amd import workloads as W
from tests.test_gpu_parity import (CLASS_SHAPES, DEV, EDGE_SHAPES, FULL_LIMIT, assert_parity,
                                   edge_samples, gemm, tile_samples, to_device)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def gemm_ex(A, B, C_in, alpha, beta, bias, act, *, pad=(0, 0, 0), off=(0, 0, 0), ret_buf=False):
    """Run sgemm_f32_ex with C preloaded with C_in (leading dimension N +
    pad[2]; padding and the space before C hold NaN).  Returns C."""
    M, K = A.shape
    N = B.shape[1]
    lda, ldb, ldc = max(K + pad[0], 1), max(N + pad[1], 1), max(N + pad[2], 1)
    bufA, pA = to_device(A, lda, off[0])
    bufB, pB = to_device(B, ldb, off[1])
    bufC, pC = to_device(C_in, ldc, off[2])
    dbias = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias)).to(DEV)
    b.sgemm_f32_ex(M, N, K, pA if K else 0, lda, pB if K else 0, ldb, pC, ldc, alpha, beta,
                   dbias, act, torch.cuda.current_stream())
    torch.cuda.synchronize()
    C = bufC[off[2]:off[2] + M * ldc].view(M, ldc)[:, :N].cpu().numpy()
    if ret_buf:
        return C, bufC.cpu().numpy(), ldc
    return C


def scale_of(K):
    """Typical |A.B| of Uniform(-1,1) inputs: sqrt(K/9)."""
    return max(1.0, float(np.sqrt(K / 9.0)))


# (alpha, beta, with bias, act): every term of the epilogue, each alone and
# all together.
COMBOS = [(-0.5, 2.0, True, b.ACT_RELU), (2.5, 0.0, True, b.ACT_NONE),
          (1.0, 1.0, False, b.ACT_NONE), (1.0, 0.0, False, b.ACT_RELU)]


@pytest.mark.parametrize("shape", CLASS_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_epilogue_tile_classes(shape):
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=11 * M + N + K)
    C_in, bias = W.epilogue_inputs(M, N, seed=M + 5 * N, scale=scale_of(K))
    for alpha, beta, with_bias, act in COMBOS:
        bs = bias if with_bias else None
        C = gemm_ex(A, B, C_in, alpha, beta, bs, act)
        R = oracle.sgemm_ex_ref_f64(A, B, C_in, alpha, beta, bs, act)
        assert_parity(C, R, f"{shape} alpha={alpha} beta={beta} bias={with_bias} act={act}")


@pytest.mark.parametrize("shape", CLASS_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_epilogue_integer_exact(shape):
    M, N, K = shape
    A, B = W.integer_inputs(M, N, K, seed=3 * M + N + 2 * K)
    C_in, bias = W.epilogue_inputs(M, N, seed=7 + M, scale=50, integer=True)
    for alpha, beta, act in [(2.0, -1.0, b.ACT_RELU), (-1.0, 3.0, b.ACT_NONE)]:
        C = gemm_ex(A, B, C_in, alpha, beta, bias, act)
        R = oracle.sgemm_ex_ref_f64(A, B, C_in, alpha, beta, bias, act)
        assert np.array_equal(C.astype(np.float64), R), f"{shape} alpha={alpha} beta={beta}"


@pytest.mark.parametrize("shape", [(300, 260, 100), (2048, 2048, 64), (4096, 4096, 32),
                                   (8, 1000, 100), (16, 4099, 300), (1000, 4, 1000),
                                   (4099, 16, 257), (8192, 1, 8192)],
                         ids=lambda s: "x".join(map(str, s)))
def test_identity_epilogue_is_the_plain_product(shape):
    """The identity epilogue runs the kernel sgemm_f32 runs, the skinny-shape
    kernels (A of at most 16 rows, B of at most 16 columns) included: the
    results are equal bit for bit."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M + K)
    C = gemm_ex(A, B, np.full((M, N), np.nan, np.float32), 1.0, 0.0, None, b.ACT_NONE)
    assert np.array_equal(C, gemm(A, B, None))


# A of at most 16 rows or B of at most 16 columns: the streaming kernels
# (vector ALU; 9 to 16 aligned rows on the matrix cores) apply the epilogue
# in their final store.
SKINNY_EX = [(1, 8192, 8192), (3, 64, 16), (8, 1000, 100), (8, 4099, 1000), (13, 2050, 520),
             (16, 8192, 1000), (16, 4099, 300), (12, 16000, 77), (17, 1, 1), (1000, 4, 1000),
             (4099, 16, 257), (8192, 1, 8192), (32769, 8, 1100), (300, 2, 0), (16, 128, 0)]


@pytest.mark.parametrize("shape", SKINNY_EX, ids=lambda s: "x".join(map(str, s)))
def test_epilogue_skinny_shapes(shape):
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=13 * M + N + K)
    C_in, bias = W.epilogue_inputs(M, N, seed=M + 3 * N, scale=scale_of(K))
    for alpha, beta, with_bias, act in COMBOS:
        bs = bias if with_bias else None
        C = gemm_ex(A, B, C_in, alpha, beta, bs, act)
        R = oracle.sgemm_ex_ref_f64(A, B, C_in, alpha, beta, bs, act)
        assert_parity(C, R, f"{shape} alpha={alpha} beta={beta} bias={with_bias} act={act}")
    Ai, Bi = W.integer_inputs(M, N, K, seed=M + 2 * N + 3 * K)
    Ci, biasi = W.epilogue_inputs(M, N, seed=5 + N, scale=50, integer=True)
    C = gemm_ex(Ai, Bi, Ci, 2.0, -1.0, biasi, b.ACT_RELU, pad=(1, 3, 2), off=(1, 2, 3))
    R = oracle.sgemm_ex_ref_f64(Ai, Bi, Ci, 2.0, -1.0, biasi, b.ACT_RELU)
    assert np.array_equal(C.astype(np.float64), R), f"{shape} integer, padded"


@pytest.mark.parametrize("shape", [(500, 700, 45), (512, 768, 45), (2048, 2048, 100),
                                   (4096, 4096, 48)], ids=lambda s: "x".join(map(str, s)))
def test_beta_zero_never_reads_C(shape):
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M * 7 + K)
    _, bias = W.epilogue_inputs(M, N, seed=3, scale=scale_of(K))
    C = gemm_ex(A, B, np.full((M, N), np.nan, np.float32), 1.5, 0.0, bias, b.ACT_RELU)
    assert np.all(np.isfinite(C))
    assert_parity(C, oracle.sgemm_ex_ref_f64(A, B, None, 1.5, 0.0, bias, b.ACT_RELU), str(shape))


@pytest.mark.parametrize("shape", [(1, 1, 1), (7, 5, 3), (64, 64, 16), (130, 70, 17)],
                         ids=lambda s: "x".join(map(str, s)))
def test_small_shapes(shape):
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=sum(shape))
    C_in, bias = W.epilogue_inputs(M, N, seed=1, scale=scale_of(K))
    C = gemm_ex(A, B, C_in, -1.25, 0.5, bias, b.ACT_RELU)
    assert_parity(C, oracle.sgemm_ex_ref_f64(A, B, C_in, -1.25, 0.5, bias, b.ACT_RELU), str(shape))


def test_k_zero_is_epilogue_of_empty_sum():
    M, N = 200, 300
    C_in, bias = W.epilogue_inputs(M, N, seed=9, scale=20, integer=True)
    A, B = np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32)
    for beta, act in [(0.5, b.ACT_RELU), (-2.0, b.ACT_NONE), (0.0, b.ACT_RELU)]:
        C = gemm_ex(A, B, C_in, 3.0, beta, bias, act)
        R = oracle.sgemm_ex_ref_f64(A, B, C_in, 3.0, beta, bias, act)
        assert np.array_equal(C.astype(np.float64), R), f"beta={beta} act={act}"


@pytest.mark.parametrize("shape", [(500, 700, 45), (2048, 2048, 64), (4096, 4096, 48)],
                         ids=lambda s: "x".join(map(str, s)))
def test_relu_keeps_nan_and_zeroes_negatives(shape):
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M + 1)
    A[5, 3] = np.nan
    C = gemm_ex(A, B, np.zeros((M, N), np.float32), 1.0, 0.0, None, b.ACT_RELU)
    assert np.all(np.isnan(C[5]))
    rest = np.delete(C, 5, axis=0)
    assert np.all(rest >= 0.0) and np.mean(rest == 0.0) > 0.3
    R = np.delete(oracle.sgemm_ex_ref_f64(A, B, act=1), 5, axis=0)
    assert_parity(rest, R, f"{shape} rows without NaN")


@pytest.mark.parametrize("pad,off", [((0, 0, 3), (0, 0, 0)), ((3, 0, 5), (0, 0, 1)),
                                     ((0, 1, 0), (1, 0, 2)), ((4, 4, 4), (4, 4, 4))])
def test_leading_dims_and_alignment(pad, off):
    M, N, K = 1030, 777, 91
    A, B = W.random_inputs(M, N, K, seed=21)
    C_in, bias = W.epilogue_inputs(M, N, seed=22, scale=scale_of(K))
    C, buf, ldc = gemm_ex(A, B, C_in, 0.75, -1.5, bias, b.ACT_RELU, pad=pad, off=off, ret_buf=True)
    assert_parity(C, oracle.sgemm_ex_ref_f64(A, B, C_in, 0.75, -1.5, bias, b.ACT_RELU), f"{pad} {off}")
    # the padding columns of C and the floats before it are never written
    if ldc > N:
        assert np.all(np.isnan(buf[off[2]:off[2] + M * ldc].reshape(M, ldc)[:, N:]))
    assert np.all(np.isnan(buf[:off[2]]))


@pytest.mark.parametrize("name", ["sq2048", "sq8192"])
def test_workload_sizes(name):
    """The benchmarked sizes with every epilogue term on: 2048^3 in full;
    8192^3 with every output written (C_in is finite, so a NaN would be an
    output never stored) and the oracle on a row and a column in every
    128 band and an entry in every 64 x 64 tile."""
    w = W.WORKLOADS[name]
    A, B = W.inputs_for(w)
    C_in, bias = W.epilogue_inputs(w.M, w.N, seed=77, scale=float(np.sqrt(w.K)))
    args = (C_in, 0.5, -1.0, bias, b.ACT_RELU)
    C = gemm_ex(A, B, *args)
    if w.M * w.N * w.K <= FULL_LIMIT:
        assert_parity(C, oracle.sgemm_ex_ref_f64(A, B, *args), w.describe())
        return
    assert np.isfinite(C).all(), f"{w.describe()}: outputs never written or not finite"
    rows, cols, er, ec = tile_samples(w.M, w.N, seed=4343)
    ex = lambda Ax, Bx, Cx, bx: oracle.sgemm_ex_ref_f64(Ax, Bx, Cx, 0.5, -1.0, bx, b.ACT_RELU)  # noqa: E731
    R_rows = ex(A[rows], B, C_in[rows], bias)
    R_cols = ex(A, np.ascontiguousarray(B[:, cols]), np.ascontiguousarray(C_in[:, cols]),
                np.ascontiguousarray(bias[cols]))
    R_e = oracle.sgemm_ex_ref_f64_entries(A, B, er, ec, *args)
    got = np.concatenate([C[rows].ravel(), C[:, cols].ravel(), C[er, ec]])
    exp = np.concatenate([R_rows.ravel(), R_cols.ravel(), R_e])
    assert_parity(got, exp, w.describe() + " (a row and a column per 128 band, an entry per tile)")


def test_deterministic_repeats():
    M, N, K = 2048, 2048, 256
    A, B = W.random_inputs(M, N, K, seed=5)
    C_in, bias = W.epilogue_inputs(M, N, seed=6, scale=scale_of(K))
    first = gemm_ex(A, B, C_in, 1.1, 0.9, bias, b.ACT_RELU)
    for _ in range(2):
        assert np.array_equal(gemm_ex(A, B, C_in, 1.1, 0.9, bias, b.ACT_RELU), first)


def test_bias_overlapping_C_rejected_on_device():
    M, N, K = 64, 64, 16
    dA = torch.zeros((M, K), dtype=torch.float32, device=DEV)
    dB = torch.zeros((K, N), dtype=torch.float32, device=DEV)
    dC = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    st = b.sgemm_f32_ex(M, N, K, dA, K, dB, N, dC, N, 1.0, 0.0, dC[3], 0, None, check=False)
    assert st == b.SGEMM_EALIAS
    st = b.sgemm_f32_ex(M, N, K, dA, K, dB, N, dC, N, 1.0, 0.0, None, 5, None, check=False)
    assert st == b.SGEMM_EINVAL_ACT
    torch.cuda.synchronize()
    assert bool((dC == 7.0).all())


@pytest.mark.parametrize("shape", EDGE_SHAPES[:4] + EDGE_SHAPES[6:8],
                         ids=lambda s: "x".join(map(str, s)))
def test_epilogue_large_wave_tile_edges(shape):
    """The fused epilogue of the large wave-tile kernels on ragged tiles,
    shifted K and 4-byte A: sampled rows, columns and entries."""
    M, N, K, pad = shape
    A, B = W.random_inputs(M, N, K, seed=K + 5)
    C_in, bias = W.epilogue_inputs(M, N, seed=M + 9, scale=scale_of(K))
    args = (C_in, -0.75, 1.25, bias, b.ACT_RELU)
    C = gemm_ex(A, B, *args, pad=(pad, 0, 0))
    rows, cols, er, ec = edge_samples(M, N, N + K)
    # whole rows, whole columns, scattered entries
    rr = np.concatenate([np.repeat(rows, N), np.repeat(np.arange(M), len(cols)), er])
    cc = np.concatenate([np.tile(np.arange(N), len(rows)), np.tile(cols, M), ec])
    R = oracle.sgemm_ex_ref_f64_entries(A, B, rr, cc, *args)
    assert_parity(C[rr, cc], R, f"{shape} fused (sampled)")


def test_epilogue_ksplit_class():
    """The K-split direct-to-LDS kernel (reached with A rows 2^22 floats
    apart, too long for the large wave-tile kernel's 32-bit offsets): every
    epilogue term, partial sums of the four groups added first."""
    M, N, K = 128, 256, 520
    A, B = W.random_inputs(M, N, K, seed=17)
    C_in, bias = W.epilogue_inputs(M, N, seed=18, scale=scale_of(K))
    args = (C_in, 1.5, -0.5, bias, b.ACT_RELU)
    C = gemm_ex(A, B, *args, pad=((1 << 22) - K, 0, 0), off=(0, 0, 1))
    assert_parity(C, oracle.sgemm_ex_ref_f64(A, B, *args), "K-split fused")


@pytest.mark.parametrize("shape,off", [((1000, 1001, 777), (0, 0, 0)), ((2048, 2048, 512), (0, 0, 1))],
                         ids=["N%4", "C-off"])
def test_epilogue_large_wave_tile_scalar_c(shape, off):
    """The large wave-tile kernel storing C one float at a time (N % 4 != 0,
    or C rows off 16 bytes): C's previous values, the bias and the store,
    each guarded at column N."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=23)
    C_in, bias = W.epilogue_inputs(M, N, seed=24, scale=scale_of(K))
    args = (C_in, 0.75, 1.25, bias, b.ACT_RELU)
    C = gemm_ex(A, B, *args, off=off)
    assert_parity(C, oracle.sgemm_ex_ref_f64(A, B, *args), f"{shape} off={off}")


@pytest.mark.parametrize("shape", [(2048, 2048, 64), (1000, 1500, 777), (500, 700, 45),
                                   (4096, 4096, 48)], ids=lambda s: "x".join(map(str, s)))
def test_signed_zero_and_nan_through_the_epilogue(shape):
    """Zero rows of A give a product row of +0; alpha < 0 turns it into
    -0.0, which every absent term must leave alone (beta == 0 with C not
    read, no bias, ReLU keeps -0.0 since -0.0 < 0 is false) -- the sign bit
    is compared with the oracle's.  A NaN in A's row 1 passes every term."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M + 4 * K)
    A[0, :] = 0.0
    A[M // 2, :] = 0.0
    A[1, K // 3] = np.nan
    C_nan = np.full((M, N), np.nan, np.float32)
    for beta, C_in, bias, act in [(0.0, C_nan, None, b.ACT_NONE), (0.0, C_nan, None, b.ACT_RELU),
                                  (1.0, np.full((M, N), -0.0, np.float32), None, b.ACT_RELU)]:
        C = gemm_ex(A, B, C_in, -1.5, beta, bias, act)
        R = oracle.sgemm_ex_ref_f64(A, B, C_in, -1.5, beta, bias, act)
        for r in (0, M // 2):
            assert np.all(C[r] == 0.0) and np.array_equal(np.signbit(C[r]), np.signbit(R[r])), \
                f"{shape} beta={beta} act={act} row {r}"
        assert np.isnan(C[1]).all()
        rest = np.delete(C, [0, 1, M // 2], axis=0)
        assert_parity(rest, np.delete(R, [0, 1, M // 2], axis=0), f"{shape} beta={beta} act={act}")
