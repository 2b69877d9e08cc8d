"""GPU parity tests of the 16-bit-input entry points gemm_bf16_f32 and
gemm_f16_f32 (bf16 / IEEE binary16 A and B, fp32 accumulate and C), called
through the C ABI and compared with the oracle's gemm_lowp_ref_f64 (the
ascending-k double sum over the exact values the 16-bit inputs hold).

Acceptance rule as for the fp32 path (oracle.parity): max|C - C_ref| <=
1e-4 * max|C_ref|.  Every product of two 16-bit values is exact in fp32, so
the same bound holds; integer-valued inputs must match bit for bit.  C, the
padding of every leading dimension and the bytes before each matrix hold
NaN, so an unwritten output or a read outside a matrix shows.  Shapes reach
both tile classes, each with its direct-to-LDS and its register loader.
"""
import numpy as np
import pytest

import oracle
from register_lds_tiled_amd import binding as b
from register_lds_tiled_amd import workloads as W
from tests.test_gpu_parity import (DEV, FULL_LIMIT, assert_parity, sampled_ref, sampled_values,
                                   tile_samples, to_device)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FMTS = ["bf16", "f16"]
NAN16 = {"bf16": 0x7FC0, "f16": 0x7E00}
ENTRY = {"bf16": b.gemm_bf16_f32, "f16": b.gemm_f16_f32}


def to_device16(X, ld, offset, fmt):
    """Row-major 16-bit storage X (uint16) in a fresh device buffer of int16
    with leading dimension ld, `offset` elements in; the rest holds NaN."""
    rows, cols = X.shape
    n = offset + max(rows * ld, 1)
    buf = torch.full((n,), np.int16(np.uint16(NAN16[fmt]).view(np.int16)).item(),
                     dtype=torch.int16, device=DEV)
    if rows and cols:
        view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
        view.copy_(torch.from_numpy(np.ascontiguousarray(X).view(np.int16)))
    return buf, buf.data_ptr() + 2 * offset


def gemm16(A16, B16, fmt, *, pad=(0, 0, 0), off=(0, 0, 0)):
    M, K = A16.shape
    N = B16.shape[1]
    lda, ldb, ldc = max(K + pad[0], 1), max(N + pad[1], 1), max(N + pad[2], 1)
    bufA, pA = to_device16(A16, lda, off[0], fmt)
    bufB, pB = to_device16(B16, ldb, off[1], fmt)
    bufC, pC = to_device(np.full((M, N), np.nan, np.float32), ldc, off[2])
    ENTRY[fmt](M, N, K, pA if K else 0, lda, pB if K else 0, ldb, pC, ldc,
               torch.cuda.current_stream())
    torch.cuda.synchronize()
    if M == 0 or N == 0:
        return np.zeros((M, N), np.float32)
    C = bufC[off[2]:off[2] + M * ldc].view(M, ldc)[:, :N].cpu().numpy()
    del bufA, bufB, bufC
    return C


# The large wave-tile kernel where A, B rows are aligned, N % 8 == 0,
# K % 8 == 0 and the k shift to whole four-stage groups, (128 - K % 128) %
# 128, is at most K / 3: 256x256 tiles beyond two 128x128 tiles per CU
# (whole tiles; ragged M and N; a grid of 144 ragged tiles; shifts of 72
# and, past three stages, 120), else 128x128 tiles (ragged 1000x1504,
# 1500x1000; whole 2048^2; shifts of 24, 96 and 120).  Otherwise, with
# aligned rows, large class (>= 128 tiles of 256x256): 8-wave tiles: whole
# tiles by DMA; ragged M, N and K tail by DMA plus edge loader; a grid of 144
# ragged tiles.  Mid class (64x128 tiles): the same cases.  Unaligned rows
# (lda = 45, 777, 2047, ...) take the mid tiles, with the dword-window loader
# for the whole stages of interior tiles and the element loader for the rest
# (odd K: A rows alternate between 4-byte and 2-byte starts; odd N: the same
# in B; N % 8 == 4: B rows 4-byte aligned only).
SHAPES = [(4096, 4096, 128), (4100, 4000, 384), (3000, 3072, 256),
          (1000, 1504, 512), (1500, 1000, 384), (2048, 2048, 128),
          (3000, 3000, 3000), (3072, 3072, 392), (2048, 2048, 104), (1024, 1024, 4000),
          (1000, 1504, 776),
          (4096, 4096, 64), (4100, 4000, 72), (4096, 4096, 45), (3000, 3072, 40),
          (2048, 2048, 56), (1000, 1504, 264), (1000, 1500, 777),
          (2048, 2048, 2047), (1024, 1001, 512), (1024, 1028, 1000),
          (1, 1, 1), (7, 5, 3), (64, 64, 32), (130, 70, 17), (256, 128, 4096)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes_random_and_integer(fmt, shape):
    M, N, K = shape
    A16, B16 = W.lowp_inputs(M, N, K, seed=M + 3 * N + K, fmt=fmt)
    assert_parity(gemm16(A16, B16, fmt), oracle.gemm_lowp_ref_f64(A16, B16, fmt), f"{fmt} {shape}")
    Ai, Bi = W.lowp_inputs(M, N, K, seed=M + N + 5 * K, fmt=fmt, integer=True)
    C = gemm16(Ai, Bi, fmt).astype(np.float64)
    assert np.array_equal(C, oracle.gemm_lowp_ref_f64(Ai, Bi, fmt)), f"{fmt} {shape} integer"


@pytest.mark.parametrize("fmt", FMTS)
def test_tile_edges_integer(fmt):
    for M in (63, 129, 255, 257):
        for N in (64, 130, 256, 300):
            for K in (31, 32, 33, 96):
                A16, B16 = W.lowp_inputs(M, N, K, seed=M * 7 + N * 3 + K, fmt=fmt, integer=True)
                C = gemm16(A16, B16, fmt).astype(np.float64)
                assert np.array_equal(C, oracle.gemm_lowp_ref_f64(A16, B16, fmt)), f"{M}x{N}x{K}"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("pad,off", [((8, 0, 3), (0, 0, 0)), ((1, 0, 0), (0, 0, 1)),
                                     ((0, 3, 0), (3, 1, 0)), ((8, 8, 4), (8, 8, 4))])
def test_leading_dims_and_alignment(fmt, pad, off):
    M, N, K = 600, 512, 136
    A16, B16 = W.lowp_inputs(M, N, K, seed=31, fmt=fmt)
    C = gemm16(A16, B16, fmt, pad=pad, off=off)
    assert_parity(C, oracle.gemm_lowp_ref_f64(A16, B16, fmt), f"{fmt} pad={pad} off={off}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("pad,off", [((8, 8, 3), (0, 0, 0)), ((8, 16, 0), (8, 8, 1))])
def test_large_wave_tile_leading_dims(fmt, pad, off):
    """The 16-bit large wave-tile kernel with padded leading dimensions and
    matrices that start past their buffers' first element (rows still
    16-byte aligned for A and B; C need not be)."""
    for M, N, K in ((4100, 4096, 256), (1100, 1024, 384)):
        A16, B16 = W.lowp_inputs(M, N, K, seed=33, fmt=fmt)
        C = gemm16(A16, B16, fmt, pad=pad, off=off)
        assert_parity(C, oracle.gemm_lowp_ref_f64(A16, B16, fmt), f"{fmt} {M}x{N}x{K} pad={pad} off={off}")


@pytest.mark.parametrize("fmt", FMTS)
def test_k_zero_and_empty(fmt):
    C = gemm16(np.zeros((70, 0), np.uint16), np.zeros((0, 90), np.uint16), fmt)
    assert C.shape == (70, 90) and np.all(C == 0.0)
    dC = torch.full((4, 4), 5.0, device=DEV)
    assert ENTRY[fmt](0, 4, 4, 0, 4, 0, 4, dC, 4, None) == b.SGEMM_OK
    torch.cuda.synchronize()
    assert bool((dC == 5.0).all())


@pytest.mark.parametrize("fmt", FMTS)
def test_nan_inf_propagate(fmt):
    M, N, K = 300, 260, 100
    A16, B16 = W.lowp_inputs(M, N, K, seed=8, fmt=fmt)
    inf = {"bf16": 0x7F80, "f16": 0x7C00}[fmt]
    A16[3, 7] = NAN16[fmt]
    B16[11, 200] = inf
    C = gemm16(A16, B16, fmt)
    R = oracle.gemm_lowp_ref_f64(A16, B16, fmt)
    assert np.array_equal(np.isnan(C), np.isnan(R)) and np.array_equal(np.isinf(C), np.isinf(R))
    fin = np.isfinite(R)
    assert np.isnan(C[3]).all() and not fin[:, 200].any()
    assert_parity(C[fin], R[fin], f"{fmt} finite part")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", ["sq2048", "sq8192"])
def test_workload_sizes(fmt, name):
    """The benchmarked sizes: 2048^3 in full against gemm_lowp_ref_f64;
    8192^3 with every output written (C starts as NaN) and a row and a
    column in every 128 band and an entry in every 64 x 64 tile, by the
    oracle on the decoded values (pinned equal to gemm_lowp_ref_f64)."""
    w = W.WORKLOADS[name]
    A16, B16 = W.lowp_inputs(w.M, w.N, w.K, seed=w.seed, fmt=fmt, dist=w.dist)
    C = gemm16(A16, B16, fmt)
    if w.M * w.N * w.K <= FULL_LIMIT:
        assert_parity(C, oracle.gemm_lowp_ref_f64(A16, B16, fmt), f"{fmt} {w.describe()}")
        return
    unwritten = int(np.isnan(C).sum())
    assert unwritten == 0, f"{fmt} {w.describe()}: {unwritten} outputs never written"
    Ad, Bd = oracle.decode16_f32(A16, fmt), oracle.decode16_f32(B16, fmt)
    got, exp = sampled_values(C, sampled_ref(Ad, Bd, tile_samples(w.M, w.N, seed=99))[1])
    assert_parity(got, exp, f"{fmt} {w.describe()} (a row and a column per 128 band, "
                            "an entry per 64x64 tile)")


@pytest.mark.parametrize("fmt", FMTS)
def test_deterministic_repeats(fmt):
    A16, B16 = W.lowp_inputs(2048, 2048, 512, seed=5, fmt=fmt)
    first = gemm16(A16, B16, fmt)
    for _ in range(2):
        assert np.array_equal(gemm16(A16, B16, fmt), first)


def test_alias_rejected_on_device():
    dA = torch.zeros((64, 64), dtype=torch.int16, device=DEV)
    dB = torch.zeros((64, 64), dtype=torch.int16, device=DEV)
    dC = torch.full((64, 64), 7.0, device=DEV)
    # C (fp32, 64 x 64) placed on A's storage
    assert b.gemm_bf16_f32(64, 64, 64, dA, 64, dB, 64, dA.data_ptr(), 64, None,
                           check=False) == b.SGEMM_EALIAS
    assert b.gemm_f16_f32(64, 64, 64, dA, 64, dB, 64, dB.data_ptr() - 4, 64, None,
                          check=False) == b.SGEMM_EALIAS
    torch.cuda.synchronize()
    assert bool((dC == 7.0).all())
