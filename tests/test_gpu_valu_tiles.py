"""GPU parity tests of the VALU path's tile configurations, each called
through the C ABI (sgemm_f32_valu_tile) and compared with the oracle.

Every configuration -- block tile, wave tile, lane tile TM x TN -- sums each
output over k in ascending order with one fused multiply-add per k, so all
of them must agree with each other bit for bit, integer inputs must match the
oracle bit for bit, and random inputs must meet max|C - C_ref| <= 1e-4
max|C_ref|.  C starts as NaN, so an output a configuration never writes
fails.  Shapes reach ragged edges in M, N and K, single rows and columns,
unaligned leading dimensions and several tiles per dimension.
"""
import numpy as np
import pytest

import oracle
from register_lds_tiled_amd import binding as b
from register_lds_tiled_amd import workloads as W
from tests.test_gpu_parity import DEV, assert_parity, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAX_TILES = 15     # the built table's size (test_all_tiles_are_parametrized checks it)


def n_tiles():
    return b.sgemm_valu_tile_count()


def gemm_tile(A, B, tile, *, pad=(0, 0, 0), off=(0, 0, 0)):
    M, K = A.shape
    N = B.shape[1]
    lda, ldb, ldc = max(K + pad[0], 1), max(N + pad[1], 1), max(N + pad[2], 1)
    bufA, pA = to_device(A, lda, off[0])
    bufB, pB = to_device(B, ldb, off[1])
    bufC, pC = to_device(np.full((M, N), np.nan, np.float32), ldc, off[2])
    b.sgemm_f32_valu_tile(M, N, K, pA, lda, pB, ldb, pC, ldc, torch.cuda.current_stream(), tile)
    torch.cuda.synchronize()
    C = bufC[off[2]:off[2] + M * ldc].view(M, ldc)[:, :N].cpu().numpy()
    del bufA, bufB, bufC
    return C


SHAPES = [(1, 1, 1), (7, 5, 3), (64, 64, 16), (127, 129, 17), (300, 260, 100),
          (257, 511, 33), (520, 390, 300), (1000, 1500, 777), (33, 1000, 7)]


@pytest.mark.parametrize("tile", range(MAX_TILES))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_tile_random(tile, shape):
    if tile >= n_tiles():
        pytest.skip("configuration not built")
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M * 13 + N + K)
    assert_parity(gemm_tile(A, B, tile), oracle.sgemm_ref_f64(A, B),
                  f"{b.sgemm_valu_tile_name(tile)} {shape}")


@pytest.mark.parametrize("tile", range(MAX_TILES))
def test_tile_integer_exact_and_padded(tile):
    if tile >= n_tiles():
        pytest.skip("configuration not built")
    for (M, N, K) in ((129, 257, 33), (1000, 1500, 777), (255, 70, 1000)):
        A, B = W.integer_inputs(M, N, K, seed=M + 2 * N + K)
        R = oracle.sgemm_ref_f64(A, B)
        assert np.array_equal(gemm_tile(A, B, tile).astype(np.float64), R), (tile, M, N, K)
        C = gemm_tile(A, B, tile, pad=(3, 1, 2), off=(1, 2, 3))
        assert np.array_equal(C.astype(np.float64), R), (tile, M, N, K, "padded")


def test_all_tiles_are_parametrized():
    assert n_tiles() == MAX_TILES


def test_all_tiles_give_the_same_bits():
    """Ascending-k fused sums in every configuration: identical results."""
    M, N, K = 1000, 1500, 777
    A, B = W.random_inputs(M, N, K, seed=1004)
    first = gemm_tile(A, B, 0)
    assert_parity(first, oracle.sgemm_ref_f64(A, B), "tile 0 ragged")
    for t in range(1, n_tiles()):
        C = gemm_tile(A, B, t)
        assert np.array_equal(C.view(np.uint32), first.view(np.uint32)), b.sgemm_valu_tile_name(t)


@pytest.mark.parametrize("shape", [(2048, 2048, 128), (4096, 4096, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_valu_path_matches_its_tiles(shape):
    """SGEMM_PATH_VALU runs one of the built configurations (the 4x4 lane
    tile on a small grid, the 8x8 one from 4 tiles of 128 x 128 per CU):
    the same bits as every configuration, and the oracle's values."""
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=77)
    dA, dB = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    dC = torch.full((M, N), float("nan"), device=DEV)
    b.sgemm_f32_path(M, N, K, dA, K, dB, N, dC, N, None, b.PATH_VALU)
    torch.cuda.synchronize()
    C = dC.cpu().numpy()
    assert np.array_equal(C.view(np.uint32), gemm_tile(A, B, 0).view(np.uint32))
    rows = np.arange(0, M, 97)
    assert_parity(C[rows], oracle.sgemm_ref_f64(A[rows], B), f"VALU path {shape}")
