"""CPU checks of the seeded input generators shared by the tests, the
benchmark and the oracle's callers: determinism, shapes and distributions,
and the 16-bit encodings (round to nearest even, against torch's and numpy's
own conversions)."""
import numpy as np
import pytest

from register_lds_tiled_amd import workloads as W


def test_random_inputs_are_seeded_and_shaped():
    A, B = W.random_inputs(7, 5, 3, seed=11)
    A2, B2 = W.random_inputs(7, 5, 3, seed=11)
    assert A.shape == (7, 3) and B.shape == (3, 5) and A.dtype == np.float32
    assert np.array_equal(A, A2) and np.array_equal(B, B2)
    assert not np.array_equal(A, W.random_inputs(7, 5, 3, seed=12)[0])
    U, _ = W.random_inputs(400, 1, 400, seed=3)
    assert U.min() >= -1.0 and U.max() <= 1.0 and abs(U.mean()) < 0.02
    G, _ = W.random_inputs(400, 1, 400, seed=3, dist="normal")
    assert abs(G.std() - 1.0) < 0.02


def test_integer_inputs_range():
    A, B = W.integer_inputs(50, 40, 30, seed=1)
    assert set(np.unique(A)) <= set(range(-3, 4)) and set(np.unique(B)) <= set(range(-3, 4))


def test_bf16_encoding_rounds_to_nearest_even():
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(5))
    X = np.concatenate([rng.uniform(-4, 4, 20000), rng.standard_normal(20000) * 1e-3]).astype(np.float32)
    # exact ties (the low 16 bits are 0x8000) with a finite exponent
    ties = (rng.integers(0, 2 ** 31, 2000, dtype=np.uint32) & 0x7FFF0000) | 0x8000
    ties = ties[(ties >> 23) & 0xFF != 0xFF]
    X = np.concatenate([X, ties.view(np.float32)])
    got = W.to_bf16_storage(X)
    want = torch.from_numpy(X).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_f16_encoding_is_numpy_binary16():
    X = np.array([1.0, -2.0, 65504.0, 2.0 ** -24, 0.1, 1.0 / 3.0], np.float32)
    got = W.to_f16_storage(X)
    assert np.array_equal(got, X.astype(np.float16).view(np.uint16))
    assert got[0] == 0x3C00 and got[1] == 0xC000 and got[2] == 0x7BFF and got[3] == 0x0001


def test_lowp_integer_inputs_are_exact():
    for fmt in ("bf16", "f16"):
        A16, B16 = W.lowp_inputs(20, 30, 40, seed=4, fmt=fmt, integer=True)
        A, B = W.integer_inputs(20, 30, 40, seed=4)
        dec = {"bf16": lambda x: (x.astype(np.uint32) << 16).view(np.float32),
               "f16": lambda x: x.view(np.float16).astype(np.float32)}[fmt]
        assert np.array_equal(dec(A16), A) and np.array_equal(dec(B16), B)
