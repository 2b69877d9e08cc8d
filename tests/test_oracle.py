"""CPU tests of the oracle against its pins, plus mutation tests that plant
plausible mistakes in a copy of the oracle source and check that a pin
catches each one.  No GPU needed."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from register_lds_tiled_amd import workloads
from tests import pins

ROOT = pins.ROOT


@pytest.fixture(scope="module")
def o():
    oracle.build()
    return oracle.OracleLib(oracle._LIB)


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)


def test_unfused_reading_does_not_match_page():
    """Evidence for the fused-FMA reading: an fp32 multiply-then-add loop in
    k order does not print the page's digits, the fused one (pinned above)
    does."""
    K, printed = pins.read_golden()
    A, B = workloads.worked_example(K)
    c = np.zeros(4, np.float32)
    for k in range(K):
        c = (c + np.float32(A[0, k]) * B[k, :4]).astype(np.float32)
    assert ["%f" % float(v) for v in c] != printed


def test_micro_full_tile_fp32_close_to_f64(o):
    A, B = workloads.worked_example(1024)
    C32 = o.micro4x4_seq_fma_f32(A, B)
    C64 = o.sgemm_ref_f64(A, B)
    ok, err, ref, tol = oracle.parity(C32, C64)
    assert ok, (err, tol)


def test_entries_match_full_on_ragged_sample(o):
    A, B = workloads.random_inputs(130, 70, 45, seed=3)
    C = o.sgemm_ref_f64(A, B)
    rng = np.random.default_rng(1)
    r = rng.integers(0, 130, 200)
    c = rng.integers(0, 70, 200)
    assert np.array_equal(o.sgemm_ref_f64_entries(A, B, r, c), C[r, c])


def test_empty_shapes(o):
    assert o.sgemm_ref_f64(np.zeros((0, 5), np.float32), np.zeros((5, 3), np.float32)).shape == (0, 3)
    assert o.sgemm_ref_f64(np.zeros((4, 5), np.float32), np.zeros((5, 0), np.float32)).shape == (4, 0)
    with pytest.raises(ValueError):
        o.sgemm_ref_f64(np.zeros((4, 5), np.float32), np.zeros((6, 2), np.float32))
    with pytest.raises(IndexError):
        o.sgemm_ref_f64_entries(np.zeros((4, 5), np.float32), np.zeros((5, 2), np.float32), [4], [0])


def test_parity_rule():
    ref = np.array([[1.0, -2.0], [0.5, 4.0]])
    ok, err, mx, tol = oracle.parity(ref + 3e-4, ref)
    assert ok and mx == 4.0 and abs(tol - 4e-4) < 1e-18
    assert not oracle.parity(ref + 5e-4, ref)[0]
    bad = ref.copy(); bad[0, 1] = np.nan
    assert not oracle.parity(bad, ref)[0]
    bad[0, 1] = np.inf
    assert not oracle.parity(bad, ref)[0]
    z = np.zeros((2, 2))
    assert oracle.parity(z, z)[0]
    assert not oracle.parity(z + 1e-30, z)[0]


# ---------------------------------------------------------------- mutation --
# Each mutant is the oracle source with one plausible mistake planted; the
# pins must reject every one of them.  Each runs in a child process so that a
# mutant that reads out of bounds cannot take the test runner down.
MUTANTS = {
    "dropped_last_term": ("for (int k = 0; k < K; ++k)\n                s +=",
                          "for (int k = 0; k + 1 < K; ++k)\n                s +="),
    "wrong_sign": ("                s += (double)A[(size_t)i * lda + k]",
                   "                s -= (double)A[(size_t)i * lda + k]"),
    "transposed_B": ("(double)B[(size_t)k * ldb + j];\n            C[(size_t)i * ldc + j] = s;",
                     "(double)B[(size_t)(j % K) * ldb + (k % N)];\n            C[(size_t)i * ldc + j] = s;"),
    "wrong_A_row": ("s += (double)A[(size_t)i * lda + k] * (double)B[(size_t)k * ldb + j];\n            C[",
                    "s += (double)A[(size_t)(M - 1 - i) * lda + k] * (double)B[(size_t)k * ldb + j];\n            C["),
    "float_accumulator": ("            double s = 0.0;\n            for (int k = 0; k < K; ++k)\n                s += (double)A[(size_t)i",
                          "            float s = 0.0f;\n            for (int k = 0; k < K; ++k)\n                s += (double)A[(size_t)i"),
    "unfused_micro": ("c = fmaf(A[(size_t)r * K + k], B[(size_t)k * 4 + j], c);",
                      "{ volatile float p = A[(size_t)r * K + k] * B[(size_t)k * 4 + j]; c = c + p; }"),
    "micro_B_transposed": ("B[(size_t)k * 4 + j], c);", "B[(size_t)j * 4 + (k % 4)], c);"),
    "epilogue_beta_dropped": ("if (beta != 0.0) v += beta * (double)Cin[(size_t)i * ldc + j];",
                              "if (beta != 0.0) v += 0.0 * (double)Cin[(size_t)i * ldc + j];"),
    "epilogue_C_transposed": ("v += beta * (double)Cin[(size_t)i * ldc + j];",
                              "v += beta * (double)Cin[(size_t)j * ldc + i];"),
    "epilogue_bias_per_row": ("if (bias) v += (double)bias[j];", "if (bias) v += (double)bias[i];"),
    "epilogue_relu_drops_nan": ("if (act == 1 && v < 0.0) v = 0.0;", "if (act == 1 && !(v > 0.0)) v = 0.0;"),
    "lowp_bf16_shift": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "lowp_f16_bias": ("ldexp((double)(m + 1024), e - 25)", "ldexp((double)(m + 1024), e - 24)"),
    "lowp_f16_subnormal": ("if (e == 0) v = ldexp((double)m, -24);", "if (e == 0) v = ldexp((double)m, -25);"),
    "lowp_f16_implicit_bit": ("ldexp((double)(m + 1024), e - 25)", "ldexp((double)m, e - 15)"),
    "lowp_B_transposed": ("b[(size_t)k * N + j] = decode16(fmt, B[(size_t)k * ldb + j]);",
                          "b[(size_t)k * N + j] = decode16(fmt, B[(size_t)(j % K) * ldb + (k % N)]);"),
    "epilogue_alpha_after_bias": ("    double v = alpha * s;\n    if (beta != 0.0) v += beta",
                                  "    double v = s;\n    if (beta != 0.0) v += beta"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "sgemm_ref.c"), encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    msrc = tmp_path / "mutant.c"
    msrc.write_text(src.replace(old, new), encoding="utf-8")
    lib = str(tmp_path / "libmutant.so")
    oracle.build(str(msrc), lib)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "pins.py"), lib],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}{r.stderr}"
