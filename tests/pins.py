"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.OracleLib`` and raises ``AssertionError``
when the oracle disagrees with:

* the first page's printed worked-example output (tests/golden/);
* exact rational sums (``fractions.Fraction``) on tiny and worked shapes,
  within the rounding bound of a double-precision sum of exact products;
* exact integer products (numpy int64 ``@``) on integer-valued inputs;
* algebraic invariants: A.I = A, I.B = B, A.0 = 0, ones.ones = K,
  (A.B)^T = B^T.A^T;
* a float64 library product (numpy ``@``) to about 1e-12 relative;
* for the fused epilogue: exact integer arithmetic done by numpy, exact
  power-of-two scaling, and its special cases (K = 0, beta = 0, NaN).

``run_all`` runs every pin and returns the names of those that failed; run as
a script (``python tests/pins.py LIB``) it loads the oracle build at ``LIB``
and exits non-zero if any pin fails -- the mutation tests use that to show
that planted mistakes are caught.
"""
from __future__ import annotations

import os
import sys
from fractions import Fraction

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from register_lds_tiled_amd import workloads  # noqa: E402

GOLDEN = os.path.join(ROOT, "tests", "golden", "worked_example_output.txt")
U64 = 2.0 ** -53


def read_golden():
    K, vals = None, None
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *rest = line.split()
            if key == "K":
                K = int(rest[0])
            elif key == "C0_3":
                vals = rest
    assert K is not None and vals is not None and len(vals) == 4
    return K, vals


def exact_product(A: np.ndarray, B: np.ndarray):
    """Exact rational C = A.B of the stored float32 values."""
    M, K = A.shape
    N = B.shape[1]
    FA = [[Fraction(float(A[i, k])) for k in range(K)] for i in range(M)]
    FB = [[Fraction(float(B[k, j])) for j in range(N)] for k in range(K)]
    C = [[sum((FA[i][k] * FB[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    absum = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    return C, absum


def assert_within_sum_bound(C, A, B, exact, absum, what):
    """A double sum of K exact products is within (K-1) u sum|a b| of the
    exact value (u = 2^-53); allow a factor 1.01 for the first-order bound."""
    K = A.shape[1]
    M, N = C.shape
    for i in range(M):
        for j in range(N):
            err = abs(Fraction(float(C[i, j])) - exact[i][j])
            bound = Fraction(1.01 * max(K - 1, 0) * U64 * float(absum[i, j]))
            assert err <= bound, f"{what}: C[{i},{j}]={C[i, j]!r} off exact by {float(err)}"


# ----------------------------------------------------------------------------

def pin_printed_worked_example(o):
    """fp32 fused sequential micro-GEMM reproduces every printed digit of the
    first page's output ("Micro Kernel 입문하기", teach-meaning.tistory.com/1544,
    section "출력 결과")."""
    K, printed = read_golden()
    A, B = workloads.worked_example(K)
    C = o.micro4x4_seq_fma_f32(A, B)
    got = ["%f" % float(v) for v in C[0, :4]]
    assert got == printed, f"micro-GEMM printed {got}, page prints {printed}"


def pin_worked_example_f64(o):
    """fp64 oracle on the worked example: within the double-sum bound of the
    exact rational result, equal to 0.02*S (S the integer pattern sum) up to
    the fp32 rounding of 0.1f/0.2f, and within 3e-4 of the printed fp32
    values (fp32 accumulation on the page's device)."""
    K, printed = read_golden()
    A, B = workloads.worked_example(K)
    C = o.sgemm_ref_f64(A, B)
    exact, absum = exact_product(A, B)
    assert_within_sum_bound(C, A, B, exact, absum, "worked example")
    for r in range(4):
        for j in range(4):
            S = sum(((r * K + k) % 7) * ((4 * k + j) % 5) for k in range(K))
            assert abs(C[r, j] - 0.02 * S) <= 1e-5, (r, j, C[r, j], 0.02 * S)
    for j in range(4):
        assert abs(C[0, j] - float(printed[j])) <= 3e-4, (j, C[0, j], printed[j])


def pin_tiny_exact(o, seeds=range(40)):
    """Random tiny shapes (M, N, K in 1..9) against exact rational sums,
    through tight and padded leading dimensions."""
    for s in seeds:
        rng = np.random.Generator(np.random.PCG64(7000 + s))
        M, N, K = (int(x) for x in rng.integers(1, 10, 3))
        A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
        exact, absum = exact_product(A, B)
        C = o.sgemm_ref_f64(A, B)
        assert_within_sum_bound(C, A, B, exact, absum, f"tiny {M}x{N}x{K}")
        # same matrices embedded in wider buffers (lda > K, ldb > N)
        Aw = np.zeros((M, K + 5), np.float32); Aw[:, 2:2 + K] = A
        Bw = np.zeros((K, N + 3), np.float32); Bw[:, 1:1 + N] = B
        Cw = o.sgemm_ref_f64(Aw[:, 2:2 + K], Bw[:, 1:1 + N])
        assert np.array_equal(Cw, C), "padded leading dimensions change the result"
        # entries function, every (i, j)
        ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        E = o.sgemm_ref_f64_entries(A, B, ii.ravel(), jj.ravel())
        assert np.array_equal(E.reshape(M, N), C), "entries differ from full product"


def pin_integer_exact(o):
    """Integer-valued inputs: every partial sum is an exactly representable
    integer, so the result must equal the exact int64 product bit for bit."""
    shapes = [(1, 1, 1), (3, 5, 7), (37, 53, 129), (64, 17, 1000), (5, 130, 3)]
    for t, (M, N, K) in enumerate(shapes):
        A, B = workloads.integer_inputs(M, N, K, seed=500 + t)
        ref = A.astype(np.int64) @ B.astype(np.int64)
        C = o.sgemm_ref_f64(A, B)
        assert np.array_equal(C, ref.astype(np.float64)), f"integer product wrong at {M}x{N}x{K}"


def pin_invariants(o):
    rng = np.random.Generator(np.random.PCG64(99))
    M, N, K = 23, 31, 19
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    assert np.array_equal(o.sgemm_ref_f64(A, np.eye(K, dtype=np.float32)), A.astype(np.float64))
    assert np.array_equal(o.sgemm_ref_f64(np.eye(K, dtype=np.float32), B), B.astype(np.float64))
    assert np.array_equal(o.sgemm_ref_f64(A, np.zeros((K, N), np.float32)), np.zeros((M, N)))
    ones = o.sgemm_ref_f64(np.ones((M, K), np.float32), np.ones((K, N), np.float32))
    assert np.array_equal(ones, np.full((M, N), float(K)))
    C = o.sgemm_ref_f64(A, B)
    Ct = o.sgemm_ref_f64(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(C.T, Ct), "(A.B)^T != B^T.A^T"
    # K = 0 is the empty sum
    assert np.array_equal(o.sgemm_ref_f64(np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32)),
                          np.zeros((3, 4)))


def pin_library_f64(o, shape=(100, 150, 77), seed=1004):
    M, N, K = shape
    A, B = workloads.random_inputs(M, N, K, seed)
    C = o.sgemm_ref_f64(A, B)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    err = np.max(np.abs(C - ref))
    assert err <= 1e-12 * np.max(np.abs(ref)), f"oracle vs float64 library: {err}"


def relu_np(x):
    """ReLU as the epilogue defines it: negatives to zero, NaN kept."""
    return np.where(x < 0, np.zeros_like(x), x)


def pin_epilogue(o):
    """The fused epilogue act(alpha*S + beta*C + bias[j]):
    * with alpha=1, beta=0, no bias, identity it is the plain product, bit
      for bit;
    * on integer-valued inputs with integer alpha, beta and bias it equals
      the exact int64 computation (and ReLU of it) done by numpy, on a square
      and on a non-square shape;
    * power-of-two alpha scales the result exactly;
    * K = 0 leaves act(beta*C + bias); beta = 0 never reads C (NaN there is
      ignored); ReLU keeps NaN;
    * the entries form agrees with the whole-matrix form everywhere."""
    rng = np.random.Generator(np.random.PCG64(31337))
    M, N, K = 29, 37, 53
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    assert np.array_equal(o.sgemm_ex_ref_f64(A, B), o.sgemm_ref_f64(A, B))
    assert np.array_equal(o.sgemm_ex_ref_f64(A, B, alpha=4.0), 4.0 * o.sgemm_ref_f64(A, B))
    cases = [(31, 31, 1, -2, 1), (M, N, 1, 0, 0), (M, N, 2, 0, 1), (M, N, -3, 1, 0),
             (M, N, 1, -2, 1), (M, N, 0, 5, 1)]
    for t, (m, n, alpha, beta, act) in enumerate(cases):
        Ai, Bi = workloads.integer_inputs(m, n, K, seed=800 + t)
        Ci = rng.integers(-20, 21, (m, n)).astype(np.float32)
        bias = rng.integers(-30, 31, n).astype(np.float32)
        exact = (alpha * (Ai.astype(np.int64) @ Bi.astype(np.int64)) + beta * Ci.astype(np.int64)
                 + bias.astype(np.int64)[None, :])
        if act:
            exact = relu_np(exact)
        got = o.sgemm_ex_ref_f64(Ai, Bi, Ci, alpha, beta, bias, act)
        assert np.array_equal(got, exact.astype(np.float64)), f"epilogue case {t}"
        r, c = np.divmod(np.arange(m * n), n)
        ent = o.sgemm_ex_ref_f64_entries(Ai, Bi, r, c, Ci, alpha, beta, bias, act)
        assert np.array_equal(ent, got.ravel()), f"epilogue entries case {t}"
    Cn = np.full((M, N), np.nan, np.float32)
    assert np.all(np.isfinite(o.sgemm_ex_ref_f64(A, B, Cn, 1.0, 0.0)))
    assert np.all(np.isfinite(o.sgemm_ex_ref_f64_entries(A, B, [0, M - 1], [N - 1, 0], Cn)))
    C0 = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    bias = rng.uniform(-1, 1, N).astype(np.float32)
    k0 = o.sgemm_ex_ref_f64(np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32),
                            C0, 1.0, 0.5, bias, 1)
    ref = relu_np(0.5 * C0.astype(np.float64) + bias.astype(np.float64)[None, :])
    assert np.array_equal(k0, ref)
    An = A.copy()
    An[5, 3] = np.nan
    out = o.sgemm_ex_ref_f64(An, B, act=1)
    assert np.all(np.isnan(out[5])) and np.all(np.isfinite(np.delete(out, 5, axis=0)))


def pin_lowp(o):
    """The 16-bit path:
    * decoding: every one of the 65536 bit patterns equals numpy's IEEE
      binary16 value, and the binary32 with the same upper half for
      bfloat16 (NaN for NaN); named values (1, -2, 65504, 2^-24, 2^-14, Inf;
      bf16 1, -2, Inf, the smallest subnormal 2^-133) exactly;
    * the product: on integer-valued inputs (exact in both formats) it equals
      numpy's exact int64 product, for both formats, square and non-square;
      on random inputs it equals the float32 oracle on the decoded values bit
      for bit (the same sum over the same values); K = 0 gives zeros."""
    bits = np.arange(65536, dtype=np.uint16)
    ref16 = bits.view(np.float16).astype(np.float32)
    got = o.decode16_f32(bits, "f16")
    fin = ~np.isnan(ref16)
    assert np.array_equal(np.isnan(got), ~fin)
    assert np.array_equal(got[fin].view(np.uint32), ref16[fin].view(np.uint32))
    refb = (bits.astype(np.uint32) << 16).view(np.float32)
    got = o.decode16_f32(bits, "bf16")
    fin = ~np.isnan(refb)
    assert np.array_equal(np.isnan(got), ~fin)
    assert np.array_equal(got[fin].view(np.uint32), refb[fin].view(np.uint32))
    named16 = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24,
               0x0400: 2.0 ** -14, 0x7C00: np.inf, 0xFC00: -np.inf, 0x8000: -0.0}
    namedb = {0x3F80: 1.0, 0xC000: -2.0, 0x7F80: np.inf, 0x0001: 2.0 ** -133, 0x4049: 3.140625}
    for fmt, named in (("f16", named16), ("bf16", namedb)):
        keys = np.array(list(named), dtype=np.uint16)
        vals = o.decode16_f32(keys, fmt).astype(np.float64)
        assert np.array_equal(vals, np.array(list(named.values()))), fmt
    assert np.isnan(o.decode16_f32(np.array([0x7E00], np.uint16), "f16")[0])
    for fmt in ("bf16", "f16"):
        for t, (M, N, K) in enumerate([(31, 31, 40), (17, 45, 23)]):
            Ai, Bi = workloads.integer_inputs(M, N, K, seed=900 + t)
            A16, B16 = workloads.lowp_inputs(M, N, K, seed=900 + t, fmt=fmt, integer=True)
            exact = Ai.astype(np.int64) @ Bi.astype(np.int64)
            assert np.array_equal(o.gemm_lowp_ref_f64(A16, B16, fmt), exact.astype(np.float64))
        A16, B16 = workloads.lowp_inputs(29, 37, 61, seed=77, fmt=fmt)
        dec = o.sgemm_ref_f64(o.decode16_f32(A16, fmt), o.decode16_f32(B16, fmt))
        assert np.array_equal(o.gemm_lowp_ref_f64(A16, B16, fmt), dec)
        Z = o.gemm_lowp_ref_f64(np.zeros((5, 0), np.uint16), np.zeros((0, 7), np.uint16), fmt)
        assert Z.shape == (5, 7) and not Z.any()


PINS = [pin_printed_worked_example, pin_worked_example_f64, pin_tiny_exact,
        pin_integer_exact, pin_invariants, pin_library_f64, pin_epilogue, pin_lowp]


def run_all(o):
    failed = []
    for pin in PINS:
        try:
            pin(o)
        except AssertionError as e:
            failed.append(f"{pin.__name__}: {e}")
    return failed


if __name__ == "__main__":
    import oracle
    lib = oracle.OracleLib(sys.argv[1])
    bad = run_all(lib)
    for b in bad:
        print("FAIL", b)
    sys.exit(1 if bad else 0)
