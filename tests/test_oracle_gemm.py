"""Pins for the oracle's GEMM references (binary64, naive binary32, comp model).

Independent references: exact rational arithmetic (fractions) on small shapes,
numpy's float64 matmul (a library routine) for layout and indexing, cases whose
partial sums are exact, and a hand-worked three-term case fixing the order.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _mixed_f32(g, shape):
    """binary32 values with mixed exponents, signed zeros and subnormals."""
    x = g.standard_normal(size=shape).astype(np.float32)
    x *= np.float32(2.0) ** g.integers(-20, 20, size=shape).astype(np.float32)
    flat = x.reshape(-1)
    n = flat.size
    idx = g.choice(n, size=max(1, n // 8), replace=False)
    flat[idx[: len(idx) // 3]] = 0.0
    flat[idx[len(idx) // 3: 2 * len(idx) // 3]] = -0.0
    sub = idx[2 * len(idx) // 3:]
    flat[sub] = (g.integers(1, 1 << 20, size=sub.size).astype(np.uint32)).view(np.float32)
    return x


def _exact(A, W, layout):
    M, K = A.shape
    B = W.T if layout == "nk" else W
    N = B.shape[1]
    C = [[Fraction(0)] * N for _ in range(M)]
    S = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            sa = Fraction(0)
            for k in range(K):
                p = Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
                s += p
                sa += abs(p)
            C[i][j] = s
            S[i][j] = sa
    return C, S


@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (6, 4, 8), (2, 7, 3)])
def test_gemm_f64_and_naive_against_exact_rationals(layout, shape):
    M, N, K = shape
    g = np.random.Generator(np.random.PCG64(M * 100 + N * 10 + K))
    A = _mixed_f32(g, (M, K))
    W = _mixed_f32(g, (N, K) if layout == "nk" else (K, N))
    C64 = oracle.gemm_f64(A, W, layout)
    C32 = oracle.gemm_f32_naive(A, W, layout)
    exact, absum = _exact(A, W, layout)
    u64, u32 = 2.0 ** -53, 2.0 ** -24
    for i in range(M):
        for j in range(N):
            err64 = abs(Fraction(float(C64[i, j])) - exact[i][j])
            err32 = abs(Fraction(float(C32[i, j])) - exact[i][j])
            # standard recursive-summation bound gamma_K = K u / (1 - K u) on sum |a b|
            assert err64 <= Fraction(K * u64 / (1 - K * u64)) * absum[i][j]
            assert err32 <= Fraction((K + 1) * u32 / (1 - (K + 1) * u32)) * absum[i][j] + Fraction(2.0 ** -149)


def test_gemm_layouts_and_indexing_against_numpy_matmul():
    g = np.random.Generator(np.random.PCG64(5))
    A = g.standard_normal((13, 37)).astype(np.float32)
    W = g.standard_normal((11, 37)).astype(np.float32)
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    bound = 37 * 2.0 ** -52 * (np.abs(A).astype(np.float64) @ np.abs(W).astype(np.float64).T)
    assert np.all(np.abs(oracle.gemm_f64(A, W, "nk") - ref) <= bound)
    assert np.all(np.abs(oracle.gemm_f64(A, np.ascontiguousarray(W.T), "kn") - ref) <= bound)
    rows = np.array([12, 0, 5])
    assert np.array_equal(oracle.gemm_f64_rows(A, W, rows), oracle.gemm_f64(A, W)[rows])
    assert np.array_equal(oracle.gemm_f32_naive_rows(A, W, rows), oracle.gemm_f32_naive(A, W)[rows])


def test_naive_equals_f64_when_partial_sums_are_exact():
    g = np.random.Generator(np.random.PCG64(9))
    A = g.integers(-64, 65, size=(9, 200)).astype(np.float32)
    W = g.integers(-64, 65, size=(17, 200)).astype(np.float32)
    C64 = oracle.gemm_f64(A, W)
    C32 = oracle.gemm_f32_naive(A, W)
    assert np.array_equal(C32.astype(np.float64), C64)
    assert np.array_equal(C64, A.astype(np.int64) @ W.astype(np.int64).T)


def test_naive_f32_sums_sequentially_without_fma():
    # a = (1, 1, 1), b = (2^24, 1, 1).  In order: 2^24 + 1 is a tie that rounds to 2^24
    # (even), twice, so the naive sum is exactly 2^24.  Any other order (or a wider
    # accumulator) gives 2^24 + 2.
    A = np.array([[1.0, 1.0, 1.0]], np.float32)
    W = np.array([[2.0 ** 24, 1.0, 1.0]], np.float32)
    assert oracle.gemm_f32_naive(A, W)[0, 0] == np.float32(2.0 ** 24)
    assert oracle.gemm_f64(A, W)[0, 0] == 2.0 ** 24 + 2
    # no fused multiply-add: (1 + 2^-12)^2 = 1 + 2^-11 + 2^-24, and the product rounds to 1 + 2^-11
    # before the add of -(1 + 2^-11), so the result is exactly 0; an FMA would leave 2^-24.
    a = np.float32(1 + 2.0 ** -12)
    A = np.array([[a, np.float32(1 + 2.0 ** -11)]], np.float32)
    W = np.array([[a, np.float32(-1.0)]], np.float32)
    assert oracle.gemm_f32_naive(A, W)[0, 0] == 0.0


def test_comp_model_exact_on_binary16_operands_and_bounded_otherwise():
    g = np.random.Generator(np.random.PCG64(12))
    A = (g.integers(-8, 9, size=(16, 256)) / 8.0).astype(np.float32)
    W = (g.integers(-8, 9, size=(32, 256)) / 8.0).astype(np.float32)
    assert np.array_equal(oracle.gemm_comp_model(A, W), oracle.gemm_f64(A, W))
    A = g.standard_normal((8, 300)).astype(np.float32)
    W = (0.02 * g.standard_normal((9, 300))).astype(np.float32)
    err = np.abs(oracle.gemm_comp_model(A, W) - oracle.gemm_f64(A, W))
    absum = np.abs(A).astype(np.float64) @ np.abs(W).astype(np.float64).T
    # each operand carries relative error <= 2^-22 (+ 2^-35 absolute): products <= ~2^-21
    assert np.all(err <= (2.0 ** -21 + 1e-12) * absum + 300 * 2.0 ** -35)


def test_plain_f16_gemm_rounds_operands_then_multiplies_exactly():
    """One-product (plain FP16) reference: on binary16 operands it is the binary64
    product itself; on other operands it equals the binary64 product of the operands
    rounded by numpy's float16 cast (an independent round-to-nearest-even
    conversion), and it differs from the unrounded product by at most the operand
    rounding (relative 2^-11 per operand)."""
    g = np.random.Generator(np.random.PCG64(13))
    A = (g.integers(-64, 65, size=(8, 96)) / 16.0).astype(np.float32)
    W = (g.integers(-64, 65, size=(12, 96)) / 64.0).astype(np.float32)
    rows = np.arange(8)
    c64, c32 = oracle.gemm_f16_plain_rows(A, W, rows)
    assert np.array_equal(c64, oracle.gemm_f64(A, W))
    A = g.standard_normal((6, 200)).astype(np.float32)
    W = (0.02 * g.standard_normal((10, 200))).astype(np.float32)
    rows = np.arange(6)
    c64, c32 = oracle.gemm_f16_plain_rows(A, W, rows)
    ref = A.astype(np.float16).astype(np.float64) @ W.astype(np.float16).astype(np.float64).T
    assert np.allclose(c64, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    absum = np.abs(A).astype(np.float64) @ np.abs(W).astype(np.float64).T
    assert np.all(np.abs(c64 - oracle.gemm_f64(A, W)) <= (2 * 2.0 ** -11 + 2.0 ** -22) * absum + 1e-9)
    assert c32.dtype == np.float32 and np.all(np.abs(c32 - c64) <= 1e-4 * absum + 1e-9)
    for layout in ("nk", "kn"):
        Wl = W if layout == "nk" else np.ascontiguousarray(W.T)
        assert np.array_equal(oracle.gemm_f16_plain_rows(A, Wl, rows, layout)[0], c64)
