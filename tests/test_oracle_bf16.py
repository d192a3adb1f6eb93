"""Pins of the oracle's BF16 three-way split (the precision mode of the GEMM).

round_bf16 is checked against torch's own bfloat16 conversion (a library
routine, round to nearest even) and hand-derived ties; the split against its
exactness and magnitude invariants; the six-product model against exact
products of bf16-representable operands and the size of the dropped terms.
"""
import numpy as np
import pytest
import torch

import heal_workloads as WL
import oracle


def _torch_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_torch_conversion():
    g = WL.rng(1)
    x = (g.standard_normal(200000) * np.exp2(g.integers(-140, 128, 200000))).astype(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(oracle.round_bf16(x), _torch_bf16(x))


def test_round_bf16_all_bf16_values_are_fixed_points():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals)]
    assert np.array_equal(oracle.round_bf16(vals), vals.astype(np.float64))


@pytest.mark.parametrize("x,expected", [
    (1 + 2.0 ** -8, 1.0),                          # tie, even neighbour below
    (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),            # tie, even neighbour above
    (-(1 + 2.0 ** -8), -1.0),
    (1 + 2.0 ** -8 + 2.0 ** -20, 1 + 2.0 ** -7),   # just above the tie
    (2.0 ** 128 - 2.0 ** 120, 2.0 ** 128 - 2.0 ** 120),   # largest bf16
    (2.0 ** 128 - 2.0 ** 119, np.inf),             # tie past the largest: overflows
    (2.0 ** -133, 2.0 ** -133),                    # smallest subnormal
    (2.0 ** -134, 0.0),                            # tie with zero (even)
    (3 * 2.0 ** -134, 2.0 ** -132),                # subnormal tie, even neighbour above
    (0.0, 0.0),
])
def test_round_bf16_hand_values(x, expected):
    assert oracle.round_bf16(np.float64(x)) == expected


def test_split_bf16x3_is_exact_and_ordered():
    g = WL.rng(2)
    x = (g.standard_normal(100000) * np.exp2(g.integers(-90, 100, 100000))).astype(np.float32)
    b0, b1, b2 = oracle.split_bf16x3(x)
    x64 = x.astype(np.float64)
    assert np.array_equal(b0 + b1 + b2, x64)          # exact while the last part stays normal
    # near the bottom of the range the last part loses bits to bf16 subnormals
    t = np.float32(-4.074164e-34)
    assert sum(oracle.split_bf16x3(t)) != np.float64(t)
    for b in (b0, b1, b2):
        assert np.array_equal(oracle.round_bf16(b), b)
    _, e0 = np.frexp(b0)
    assert np.all(np.abs(b1) <= np.ldexp(1.0, e0 - 9))   # half a bf16 ulp of b0
    _, e1 = np.frexp(np.where(b1 == 0, 1.0, b1))
    assert np.all(np.abs(b2) <= np.where(b1 == 0, 0.0, np.ldexp(1.0, e1 - 9)))


def test_split_bf16x3_parts_of_bf16_values():
    x = np.array([1.0, -3.5, 2.0 ** 100, 1.5 * 2.0 ** -120], np.float32)
    b0, b1, b2 = oracle.split_bf16x3(x)
    assert np.array_equal(b0, x.astype(np.float64)) and not b1.any() and not b2.any()


@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_bf16x3_model_exact_on_bf16_operands(layout):
    """bf16-representable small integers: the model is the exact product."""
    g = WL.rng(3)
    A = g.integers(-120, 121, (9, 40)).astype(np.float32)
    W = g.integers(-120, 121, (13, 40) if layout == "nk" else (40, 13)).astype(np.float32)
    B = W.T if layout == "nk" else W
    exact = A.astype(np.int64) @ B.astype(np.int64)
    assert np.array_equal(oracle.gemm_bf16x3_model(A, W, layout), exact.astype(np.float64))


def test_bf16x3_model_error_is_the_dropped_terms():
    """Against the binary64 product the model is off by the three dropped
    terms only: normwise at most 2^-23 (|a1 b2| + |a2 b1| <= 2 * 2^-8 * 2^-16,
    |a2 b2| far below), while dropping any kept term costs ~2^-9."""
    g = WL.rng(4)
    A = WL.normal(g, (20, 300))
    W = WL.normal(g, (30, 300), std=0.05)
    from metrics import gemm_normwise_error
    C = oracle.gemm_bf16x3_model(A, W)
    C64 = oracle.gemm_f64(A, W)
    assert gemm_normwise_error(C, C64, A, W) <= 2.0 ** -23
    a0, a1, a2 = oracle.split_bf16x3(A)
    b0, b1, b2 = oracle.split_bf16x3(W)
    wrong = C - a1 @ b0.T        # a mistake of the kind a pin must catch
    assert gemm_normwise_error(wrong, C64, A, W) > 2.0 ** -12
