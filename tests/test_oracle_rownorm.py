"""Pins for the oracle's row normalization and the split of a normalized row.

Independent references used here:
  * the defining inequality 2^14 <= max|x| 2^e < 2^15, checked in binary64
    with numpy's ldexp (exact for these magnitudes);
  * numpy's float32 -> float16 conversion (round to nearest even, subnormals
    kept), which the oracle does not call;
  * the oracle's pages-form split (pinned in test_oracle_fp16_split.py): the
    residual of a normalized element equals its lo / 2^10 wherever that is a
    normal binary16;
  * exact binary64 products for the GEMM model, and its exact invariance
    under power-of-two scaling of a row.
"""
import numpy as np
import pytest

import heal_workloads as WL
import oracle


def _wide_rows(seed, rows=400, K=96):
    """Rows whose scales span binary32's range, subnormal rows included."""
    g = WL.rng(seed)
    scale = np.exp2(g.integers(-148, 120, size=rows)).astype(np.float64)
    X = (g.standard_normal((rows, K)) * scale[:, None])
    with np.errstate(over="ignore", under="ignore"):
        return X.astype(np.float32)


def test_row_exponent_defining_inequality():
    X = _wide_rows(1)
    e = oracle.row_exponent(X)
    m = np.abs(X.astype(np.float64)).max(axis=1)
    nz = m > 0
    y = np.ldexp(m[nz], e[nz].astype(np.int64))
    assert np.all(y >= 2.0 ** 14) and np.all(y < 2.0 ** 15)
    assert np.all(e[~nz] == 0)


@pytest.mark.parametrize("mx,want", [(2.0 ** 14, 0), (2.0 ** 15, -1), (1.0, 14), (2.0 ** 15 - 1, 0),
                                     (65504.0, -1), (2.0 ** -149, 163), (3.0e38, -113), (0.75, 15)])
def test_row_exponent_hand_cases(mx, want):
    x = np.array([[0.0, -mx, mx / 2]], np.float32)
    assert oracle.row_exponent(x)[0] == want


def test_row_exponent_zero_row_and_sign():
    x = np.zeros((2, 5), np.float32)
    x[1, 3] = -3.0
    assert list(oracle.row_exponent(x)) == [0, 13]


def test_split_rownorm_matches_numpy_binary16():
    X = _wide_rows(2)
    hi, res, e = oracle.split_rownorm(X)
    xs = np.ldexp(X.astype(np.float64), e[:, None].astype(np.int64)).astype(np.float32)
    h_np = xs.astype(np.float16)
    assert np.array_equal(hi, h_np.view(np.uint16))
    r_np = (xs - h_np.astype(np.float32)).astype(np.float16)
    assert np.array_equal(res, r_np.view(np.uint16))


def test_split_rownorm_residual_is_pages_lo_scaled():
    """Wherever the pages' lo part divided by 2^10 is a normal binary16, the
    residual is exactly that value."""
    X = _wide_rows(3)
    hi, res, e = oracle.split_rownorm(X)
    xs = np.ldexp(X.astype(np.float64), e[:, None].astype(np.int64)).astype(np.float32)
    hi2, lo2 = oracle.split_f16(xs)
    assert np.array_equal(hi, hi2)
    lo_v = oracle.f16_bits_to_f64(lo2) / 1024.0
    normal = np.abs(lo_v) >= 2.0 ** -14
    assert normal.mean() > 0.9   # the rest: zero residuals (rows with few bits) and tiny ones
    assert np.array_equal(oracle.f16_bits_to_f64(res)[normal], lo_v[normal])


def test_split_rownorm_reconstruction_bound_at_every_scale():
    """|x' - (hi + res)| <= 2^-22 |x'| + 2^-25 on normalized rows: the same
    relative accuracy whatever the row's scale, since |x'| >= 2^14 at the max."""
    X = _wide_rows(4)
    hi, res, e = oracle.split_rownorm(X)
    xs = np.ldexp(X.astype(np.float64), e[:, None].astype(np.int64)).astype(np.float32).astype(np.float64)
    rec = oracle.f16_bits_to_f64(hi) + oracle.f16_bits_to_f64(res)
    assert np.all(np.abs(xs - rec) <= 2.0 ** -22 * np.abs(xs) + 2.0 ** -25)
    assert np.all(np.abs(xs).max(axis=1)[np.abs(xs).max(axis=1) > 0] < 65504.0)


def test_rownorm_model_exact_on_binary16_operands():
    g = WL.rng(5)
    A = (g.integers(-8, 9, size=(7, 64)) / 8.0).astype(np.float32)
    W = (g.integers(-8, 9, size=(9, 64)) / 64.0).astype(np.float32)
    assert np.array_equal(oracle.gemm_rownorm_model(A, W), oracle.gemm_f64(A, W))
    assert np.array_equal(oracle.gemm_rownorm_model(A, W, norm_w=False), oracle.gemm_f64(A, W))


@pytest.mark.parametrize("j", [-90, -30, -7, 12, 60])
def test_rownorm_model_scale_invariant(j):
    """Scaling a row of A by 2^j scales that row of the model's product by 2^j,
    bit for bit (the normalized operands are the same)."""
    g = WL.rng(6)
    A = g.standard_normal((5, 200)).astype(np.float32)
    W = (g.standard_normal((11, 200)) * 0.02).astype(np.float32)
    A2 = np.ldexp(A, j).astype(np.float32)
    c1 = oracle.gemm_rownorm_model(A, W)
    c2 = oracle.gemm_rownorm_model(A2, W)
    assert np.array_equal(np.ldexp(c1, j), c2)


@pytest.mark.parametrize("sa", [1.0, 1e-3, 1e-8, 1e-30, 1e20])
def test_rownorm_model_within_representation_bound(sa):
    """Against the binary64 product, the model's normwise error stays at the
    split's representation level (three products, residuals of 11 bits) at
    every activation scale."""
    g = WL.rng(7)
    A = (g.standard_normal((6, 512)) * sa).astype(np.float32)
    W = (g.standard_normal((20, 512)) * 0.02).astype(np.float32)
    C = oracle.gemm_rownorm_model(A, W)
    C64 = oracle.gemm_f64(A, W)
    denom = np.linalg.norm(A.astype(np.float64), axis=1)[:, None] * np.linalg.norm(W.astype(np.float64), axis=1)[None]
    assert (np.abs(C - C64) / denom).max() < 2.0 ** -21


def test_rownorm_model_dropping_a_product_is_detected():
    """A model missing the A_res.B_hi product misses the binary64 product by far
    more than the representation bound (so the pin above would catch it)."""
    g = WL.rng(8)
    A = g.standard_normal((4, 256)).astype(np.float32)
    W = (g.standard_normal((8, 256)) * 0.02).astype(np.float32)
    ah, ar, ea = oracle.split_rownorm(A)
    bh, br, eb = oracle.split_rownorm(W)
    f = oracle.f16_bits_to_f64
    C = np.ldexp(f(ah) @ f(bh).T + f(ah) @ f(br).T, -(ea[:, None] + eb[None, :]).astype(np.int64))
    C64 = oracle.gemm_f64(A, W)
    denom = np.linalg.norm(A.astype(np.float64), axis=1)[:, None] * np.linalg.norm(W.astype(np.float64), axis=1)[None]
    assert (np.abs(C - C64) / denom).max() > 2.0 ** -16
