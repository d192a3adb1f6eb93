"""Pins for the oracle's INT16 quantizer.

The method (HEAL paper, section 3, "Mitigating QKV Truncation Error via INT16
Quantization"): Q_INT16(X) = Round((2^15 - 1) X / max|X|), step
Delta = M / (2^15 - 1), error uniform in [-Delta/2, Delta/2] (MSE Delta^2/12),
and E[MSE_FP16] / E[MSE_INT16] > 256 sigma^2 / M^2.

Independent references: hand-derived tie rows (golden), exact rational
rounding of 32767 x / M away from ties, closed-form error bounds of the
binary32 op order, and the uniform-error statistics the pages state.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import heal_workloads as W
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _nearest_f32(fr: Fraction) -> np.float32:
    """The binary32 value nearest to a positive rational (by exhaustive neighbour check)."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: abs(Fraction(float(c)) - fr))


def test_quant_golden_ties():
    with open(os.path.join(GOLDEN, "quant_ties.json")) as f:
        g = json.load(f)
    for row in g["rows"]:
        x = np.array([row["x"]], np.float32)
        codes, scales = oracle.quant_i16(x)
        assert codes[0].tolist() == row["codes"], row["derivation"]
        num, den = row["scale"].split("/")
        want = Fraction(int(num), int(den))
        want32 = np.float32(0) if want == 0 else _nearest_f32(want)
        assert scales[0] == want32


@pytest.fixture(scope="module")
def qdata():
    Q, K, V = W.qkv(tokens=512, Hq=8, Hkv=2, D=128, seed=4242)
    X = np.concatenate([Q.reshape(-1, 128), K.reshape(-1, 128), V.reshape(-1, 128)])
    codes, scales = oracle.quant_i16(X)
    return X, codes, scales


def test_quant_range_absmax_and_symmetry(qdata):
    X, codes, scales = qdata
    assert codes.min() >= -32767 and codes.max() <= 32767
    idx = np.argmax(np.abs(X), axis=1)
    top = codes[np.arange(X.shape[0]), idx]
    assert np.array_equal(np.abs(top), np.full(X.shape[0], 32767))
    assert np.array_equal(np.sign(top), np.sign(X[np.arange(X.shape[0]), idx]).astype(np.int16))
    c2, s2 = oracle.quant_i16(-X)
    assert np.array_equal(c2, -codes)
    assert np.array_equal(s2, scales)


def test_quant_zero_row_and_single_element():
    codes, scales = oracle.quant_i16(np.zeros((3, 64), np.float32))
    assert np.all(codes == 0) and np.all(scales == 0)
    codes, scales = oracle.quant_i16(np.array([[-3.0]], np.float32))
    assert codes[0, 0] == -32767 and scales[0] == np.float32(3.0) / np.float32(32767.0)


def test_quant_matches_exact_rational_rounding_away_from_ties(qdata):
    X, codes, scales = qdata
    M = np.max(np.abs(X), axis=1).astype(np.float64)
    v = 32767.0 * X.astype(np.float64) / M[:, None]      # ideal scaled value (error ~1e-12)
    # the binary32 op order t = fl(32767 x), u = fl(t / M) moves v by at most |v| 2^-23 <= 2^-8
    assert np.all(np.abs(codes - v) <= 0.5 + 2.0 ** -8)
    frac = np.abs(v - np.floor(v) - 0.5)                 # distance to the nearest half-integer
    clear = frac > 2.0 ** -8 + 1e-9
    ideal = np.rint(v)                                   # round half even, exact away from ties
    assert np.array_equal(codes[clear], ideal[clear].astype(np.int16))
    assert clear.mean() > 0.99
    # exact check with rationals on a sample, including the near-tie elements
    g = np.random.Generator(np.random.PCG64(1))
    pick = list(zip(*np.nonzero(~clear)))[:200] + [tuple(p) for p in g.integers(0, [X.shape[0], 128], size=(300, 2))]
    for r, d in pick:
        ex = Fraction(32767) * Fraction(float(X[r, d])) / Fraction(float(M[r]))
        assert abs(Fraction(int(codes[r, d])) - ex) <= Fraction(1, 2) + Fraction(1, 256)


def test_quant_scale_is_rounded_max_over_32767(qdata):
    X, codes, scales = qdata
    M = np.max(np.abs(X), axis=1)
    for r in range(0, X.shape[0], 97):
        assert scales[r] == _nearest_f32(Fraction(float(M[r])) / 32767)


def test_quant_dequant_error_bounds(qdata):
    X, codes, scales = qdata
    xhat = oracle.dequant_f32(codes, scales).astype(np.float64)
    s = scales.astype(np.float64)[:, None]
    # the pages' |x - dequant| <= s/2, widened by the three binary32 roundings involved
    assert np.all(np.abs(X - xhat) <= (s / 2) * (1 + 2.0 ** -6))


def test_quant_mse_is_uniform_error_delta_sq_over_12(qdata):
    X, codes, scales = qdata
    M = np.max(np.abs(X), axis=1).astype(np.float64)
    delta = M / 32767.0
    err = X.astype(np.float64) - codes.astype(np.float64) * delta[:, None]
    mask = np.abs(X) < M[:, None]                        # the absmax element has no error
    ratio = np.mean((err[mask] / np.broadcast_to(delta[:, None], X.shape)[mask]) ** 2) / (1.0 / 12.0)
    assert abs(ratio - 1.0) < 0.02


def test_quant_mse_ratio_bound_against_fp16(qdata):
    X, codes, scales = qdata
    x64 = X.astype(np.float64)
    M = np.max(np.abs(X), axis=1).astype(np.float64)
    sigma2 = np.mean(x64 ** 2, axis=1)
    mse_int16 = np.mean((x64 - codes * (M / 32767.0)[:, None]) ** 2, axis=1)
    mse_fp16 = np.mean((x64 - X.astype(np.float16).astype(np.float64)) ** 2, axis=1)
    holds = mse_fp16 / mse_int16 > 256.0 * sigma2 / M ** 2
    assert holds.mean() >= 0.999
