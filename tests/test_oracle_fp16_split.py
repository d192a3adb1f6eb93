"""Pins for the oracle's binary16 conversion, operand split and dual-FP16 dequant.

Independent references used here:
  * numpy's float32/float64 -> float16 conversion (IEEE round-to-nearest-even,
    subnormals kept): a library routine that the oracle does not call;
  * the closed-form split bound |x - (hi + lo/2^10)| <= 2^-22 |x| + 2^-35;
  * hand-derived golden cases (tests/golden/dual_fp16.json).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f16_np(x):
    with np.errstate(over="ignore"):
        return np.asarray(x).astype(np.float16).view(np.uint16)


def _stratified_f32(n_per_exp=20000, seed=7):
    g = np.random.Generator(np.random.PCG64(seed))
    parts = []
    # every binary32 exponent that reaches binary16 (and a margin beyond both ends)
    for e in range(-40, 18):
        mant = g.integers(0, 1 << 23, size=n_per_exp, dtype=np.uint32)
        bits = ((e + 127) << 23) | mant
        parts.append(np.asarray(bits, np.uint32))
    # binary32 values lying exactly on binary16 rounding ties (low 13 bits = 0x1000)
    mant = (g.integers(0, 1 << 10, size=50000, dtype=np.uint32) << 13) | 0x1000
    exps = g.integers(127 - 14, 127 + 16, size=50000, dtype=np.uint32)
    parts.append((exps << 23) | mant)
    bits = np.concatenate(parts)
    x = bits.view(np.float32)
    return np.concatenate([x, -x])


def test_f16_conversion_matches_numpy_stratified():
    x = _stratified_f32()
    assert np.array_equal(oracle.f32_to_f16_bits(x), _f16_np(x))


def test_f16_conversion_special_values():
    x = np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 1e30,
                  2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -11),
                  1e-45, 3.0e-8], np.float32)
    assert np.array_equal(oracle.f32_to_f16_bits(x), _f16_np(x))
    assert oracle.f32_to_f16_bits(np.array([np.nan], np.float32))[0] & 0x7C00 == 0x7C00


def test_f16_decode_all_encodings():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = oracle.f16_bits_to_f64(h)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_split_exact_for_binary16_values():
    # every finite binary16 value is carried by hi alone, with lo == +-0
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16)
    keep = np.isfinite(v)
    x = v[keep].astype(np.float32)
    hi, lo = oracle.split_f16(x)
    assert np.array_equal(hi, h[keep])
    assert np.all((lo & 0x7FFF) == 0)


def test_split_closed_form_bound_and_residual_rounding():
    x = _stratified_f32(n_per_exp=10000, seed=11)
    x = x[np.abs(x) < 65504]
    hi, lo = oracle.split_f16(x)
    hv = hi.view(np.float16).astype(np.float64)
    lv = lo.view(np.float16).astype(np.float64)
    x64 = x.astype(np.float64)
    err = np.abs(x64 - (hv + lv / 1024.0))
    bound = 2.0 ** -22 * np.abs(x64) + 2.0 ** -35
    assert np.all(err <= bound)
    # hi is the binary16 rounding of x, lo the binary16 rounding of the exact residual * 2^10
    assert np.array_equal(hi, _f16_np(x))
    assert np.array_equal(lo, _f16_np((x64 - hv) * 1024.0))


def test_split_golden():
    with open(os.path.join(GOLDEN, "dual_fp16.json")) as f:
        g = json.load(f)
    for case in g["fp32_values"]:
        x = np.array([int(case["x"], 16)], np.uint32).view(np.float32)
        hi, lo = oracle.split_f16(x)
        assert hi[0] == int(case["hi"], 16), case
        assert lo[0] == int(case["lo"], 16), case


def test_dequant_f16x2_golden():
    with open(os.path.join(GOLDEN, "dual_fp16.json")) as f:
        g = json.load(f)
    codes = np.array([[c["q"] for c in g["int16_codes"]]], np.int16)
    hi, lo = oracle.dequant_f16x2(codes)
    for i, c in enumerate(g["int16_codes"]):
        assert hi[0, i] == int(c["hi"], 16), c
        assert lo[0, i] == int(c["lo"], 16), c


def test_dequant_f16x2_exhaustive_exact():
    # every int16 code is carried exactly by the dual-FP16 pair (the "20 bits" of the
    # dual-FP16 pairing hold the 16-bit code without loss)
    q = np.arange(-32768, 32768, dtype=np.int32).astype(np.int16).reshape(1, -1)
    hi, lo = oracle.dequant_f16x2(q)
    hv = hi.view(np.float16).astype(np.float64)
    lv = lo.view(np.float16).astype(np.float64)
    qv = q.astype(np.float64)
    assert np.array_equal(hv + lv / 1024.0, qv)
    assert np.max(np.abs(qv - hv)) <= 8
    assert np.max(np.abs(lv)) <= 8192
    assert np.array_equal(hi, _f16_np(q.astype(np.float32)))


def test_dequant_f32_single_rounding():
    g = np.random.Generator(np.random.PCG64(3))
    q = g.integers(-32767, 32768, size=(300, 128)).astype(np.int16)
    s = (np.exp(g.uniform(-12, 2, size=300)) / 32767).astype(np.float32)
    got = oracle.dequant_f32(q, s)
    # q*s is exact in binary64 (15 + 24 bits), so one rounding to binary32 is the correct result
    ref = (q.astype(np.float64) * s[:, None].astype(np.float64)).astype(np.float32)
    assert np.array_equal(got, ref)
