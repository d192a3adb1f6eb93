"""The seeded input recipe (the synthetic stand-ins for the pages' workloads):
shapes, dtype, determinism, outlier-channel counts and gains, per-head gain
ranges.  Host only."""
import numpy as np

import heal_workloads as WL


def _outlier_cols(A, thresh):
    return np.flatnonzero(np.abs(A).max(axis=0) > thresh)


def test_same_seed_same_inputs_and_float32():
    a1, w1 = WL.decode_gemm(8, 4096, 1024, seed=2000)
    a2, w2 = WL.decode_gemm(8, 4096, 1024, seed=2000)
    assert a1.dtype == np.float32 and w1.dtype == np.float32
    assert a1.shape == (8, 4096) and w1.shape == (1024, 4096)
    assert np.array_equal(a1, a2) and np.array_equal(w1, w2)
    a3, _ = WL.decode_gemm(8, 4096, 1024, seed=2001)
    assert not np.array_equal(a1, a3)


def test_decode_activation_has_round_0p001K_channels_times_50():
    for K in (4096, 14336):
        A, W = WL.decode_gemm(64, K, 16, seed=7)
        cols = _outlier_cols(A, 10.0)   # N(0,1) over 64 rows stays far below 10; x50 goes well above
        assert len(cols) == round(0.001 * K)
        rest = np.delete(A, cols, axis=1)
        assert abs(rest.std() - 1.0) < 0.02 and abs(A[:, cols].std() / 50.0 - 1.0) < 0.2
        assert abs(W.std() - 0.02) < 0.002


def test_prefill_activation_has_four_channels_times_1000():
    A, _ = WL.prefill_gemm(256, 4096, 8, seed=3000)
    cols = _outlier_cols(A, 100.0)
    assert len(cols) == 4
    assert abs(np.abs(A[:, cols]).max() / 1000.0) > 2.0   # |x| reaches thousands


def test_overflow_activation_passes_fp16_range():
    A, _ = WL.overflow_gemm(16, 4096, 8, seed=11)
    cols = _outlier_cols(A, 1e3)
    assert len(cols) == round(0.005 * 4096)
    assert np.abs(A).max() > 65504.0


def test_qkv_gains_are_per_head_and_within_0p1_to_30():
    q, k, v = WL.qkv(4096, 8, 2, 128, seed=4000)
    assert q.shape == (4096, 8, 128) and k.shape == (4096, 2, 128) and v.shape == (4096, 2, 128)
    for X in (q, k, v):
        s = X.std(axis=(0, 2))                 # one factor per head, shared by all tokens
        assert np.all(s > 0.1 * 0.95) and np.all(s < 30.0 * 1.05)
        half = X.shape[0] // 2
        assert np.allclose(X[:half].std(axis=(0, 2)), X[half:].std(axis=(0, 2)), rtol=0.05)


def test_attention_inputs_are_standard_normal():
    q, k, v = WL.attention_fp32(2, 512, 8, 2, 128, seed=5000)
    assert q.shape == (2, 8, 128) and k.shape == (2, 512, 2, 128)
    for X in (k, v):
        assert abs(X.mean()) < 0.01 and abs(X.std() - 1.0) < 0.01
