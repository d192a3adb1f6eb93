"""Pins for the oracle's INT16 decode attention.

Independent references: the one-token case (softmax of one score is 1, so the
output is the dequantized value row), equal scores (output is the mean), and
a high-precision mpmath evaluation on tiny shapes written from the definition
softmax(q K^T / sqrt(D)) V with grouped-query heads h -> h // (Hq / Hkv).
No attention value is printed on the pages: beyond these cases attention
parity is unpinned.
"""
import mpmath
import numpy as np
import pytest

import oracle


def _codes(g, shape):
    return g.integers(-32767, 32768, size=shape).astype(np.int16)


def _scales(g, shape):
    return (np.exp(g.uniform(-3, 1, size=shape)) / 32767).astype(np.float32)


def test_single_token_returns_value_row():
    g = np.random.Generator(np.random.PCG64(2))
    B, T, Hq, Hkv, D = 2, 1, 8, 2, 16
    q, qs = _codes(g, (B, Hq, D)), _scales(g, (B, Hq))
    k, ks = _codes(g, (B, T, Hkv, D)), _scales(g, (B, T, Hkv))
    v, vs = _codes(g, (B, T, Hkv, D)), _scales(g, (B, T, Hkv))
    o = oracle.attn_decode_f64(q, qs, k, ks, v, vs)
    for b in range(B):
        for h in range(Hq):
            want = v[b, 0, h // 4].astype(np.float64) * np.float64(vs[b, 0, h // 4])
            assert np.array_equal(o[b, h], want)


def test_equal_scores_give_mean_of_values():
    g = np.random.Generator(np.random.PCG64(3))
    B, T, Hq, Hkv, D = 1, 37, 4, 1, 8
    q, qs = _codes(g, (B, Hq, D)), _scales(g, (B, Hq))
    k = np.zeros((B, T, Hkv, D), np.int16)
    ks = _scales(g, (B, T, Hkv))
    v, vs = _codes(g, (B, T, Hkv, D)), _scales(g, (B, T, Hkv))
    o = oracle.attn_decode_f64(q, qs, k, ks, v, vs)
    vt = v.astype(np.float64) * vs[..., None].astype(np.float64)
    want = vt[0, :, 0, :].mean(axis=0)
    assert np.allclose(o[0], want[None, :], rtol=1e-13, atol=1e-16)


def _mp_attention(q, qs, k, ks, v, vs):
    mpmath.mp.dps = 40
    B, Hq, D = q.shape
    T, Hkv = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            qv = [mpmath.mpf(int(q[b, h, d])) * mpmath.mpf(float(qs[b, h])) for d in range(D)]
            sc = []
            for t in range(T):
                kv = [mpmath.mpf(int(k[b, t, g, d])) * mpmath.mpf(float(ks[b, t, g])) for d in range(D)]
                sc.append(mpmath.fsum(a * c for a, c in zip(qv, kv)) / mpmath.sqrt(D))
            w = [mpmath.exp(s) for s in sc]
            z = mpmath.fsum(w)
            for d in range(D):
                out[b, h, d] = float(mpmath.fsum(w[t] * mpmath.mpf(int(v[b, t, g, d])) * mpmath.mpf(float(vs[b, t, g]))
                                                 for t in range(T)) / z)
    return out


@pytest.mark.parametrize("B,T,Hq,Hkv,D", [(2, 5, 4, 2, 8), (1, 9, 6, 3, 4), (1, 3, 2, 1, 16)])
def test_f64_and_naive_f32_against_high_precision(B, T, Hq, Hkv, D):
    g = np.random.Generator(np.random.PCG64(B * 1000 + T * 10 + Hq))
    q, qs = _codes(g, (B, Hq, D)), _scales(g, (B, Hq))
    k, ks = _codes(g, (B, T, Hkv, D)), _scales(g, (B, T, Hkv))
    v, vs = _codes(g, (B, T, Hkv, D)), _scales(g, (B, T, Hkv))
    ref = _mp_attention(q, qs, k, ks, v, vs)
    norm = oracle.attn_decode_weight_norm(q, qs, k, ks, v, vs)
    o64 = oracle.attn_decode_f64(q, qs, k, ks, v, vs)
    o32 = oracle.attn_decode_f32_naive(q, qs, k, ks, v, vs)
    assert np.all(np.abs(o64 - ref) <= 1e-13 * norm)
    assert np.all(np.abs(o32 - ref) <= 2e-5 * norm)
    # the normaliser really is sum_t P_t |v_t|: it bounds |o| and equals it for one-signed values
    assert np.all(np.abs(ref) <= norm * (1 + 1e-12))


def test_prefill_reference_is_causal_and_matches_decode_at_each_prefix():
    """Prefill reference (causal self-attention of every position): position 0 is
    token 0's value row; changing keys or values after position t leaves position t
    unchanged; the last position is the decode reference over all T tokens."""
    import heal_workloads as WL
    B, T, Hq, Hkv, D = 2, 9, 4, 2, 128
    qf, kf, vf = WL.attention_prefill_fp32(B, T, Hq, Hkv, D, seed=11)
    q, qs = oracle.quant_i16(qf)
    k, ks = oracle.quant_i16(kf)
    v, vs = oracle.quant_i16(vf)
    pos = list(range(T))
    o = oracle.attn_prefill_f64(q, qs, k, ks, v, vs, pos)
    assert o.shape == (B, T, Hq, D)
    v0 = v[:, 0].astype(np.float64) * vs[:, 0][..., None]          # [B, Hkv, D]
    assert np.allclose(o[:, 0], np.repeat(v0, Hq // Hkv, axis=1), rtol=1e-15, atol=0)
    k2, v2 = k.copy(), v.copy()
    k2[:, 5:] = -k2[:, 5:]
    v2[:, 5:] = 7
    o2 = oracle.attn_prefill_f64(q, qs, k2, ks, v2, vs, pos)
    assert np.array_equal(o2[:, :5], o[:, :5]) and not np.array_equal(o2[:, 5:], o[:, 5:])
    last = oracle.attn_decode_f64(q[:, T - 1], qs[:, T - 1], k, ks, v, vs)
    assert np.array_equal(o[:, T - 1], last)
