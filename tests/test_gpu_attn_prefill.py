"""GPU parity of INT16 prefill (causal) attention against the CPU oracle.

The oracle's prefill reference is the decode reference over keys 0 .. t for
each query position t.  Tolerance as for decode attention: per output, the
error normalized by sum_t P_t |v_t[d]| must be at most 2x that of naive FP32
attention plus the dual-FP16 weight split's 2^-21, and at most 1e-5.
"""
import numpy as np
import pytest
import torch

import error_compensated_gemm_heal_amd as heal
import heal_workloads as WL
import oracle
from metrics import attn_normwise_error

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, T, Hq, Hkv, seed):
    qf, kf, vf = WL.attention_prefill_fp32(B, T, Hq, Hkv, 128, seed)
    return oracle.quant_i16(qf) + oracle.quant_i16(kf) + oracle.quant_i16(vf)


def _positions(T):
    if T <= 130:
        return list(range(T))
    g = WL.rng(T)
    pick = set(g.choice(T, size=24, replace=False).tolist()) | {0, 1, 63, 64, 65, 127, 128, T - 2, T - 1}
    return sorted(p for p in pick if 0 <= p < T)


def _check(B, T, Hq, Hkv, seed, inputs=None):
    print(f"attn prefill B={B} T={T} Hq={Hq} Hkv={Hkv}", flush=True)
    ins = inputs if inputs is not None else _inputs(B, T, Hq, Hkv, seed)
    dev = [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in ins]
    o = heal.heal_attn_prefill_i16(*dev).cpu().numpy()
    pos = _positions(T)
    o64 = oracle.attn_prefill_f64(*ins, pos)
    o32 = oracle.attn_prefill_f32_naive(*ins, pos)
    wn = oracle.attn_prefill_weight_norm(*ins, pos)
    og = o[:, pos]
    e_gpu = attn_normwise_error(og, o64, wn)
    e_naive = attn_normwise_error(o32, o64, wn)
    print(f"   e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert np.all(np.isfinite(o))
    assert e_gpu <= min(2 * e_naive + 2.0 ** -21, 1e-5), (e_gpu, e_naive)
    return o


@pytest.mark.parametrize("B,T,Hq,Hkv", [(1, 1, 4, 1), (1, 5, 2, 2), (1, 64, 4, 2), (2, 100, 8, 2),
                                        (1, 129, 4, 4), (1, 192, 4, 2), (1, 257, 6, 3), (2, 333, 16, 2),
                                        (1, 383, 8, 4), (1, 1000, 8, 1)])
def test_attn_prefill_shapes(B, T, Hq, Hkv):
    o = _check(B, T, Hq, Hkv, seed=B * 1000 + T)
    if T >= 1:   # position 0 attends only itself: its output is token 0's value row
        q, qs, k, ks, v, vs = _inputs(B, T, Hq, Hkv, seed=B * 1000 + T)
        v0 = np.repeat(v[:, 0].astype(np.float64) * vs[:, 0][..., None], Hq // Hkv, axis=1)
        assert np.allclose(o[:, 0], v0, rtol=2.0 ** -20, atol=0)


def test_attn_prefill_peaked_scores():
    B, T, Hq, Hkv = 1, 200, 4, 1
    q, qs, k, ks, v, vs = _inputs(B, T, Hq, Hkv, seed=9)
    k = k.copy()
    k[0, 150, 0] = q[0, 199, 0]          # query 199 of head 0 aligns with key 150
    _check(B, T, Hq, Hkv, seed=0, inputs=(q, qs, k, ks, v, vs))


def test_attn_prefill_flat_scores_give_prefix_means():
    """Every key the same row: the weights of query t are uniform over keys
    0 .. t, so its output is the mean of the dequantized values of its prefix."""
    B, T, Hq, Hkv = 1, 150, 4, 1
    q, qs, k, ks, v, vs = _inputs(B, T, Hq, Hkv, seed=21)
    k = np.broadcast_to(k[:, :1], k.shape).copy()
    ks = np.broadcast_to(ks[:, :1], ks.shape).copy()
    o = _check(B, T, Hq, Hkv, seed=0, inputs=(q, qs, k, ks, v, vs))
    vt = v.astype(np.float64) * vs.astype(np.float64)[..., None]           # [B, T, Hkv, D]
    means = np.cumsum(vt, axis=1) / np.arange(1, T + 1)[None, :, None, None]
    scale = np.cumsum(np.abs(vt), axis=1) / np.arange(1, T + 1)[None, :, None, None]
    for h in range(Hq):
        err = np.abs(o[:, :, h] - means[:, :, 0]) / scale[:, :, 0]
        assert err.max() <= 1e-5, (h, err.max())


def test_attn_prefill_full_size_sampled_positions():
    """The measured shape (one 2048-token prompt, 32 query / 8 KV heads), sampled
    query positions against the binary64 oracle."""
    _check(1, 2048, 32, 8, seed=5500)


def test_attn_prefill_long_prompt_sampled_positions():
    """An 8191-token prompt (64 query blocks, the last one ragged; 128 key
    blocks for the last queries), sampled positions against the binary64 oracle."""
    _check(1, 8191, 8, 2, seed=5501)


def test_attn_prefill_pipeline_with_gpu_quantizer_and_last_position_equals_decode():
    """GPU quantizer -> prefill attention; its last position equals decode attention
    of the same query over the same cache within the tolerance of each."""
    B, T, Hq, Hkv = 2, 190, 8, 2
    qf, kf, vf = WL.attention_prefill_fp32(B, T, Hq, Hkv, 128, seed=12)
    qc, qs = heal.heal_qkv_quant_i16(torch.from_numpy(qf).to(DEV))
    kc, ks = heal.heal_qkv_quant_i16(torch.from_numpy(kf).to(DEV))
    vc, vs = heal.heal_qkv_quant_i16(torch.from_numpy(vf).to(DEV))
    o = heal.heal_attn_prefill_i16(qc, qs, kc, ks, vc, vs).cpu().numpy()
    ins = oracle.quant_i16(qf) + oracle.quant_i16(kf) + oracle.quant_i16(vf)
    pos = [0, 57, 128, T - 1]
    o64 = oracle.attn_prefill_f64(*ins, pos)
    wn = oracle.attn_prefill_weight_norm(*ins, pos)
    assert attn_normwise_error(o[:, pos], o64, wn) <= 1e-5
    od = heal.heal_attn_decode_i16(qc[:, T - 1].contiguous(), qs[:, T - 1].contiguous(), kc, ks, vc, vs).cpu().numpy()
    assert attn_normwise_error(o[:, T - 1], od, wn[:, -1]) <= 2e-5
