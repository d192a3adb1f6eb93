"""GPU parity of INT16 decode attention against the CPU oracle.

Inputs are N(0,1) Q/K/V quantized by the oracle's INT16 quantizer (the codes
are bit-identical to the GPU quantizer's, which test_gpu_quant_split checks).
Tolerance: per output, |o - o64| normalized by sum_t P_t |v_t[d]| must be at
most 2x the naive FP32 attention error (plus the dual-FP16 weight split's own
2^-21 where the naive error is a handful of roundings) and at most 1e-5.
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
    qf, kf, vf = WL.attention_fp32(B, T, Hq, Hkv, 128, seed)
    q, qs = oracle.quant_i16(qf)
    k, ks = oracle.quant_i16(kf)
    v, vs = oracle.quant_i16(vf)
    return q, qs, k, ks, v, vs


def _check(B, T, Hq, Hkv, seed, inputs=None):
    print(f"attn B={B} T={T} Hq={Hq} Hkv={Hkv}", flush=True)
    ins = inputs if inputs is not None else _inputs(B, T, Hq, Hkv, seed)
    dev = [torch.from_numpy(x).to(DEV) for x in ins]
    o = heal.heal_attn_decode_i16(*dev)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    o64 = oracle.attn_decode_f64(*ins)
    o32 = oracle.attn_decode_f32_naive(*ins)
    wn = oracle.attn_decode_weight_norm(*ins)
    e_gpu = attn_normwise_error(o, o64, wn)
    e_naive = attn_normwise_error(o32, o64, wn)
    print(f"   e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert np.all(np.isfinite(o))
    assert e_gpu <= min(2 * e_naive + 2.0 ** -21, 1e-5), (e_gpu, e_naive)
    return o, o64


def test_attn_single_token_is_value_row():
    o, o64 = _check(2, 1, 8, 2, seed=1)
    assert np.allclose(o, o64, rtol=2.0 ** -20, atol=0)


@pytest.mark.parametrize("B,T,Hq,Hkv", [(1, 5, 4, 1), (2, 37, 8, 2), (1, 128, 4, 4), (2, 300, 6, 3),
                                        (1, 129, 8, 1), (3, 1000, 16, 2), (1, 257, 7, 1), (2, 64, 2, 2),
                                        (1, 3000, 8, 2), (1, 20000, 8, 8)])
def test_attn_ragged_shapes(B, T, Hq, Hkv):
    _check(B, T, Hq, Hkv, seed=B * 100 + T)


def test_attn_peaked_and_flat_scores():
    B, T, Hq, Hkv = 1, 200, 4, 1
    q, qs, k, ks, v, vs = _inputs(B, T, Hq, Hkv, seed=5)
    k = k.copy()
    k[0, 77, 0] = q[0, 0]                 # one token aligned with head 0: a peaked softmax
    k[0, :, 0, :] = np.where(np.arange(T)[:, None] == 77, k[0, :, 0, :], 0)   # others flat (zero score)
    _check(B, T, Hq, Hkv, seed=0, inputs=(q, qs, k, ks, v, vs))


def test_attn_qwen_decode_full_size():
    """Decode attention: batch 16, context 8192, 32 query / 8 KV heads, D = 128."""
    _check(16, 8192, 32, 8, seed=5000)


def test_attn_pipeline_with_gpu_quantizer():
    """a4 -> a6 on the device: the GPU quantizer's codes feed the attention kernel."""
    B, T, Hq, Hkv = 2, 333, 8, 2
    qf, kf, vf = WL.attention_fp32(B, T, Hq, Hkv, 128, seed=6)
    qc, qs = heal.heal_qkv_quant_i16(torch.from_numpy(qf).to(DEV))
    kc, ks = heal.heal_qkv_quant_i16(torch.from_numpy(kf).to(DEV))
    vc, vs = heal.heal_qkv_quant_i16(torch.from_numpy(vf).to(DEV))
    o = heal.heal_attn_decode_i16(qc, qs, kc, ks, vc, vs).cpu().numpy()
    ins = (oracle.quant_i16(qf) + oracle.quant_i16(kf) + oracle.quant_i16(vf))
    o64 = oracle.attn_decode_f64(*ins)
    wn = oracle.attn_decode_weight_norm(*ins)
    assert attn_normwise_error(o, o64, wn) <= 1e-5
