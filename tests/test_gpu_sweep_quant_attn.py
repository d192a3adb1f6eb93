"""Seeded sweeps of the INT16 quantizer, its dequant and the two attention kernels
against the CPU oracle.

Quant and dequant: row counts and row lengths D (multiples of 4 up to 4096) drawn from one seeded
generator, values at scales 2^-60 .. 2^60 with zero rows and single large
elements mixed in; codes, scales and both dequant forms must match the oracle bit
for bit.  Attention: batch, context length, query/KV head counts (GQA groups 1 to
8) drawn the same way, against the binary64 oracle at the bar of the attention
tests (2x the naive FP32 error plus 2^-21, at most 1e-5).
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


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


def _quant_cases(n=40, seed=9300):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        # the quantizer's contract: D a multiple of 4, 4 .. 4096
        D = int(g.choice([4, 8, 12, 64, 128, 132, 500, 1024, 4096])) if i % 2 else 4 * int(g.integers(1, 1025))
        rows = int(g.integers(1, max(2, 400000 // D)))
        out.append((i, rows, D, int(g.integers(-60, 61))))
    return out


@pytest.mark.parametrize("case", _quant_cases(), ids=lambda c: f"{c[0]}-rows{c[1]}-D{c[2]}-e{c[3]}")
def test_quant_dequant_seeded_sweep(case):
    i, rows, D, e = case
    print(f"quant sweep {i}: rows={rows} D={D} scale=2^{e}", flush=True)
    g = WL.rng(9400 + i)
    X = (g.standard_normal((rows, D)) * np.exp2(e)).astype(np.float32)
    X[g.random(rows) < 0.05] = 0.0                       # zero rows
    hot = g.random(rows) < 0.05                          # one large element in some rows
    X[hot, g.integers(0, D, size=int(hot.sum()))] *= np.float32(1000.0)
    codes_ref, scales_ref = oracle.quant_i16(X)
    codes, scales = heal.heal_qkv_quant_i16(torch.from_numpy(X).to(DEV))
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), scales_ref.view(np.uint32))
    out = heal.heal_kv_dequant_i16(codes, scales, "f32").cpu().numpy()
    assert np.array_equal(out.view(np.uint32), oracle.dequant_f32(codes_ref, scales_ref).view(np.uint32))
    hi, lo = heal.heal_kv_dequant_i16(codes, None, "f16x2")
    hr, lr = oracle.dequant_f16x2(codes_ref)
    assert np.array_equal(_u16(hi), hr) and np.array_equal(_u16(lo), lr)


def _attn_cases(n, seed, tmax):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(g.choice([1, 2, 4, 8]))
        G = int(g.choice([1, 2, 3, 4, 5, 8]))
        out.append((i, int(g.integers(1, 4)), int(g.integers(1, tmax)), G * Hkv, Hkv))
    return out


@pytest.mark.parametrize("case", _attn_cases(16, 9500, 2500), ids=lambda c: f"{c[0]}-B{c[1]}-T{c[2]}-{c[3]}x{c[4]}")
def test_attn_decode_seeded_sweep(case):
    i, B, T, Hq, Hkv = case
    print(f"attn decode sweep {i}: B={B} T={T} Hq={Hq} Hkv={Hkv}", flush=True)
    qf, kf, vf = WL.attention_fp32(B, T, Hq, Hkv, 128, 9600 + i)
    ins = oracle.quant_i16(qf) + oracle.quant_i16(kf) + oracle.quant_i16(vf)
    o = heal.heal_attn_decode_i16(*[torch.from_numpy(x).to(DEV) for x in ins]).cpu().numpy()
    o64 = oracle.attn_decode_f64(*ins)
    o32 = oracle.attn_decode_f32_naive(*ins)
    wn = oracle.attn_decode_weight_norm(*ins)
    e_gpu, e_naive = attn_normwise_error(o, o64, wn), attn_normwise_error(o32, o64, wn)
    print(f"  e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert np.all(np.isfinite(o))
    assert e_gpu <= min(2 * e_naive + 2.0 ** -21, 1e-5), (e_gpu, e_naive)


@pytest.mark.parametrize("case", _attn_cases(12, 9700, 700), ids=lambda c: f"{c[0]}-B{c[1]}-T{c[2]}-{c[3]}x{c[4]}")
def test_attn_prefill_seeded_sweep(case):
    i, B, T, Hq, Hkv = case
    B = min(B, 2)
    print(f"attn prefill sweep {i}: B={B} T={T} Hq={Hq} Hkv={Hkv}", flush=True)
    qf, kf, vf = WL.attention_prefill_fp32(B, T, Hq, Hkv, 128, 9800 + i)
    ins = oracle.quant_i16(qf) + oracle.quant_i16(kf) + oracle.quant_i16(vf)
    dev = [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in ins]
    o = heal.heal_attn_prefill_i16(*dev).cpu().numpy()
    g = WL.rng(9900 + i)
    pos = sorted(set(g.choice(T, size=min(T, 20), replace=False).tolist()) | {0, T - 1})
    o64 = oracle.attn_prefill_f64(*ins, pos)
    o32 = oracle.attn_prefill_f32_naive(*ins, pos)
    wn = oracle.attn_prefill_weight_norm(*ins, pos)
    og = o[:, pos]
    e_gpu, e_naive = attn_normwise_error(og, o64, wn), attn_normwise_error(o32, o64, wn)
    print(f"  e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert np.all(np.isfinite(o))
    assert e_gpu <= min(2 * e_naive + 2.0 ** -21, 1e-5), (e_gpu, e_naive)
