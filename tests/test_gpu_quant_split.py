"""GPU parity of the bit-exact rows: operand split, INT16 quant, INT16 dequant.

Every comparison is element-by-element and exact (codes, scales, fp16 bit
patterns, fp32 values) against the CPU oracle on the same seeded inputs.
"""
import numpy as np
import pytest
import torch

import error_compensated_gemm_heal_amd as heal
import heal_workloads as WL
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _u16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _special_f32():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, -65504.0, 65519.98828125, 2.0 ** -24, 2.0 ** -25, -(2.0 ** -25),
            2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -11), 1e-8, 1e-30, 1e-40, 3.0e-5, 1 + 2 ** -11, 1 + 3 * 2 ** -11,
            0.1, 1.0 / 3.0, 1000.5, 12345.678]
    return np.array(vals, np.float32)


@pytest.mark.parametrize("n", [0, 1, 3, 5, 64, 1027, (1 << 20) + 3])
def test_split_bit_exact(n):
    print(f"split n={n}", flush=True)
    g = WL.rng(100 + n % 97)
    x = WL.normal(g, (n,))
    x *= np.float32(2.0) ** g.integers(-30, 16, size=n).astype(np.float32)
    sp = _special_f32()
    x[: min(n, sp.size)] = sp[: min(n, sp.size)]
    hi_ref, lo_ref = oracle.split_f16(x)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    hi, lo = heal.heal_split_f32(torch.from_numpy(x).to(DEV), dev_status=status)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(hi), hi_ref)
    assert np.array_equal(_u16(lo), lo_ref)
    assert status.item() == (heal.HEAL_FLAG_F16_RANGE if np.any(np.abs(x) >= 65520) else 0)


def test_split_weight_distribution_subnormals():
    # weights ~ N(0, 0.02): about 0.24% of them are fp16-subnormal; none may be flushed
    W = WL.weights_nk(512, 4096, seed=2002)
    hi_ref, lo_ref = oracle.split_f16(W)
    hi, lo = heal.heal_split_f32(torch.from_numpy(W).to(DEV))
    assert np.array_equal(_u16(hi), hi_ref)
    assert np.array_equal(_u16(lo), lo_ref)
    assert ((hi_ref & 0x7C00) == 0).mean() > 0.001


def test_split_range_flag():
    x = np.array([1.0, 65519.98828125, 70000.0, -2.0], np.float32)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    hi, lo = heal.heal_split_f32(torch.from_numpy(x).to(DEV), dev_status=status)
    assert status.item() == heal.HEAL_FLAG_F16_RANGE
    hi_ref, lo_ref = oracle.split_f16(x)
    assert np.array_equal(_u16(hi), hi_ref)


def _quant_check(X):
    codes_ref, scales_ref = oracle.quant_i16(X)
    codes, scales = heal.heal_qkv_quant_i16(torch.from_numpy(X).to(DEV))
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), scales_ref.view(np.uint32))
    return codes, scales, codes_ref, scales_ref


@pytest.mark.parametrize("D", [4, 8, 20, 64, 128, 256, 1000, 4096])
def test_quant_bit_exact_row_lengths(D):
    print(f"quant D={D}", flush=True)
    g = WL.rng(300 + D)
    rows = max(3, 200000 // D)
    X = WL.normal(g, (rows, D)) * np.exp(g.uniform(-8, 8, size=(rows, 1))).astype(np.float32)
    X[0] = 0.0                                    # zero row
    X[1] = 0.0
    X[1, D // 2] = -3.5                           # one non-zero element
    X[2] = -np.abs(X[2])                          # one-signed row
    _quant_check(X)


def test_quant_tiny_and_huge_magnitudes():
    g = WL.rng(9)
    X = WL.normal(g, (64, 128))
    X[:16] *= np.float32(1e-36)                   # row maxima near the fp32 normal limit
    X[16:32] *= np.float32(1e-41)                 # subnormal rows
    X[32:48] *= np.float32(1e30)                  # below the 32767 x overflow bound (~1.04e34)
    _quant_check(X)


def test_quant_golden_ties_on_gpu():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "quant_ties.json")
    for row in json.load(open(path))["rows"]:
        x = np.array(row["x"], np.float32)
        D = (x.size + 3) // 4 * 4
        X = np.zeros((1, D), np.float32)
        X[0, : x.size] = x
        codes, _ = heal.heal_qkv_quant_i16(torch.from_numpy(X).to(DEV))
        assert codes.cpu().numpy()[0, : x.size].tolist() == row["codes"]


def test_quant_smoke_case_and_dequant():
    X = WL.smoke_quant()
    codes, scales, codes_ref, scales_ref = _quant_check(X)
    out = heal.heal_kv_dequant_i16(codes, scales, "f32").cpu().numpy()
    assert np.array_equal(out.view(np.uint32), oracle.dequant_f32(codes_ref, scales_ref).view(np.uint32))
    hi, lo = heal.heal_kv_dequant_i16(codes, None, "f16x2")
    hr, lr = oracle.dequant_f16x2(codes_ref)
    assert np.array_equal(_u16(hi), hr) and np.array_equal(_u16(lo), lr)


def test_dequant_all_codes():
    q = np.arange(-32768, 32768, dtype=np.int32).astype(np.int16).reshape(512, 128)
    s = (np.exp(WL.rng(4).uniform(-10, 3, size=512)) / 32767).astype(np.float32)
    qd = torch.from_numpy(q).to(DEV)
    out = heal.heal_kv_dequant_i16(qd, torch.from_numpy(s).to(DEV), "f32").cpu().numpy()
    assert np.array_equal(out.view(np.uint32), oracle.dequant_f32(q, s).view(np.uint32))
    hi, lo = heal.heal_kv_dequant_i16(qd, None, "f16x2")
    hr, lr = oracle.dequant_f16x2(q)
    assert np.array_equal(_u16(hi), hr) and np.array_equal(_u16(lo), lr)


def test_quant_dequant_qwen_layer_full_size_every_row():
    """Full Qwen3-8B-like layer: 32 x 2048 tokens, 32 + 8 + 8 heads of 128.

    The whole tensor is quantized and dequantized on the GPU exactly as the
    benchmark does (one [tokens, 48, 128] launch each), and every one of its
    3.1 M rows is compared bit for bit with the oracle's quantizer and
    dequantizer (402.65 M codes, scales and fp32 values)."""
    print("quant full size: generating", flush=True)
    tokens = 32 * 2048
    Q, K, V = WL.qkv(tokens, 32, 8, 128, seed=4000)
    X = np.concatenate([Q, K, V], axis=1)          # [tokens, 48, 128]
    del Q, K, V
    Xd = torch.from_numpy(X).to(DEV)
    codes, scales = heal.heal_qkv_quant_i16(Xd)
    deq = heal.heal_kv_dequant_i16(codes, scales, "f32")
    torch.cuda.synchronize()
    del Xd
    print("quant full size: oracle", flush=True)
    cr, sr = oracle.quant_i16(X)
    del X
    print("quant full size: comparing", flush=True)
    assert np.array_equal(codes.cpu().numpy(), cr)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(deq.cpu().numpy().view(np.uint32), oracle.dequant_f32(cr, sr).view(np.uint32))


def test_calibration_kernels_run():
    """The roofline calibration kernels (measurement only) run and return finite values."""
    out, flops = heal.heal_calib_mfma_f16(10, 8)
    assert flops == 8 * 4 * 10 * 16 * 32768
    assert torch.isfinite(out[: 8 * 256]).all().item()
    buf = torch.arange(1 << 20, dtype=torch.float32, device="cuda:0")
    r = heal.heal_calib_read(buf, 64)
    torch.cuda.synchronize()
    assert torch.isfinite(r).all().item()
