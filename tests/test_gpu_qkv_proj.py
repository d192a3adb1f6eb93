"""Fused Q/K/V projection stored as INT16 (heal_qkv_proj_quant_i16).

Bit-exact cases use operands on small dyadic grids, for which every partial
sum of the product is exact in fp32: the GPU product then equals the oracle's
binary64 product, so the codes must equal, bit for bit, the oracle's INT16
quantization of that product.  General operands are checked against the
binary64 product within the GEMM tolerance plus half a quantization step.
The scatter is checked slot by slot: K/V rows at slot_mapping[m], nothing at
negative slots, untouched slots keep their contents, out-of-range slots are
flagged.  A pipeline test runs the projection into a KV cache and decode
attention over that cache.
"""
import numpy as np
import pytest
import torch

import error_compensated_gemm_heal_amd as heal
import heal_workloads as WL
import oracle
from metrics import attn_normwise_error, gemm_tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENT = np.int16(0x5A5A)


def _grid_operands(M, K, N, seed):
    """A on multiples of 1/8 in [-1, 1], W on multiples of 1/64 in [-1/8, 1/8]:
    binary16-exact, and every partial sum over K <= 1024 is exact in fp32."""
    g = WL.rng(seed)
    A = (g.integers(-8, 9, size=(M, K)) / 8.0).astype(np.float32)
    W = (g.integers(-8, 9, size=(N, K)) / 64.0).astype(np.float32)
    return A, W


def _slots(M, num_slots, seed):
    g = WL.rng(seed)
    s = g.permutation(num_slots)[:M].astype(np.int64)
    s[::5] = -1                               # padding tokens write no K/V
    return s


def _caches(num_slots, Hkv, D):
    kc = torch.full((num_slots, Hkv, D), int(SENT), dtype=torch.int16, device=DEV)
    vc = torch.full((num_slots, Hkv, D), int(SENT), dtype=torch.int16, device=DEV)
    ks = torch.full((num_slots, Hkv), -1.0, dtype=torch.float32, device=DEV)
    vs = torch.full((num_slots, Hkv), -1.0, dtype=torch.float32, device=DEV)
    return kc, ks, vc, vs


def _run(A, W, Hq, Hkv, D, slots, num_slots, weight="fp32", status=None):
    Ad = torch.from_numpy(A).to(DEV)
    Wd = torch.from_numpy(W.astype(np.float16) if weight != "fp32" else W).to(DEV)
    if weight == "packed16":
        Wd = heal.heal_pack_w(Wd)
    kc, ks, vc, vs = _caches(num_slots, Hkv, D)
    qc, qs = heal.heal_qkv_proj_quant_i16(Ad, Wd, Hq, Hkv, D, torch.from_numpy(slots).to(DEV), kc, ks, vc, vs,
                                          dev_status=status)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (qc, qs, kc, ks, vc, vs)]


def _check_scatter(codes, scales, out, slots, Hq, Hkv):
    qc, qs, kc, ks, vc, vs = out
    assert np.array_equal(qc, codes[:, :Hq]) and np.array_equal(qs, scales[:, :Hq])
    written = np.zeros(kc.shape[0], bool)
    for m, slot in enumerate(slots):
        if slot < 0:
            continue
        written[slot] = True
        assert np.array_equal(kc[slot], codes[m, Hq:Hq + Hkv]) and np.array_equal(ks[slot], scales[m, Hq:Hq + Hkv])
        assert np.array_equal(vc[slot], codes[m, Hq + Hkv:]) and np.array_equal(vs[slot], scales[m, Hq + Hkv:])
    assert np.all(kc[~written] == SENT) and np.all(vc[~written] == SENT)
    assert np.all(ks[~written] == -1.0) and np.all(vs[~written] == -1.0)


@pytest.mark.parametrize("weight", ["fp32", "fp16", "packed16"])
@pytest.mark.parametrize("M", [1, 16, 64, 300])
def test_qkv_proj_codes_bit_exact_on_exact_operands(M, weight):
    """Decode (M <= 64) and prefill paths, fp32, fp16 and packed fp16 weights."""
    K, Hq, Hkv, D = 512, 4, 2, 128
    H = Hq + 2 * Hkv
    print(f"qkv proj exact M={M} {weight}", flush=True)
    A, W = _grid_operands(M, K, H * D, seed=8000 + M)
    num_slots = 2 * M + 3
    slots = _slots(M, num_slots, seed=M)
    out = _run(A, W, Hq, Hkv, D, slots, num_slots, weight)
    C64 = oracle.gemm_f64(A, W)
    codes, scales = oracle.quant_i16(C64.astype(np.float32).reshape(M, H, D))
    _check_scatter(codes, scales, out, slots, Hq, Hkv)


def _gemm_then_quant(A, W, Hq, Hkv, D, weight="fp32"):
    """The GPU GEMM, then the standalone GPU quantizer over its fp32 product."""
    M, H = A.shape[0], Hq + 2 * Hkv
    Ad = torch.from_numpy(A).to(DEV)
    Wd = torch.from_numpy(W.astype(np.float16) if weight != "fp32" else W).to(DEV)
    if weight == "packed16":
        Wd = heal.heal_pack_w(Wd)
    C = heal.heal_gemm_f32c(Ad, Wd)
    codes, scales = heal.heal_qkv_quant_i16(C.view(M, H, D))
    return codes.cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("M,K,Hq,Hkv,weight", [(300, 200, 4, 2, "fp32"), (300, 200, 4, 2, "packed16"),
                                                (1000, 100, 8, 2, "fp16"), (257, 96, 3, 1, "fp32"),
                                                (2048, 4096, 32, 8, "fp32"),
                                                (2048, 4096, 32, 8, "packed16")])
def test_qkv_proj_fused_epilogue_equals_gemm_then_quant(M, K, Hq, Hkv, weight):
    """Shapes the prefill kernel runs without its k split quantize in the GEMM's
    epilogue (the workspace then holds the packed operands only): codes and
    scales equal, bit for bit, the GEMM's stored product quantized by the
    standalone kernel, for random operands."""
    D, H = 128, Hq + 2 * Hkv
    print(f"qkv fused M={M} K={K} Hq={Hq} Hkv={Hkv} {weight}", flush=True)
    flags = 0 if weight == "fp32" else (heal.HEAL_W_F16 | (heal.HEAL_W_PACKED if weight == "packed16" else 0))
    assert heal.heal_qkv_proj_quant_workspace(M, K, Hq, Hkv, D, flags) == \
        heal.heal_gemm_f32c_workspace(M, H * D, K, flags)
    g = WL.rng(8400 + M + K)
    A = WL.normal(g, (M, K))
    W = WL.normal(g, (H * D, K), std=0.02)
    num_slots = M + 37
    slots = _slots(M, num_slots, seed=M + 1)
    out = _run(A, W, Hq, Hkv, D, slots, num_slots, weight)
    codes, scales = _gemm_then_quant(A, W, Hq, Hkv, D, weight)
    _check_scatter(codes, scales, out, slots, Hq, Hkv)


@pytest.mark.parametrize("mode", ["one_product", "bf16x3"])
@pytest.mark.parametrize("M", [7, 300])
def test_qkv_proj_precision_modes_exact_operands(mode, M):
    """The GEMM's one-product and BF16 three-way modes through the projection (the
    two-pass form): on dyadic-grid operands, which both modes hold exactly, the codes
    equal the oracle's quantization of the binary64 product."""
    K, Hq, Hkv, D = 384, 4, 2, 128
    H = Hq + 2 * Hkv
    A, W = _grid_operands(M, K, H * D, seed=8600 + M)
    slots = _slots(M, M + 5, seed=M + 7)
    kc, ks, vc, vs = _caches(M + 5, Hkv, D)
    qc, qs = heal.heal_qkv_proj_quant_i16(torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV), Hq, Hkv, D,
                                          torch.from_numpy(slots).to(DEV), kc, ks, vc, vs,
                                          one_product=(mode == "one_product"), bf16x3=(mode == "bf16x3"))
    out = [t.cpu().numpy() for t in (qc, qs, kc, ks, vc, vs)]
    codes, scales = oracle.quant_i16(oracle.gemm_f64(A, W).astype(np.float32).reshape(M, H, D))
    _check_scatter(codes, scales, out, slots, Hq, Hkv)


def test_qkv_proj_fused_epilogue_exact_operands():
    """A fused shape on dyadic-grid operands: bit-equal to the oracle's INT16
    quantization of the binary64 product."""
    M, K, Hq, Hkv, D = 300, 200, 4, 2, 128
    H = Hq + 2 * Hkv
    A, W = _grid_operands(M, K, H * D, seed=8500)
    slots = _slots(M, 2 * M, seed=3)
    out = _run(A, W, Hq, Hkv, D, slots, 2 * M)
    codes, scales = oracle.quant_i16(oracle.gemm_f64(A, W).astype(np.float32).reshape(M, H, D))
    _check_scatter(codes, scales, out, slots, Hq, Hkv)


@pytest.mark.parametrize("M", [8, 200])
def test_qkv_proj_general_operands_within_bound(M):
    """Random operands: each dequantized value is within half a quantization step
    (the quantizer's own bound) plus the GEMM tolerance of the binary64 product."""
    K, Hq, Hkv, D = 768, 4, 2, 128
    H = Hq + 2 * Hkv
    g = WL.rng(8100 + M)
    A = WL.normal(g, (M, K))
    W = WL.normal(g, (H * D, K), std=0.02)
    slots = np.arange(M, dtype=np.int64)
    qc, qs, kc, ks, vc, vs = _run(A, W, Hq, Hkv, D, slots, M)
    codes = np.concatenate([qc, kc, vc], axis=1).astype(np.float64)            # [M, H, D]
    scales = np.concatenate([qs, ks, vs], axis=1).astype(np.float64)           # [M, H]
    deq = codes * scales[:, :, None]
    C64 = oracle.gemm_f64(A, W).reshape(M, H, D)
    norm_a = np.linalg.norm(A.astype(np.float64), axis=1)[:, None, None]
    norm_b = np.linalg.norm(W.astype(np.float64), axis=1).reshape(1, H, D)
    bar = scales[:, :, None] / 2 * (1 + 2.0 ** -6) + 1e-5 * norm_a * norm_b
    assert np.all(np.abs(deq - C64) <= bar)


def test_qkv_proj_slot_out_of_range_is_flagged_and_skipped():
    K, Hq, Hkv, D, M = 256, 2, 1, 128, 6
    A, W = _grid_operands(M, K, (Hq + 2 * Hkv) * D, seed=8200)
    slots = np.array([0, 7, 2, 1, -1, 3], np.int64)      # 7 is past the 5 slots
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = _run(A, W, Hq, Hkv, D, slots, 5, status=st)
    assert st.item() == heal.HEAL_FLAG_SLOT_RANGE
    C64 = oracle.gemm_f64(A, W)
    codes, scales = oracle.quant_i16(C64.astype(np.float32).reshape(M, Hq + 2 * Hkv, D))
    slots_ok = np.where(slots >= 5, -1, slots)
    _check_scatter(codes, scales, out, slots_ok, Hq, Hkv)


def test_qkv_proj_fused_epilogue_slot_out_of_range():
    """The INT16 epilogue of the GEMM (a shape without k split) flags slots past
    the cache and writes nothing for them, like the two-pass form."""
    M, K, Hq, Hkv, D = 300, 160, 2, 1, 128
    H = Hq + 2 * Hkv
    assert heal.heal_qkv_proj_quant_workspace(M, K, Hq, Hkv, D, 0) == heal.heal_gemm_f32c_workspace(M, H * D, K, 0)
    A, W = _grid_operands(M, K, H * D, seed=8700)
    num_slots = 280
    slots = np.arange(M, dtype=np.int64)          # tokens 280 .. 299 fall past the cache
    slots[::7] = -1
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = _run(A, W, Hq, Hkv, D, slots, num_slots, status=st)
    assert st.item() == heal.HEAL_FLAG_SLOT_RANGE
    codes, scales = oracle.quant_i16(oracle.gemm_f64(A, W).astype(np.float32).reshape(M, H, D))
    _check_scatter(codes, scales, out, np.where(slots >= num_slots, -1, slots), Hq, Hkv)


def test_qkv_proj_into_cache_then_decode_attention():
    """Projection of B sequences of T tokens into a contiguous KV cache (slot =
    b T + t, i.e. [B, T, Hkv, D]), then decode attention of each sequence's last
    token over its T cached tokens, against the oracle on the oracle's own codes."""
    B, T, Hq, Hkv, D, K = 2, 96, 8, 2, 128, 256
    H = Hq + 2 * Hkv
    A, W = _grid_operands(B * T, K, H * D, seed=8300)
    slots = np.arange(B * T, dtype=np.int64)
    qc, qs, kc, ks, vc, vs = _run(A, W, Hq, Hkv, D, slots, B * T)
    codes, scales = oracle.quant_i16(oracle.gemm_f64(A, W).astype(np.float32).reshape(B * T, H, D))
    last = np.arange(B) * T + T - 1
    ins = (codes[last, :Hq], scales[last, :Hq],
           codes[:, Hq:Hq + Hkv].reshape(B, T, Hkv, D), scales[:, Hq:Hq + Hkv].reshape(B, T, Hkv),
           codes[:, Hq + Hkv:].reshape(B, T, Hkv, D), scales[:, Hq + Hkv:].reshape(B, T, Hkv))
    dev = [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in
           (qc[last], qs[last], kc.reshape(B, T, Hkv, D), ks.reshape(B, T, Hkv), vc.reshape(B, T, Hkv, D),
            vs.reshape(B, T, Hkv))]
    o = heal.heal_attn_decode_i16(*dev).cpu().numpy()
    o64 = oracle.attn_decode_f64(*[np.ascontiguousarray(x) for x in ins])
    o32 = oracle.attn_decode_f32_naive(*[np.ascontiguousarray(x) for x in ins])
    wn = oracle.attn_decode_weight_norm(*[np.ascontiguousarray(x) for x in ins])
    e_gpu = attn_normwise_error(o, o64, wn)
    e_naive = attn_normwise_error(o32, o64, wn)
    assert e_gpu <= min(2 * e_naive + 2.0 ** -21, 1e-5), (e_gpu, e_naive)
