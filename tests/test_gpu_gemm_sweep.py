"""A seeded sweep of GEMM shapes, weight forms and layouts against the CPU oracle.

Each case draws M, N, K, the weight's layout and form (fp32 streamed, binary16,
packed once) from one seeded generator, so the sweep reaches combinations the
hand-picked cases do not: ragged N and K on every path, M on both sides of the
decode/prefill switch (64/65) and of the row-tile switches (16/17, 32/33), and
N >= 4096 at M <= 16 with short k chunks, where the chunks are the waves of one
workgroup; the activation's absolute scale is a power of two from 2^-30 to 2^13.  Every case meets the normwise bar of tests/metrics.py against the
binary64 oracle; on the decode path (M <= 64, [N, K] weights) the rows of the
call also equal the first rows of the same product at M = 64, bit for bit (the
k chunking depends on N and K only).
"""
import numpy as np
import pytest
import torch

import error_compensated_gemm_heal_amd as heal
import heal_workloads as WL
import oracle
from metrics import gemm_normwise_error, gemm_tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MS = [1, 2, 5, 8, 13, 16, 17, 31, 32, 33, 48, 64, 65, 100, 257]


def _cases(n=120, seed=9100):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(g.choice(MS))
        if M <= 16 and i % 3 == 0:
            N = int(g.integers(4081, 6001))       # 256+ slices of 16 rows
            K = int(g.integers(300, 2049))         # short chunks: at most 4 blocks each
        else:
            N = int(g.integers(1, 700))
            K = int(g.integers(1, 3001))
        layout = "kn" if (M > 64 and g.random() < 0.3) else "nk"
        form = str(g.choice(["fp32", "f16", "packed"]))
        scale = float(2.0 ** int(g.integers(-30, 14)))   # the activation's absolute scale
        out.append((i, M, N, K, layout, form, scale))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}-{c[4]}-{c[5]}")
def test_gemm_seeded_sweep(case):
    i, M, N, K, layout, form, scale = case
    print(f"sweep case {i}: M={M} N={N} K={K} {layout} {form} scale={scale:g}", flush=True)
    M64 = 64 if M <= 64 else M
    A, W = WL.decode_gemm(M64, K, N, seed=9200 + i)
    A = A * np.float32(scale)          # a power of two: exact
    if layout == "kn":
        W = np.ascontiguousarray(W.T)
    if form == "f16":
        W = W.astype(np.float16)
    W32 = W.astype(np.float32)
    Ad, Wd = torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV)
    Wop = heal.heal_pack_w(Wd, layout) if form == "packed" else Wd
    kw = {} if form == "packed" else {"w_layout": layout}
    C = heal.heal_gemm_f32c(Ad[:M], Wop, **kw).cpu().numpy()
    C64 = oracle.gemm_f64(A[:M], W32, layout)
    C32 = oracle.gemm_f32_naive(A[:M], W32, layout)
    e_gpu = gemm_normwise_error(C, C64, A[:M], W32, layout)
    e_naive = gemm_normwise_error(C32, C64, A[:M], W32, layout)
    print(f"  e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert np.all(np.isfinite(C))
    assert e_gpu <= gemm_tolerance(e_naive, K), (e_gpu, e_naive)
    if M < 64 and layout == "nk":
        C_all = heal.heal_gemm_f32c(Ad, Wop, **kw).cpu().numpy()
        assert np.array_equal(C, C_all[:M])


# ---- the operand split and the packed layout, bit for bit --------------------------------

def _pack_cases(n=30, seed=9150):
    g = np.random.default_rng(seed)
    return [(i, int(g.integers(1, 700)), int(g.integers(1, 20000)), str(g.choice(["nk", "kn"])),
             int(g.integers(-60, 40))) for i in range(n)]


@pytest.mark.parametrize("case", _pack_cases(), ids=lambda c: f"{c[0]}-R{c[1]}-K{c[2]}-{c[3]}-e{c[4]}")
def test_pack_and_split_seeded_sweep(case):
    """heal_pack_w's hi parts, residuals and row exponents equal the oracle's split
    of the normalized rows (both layouts, the one-pass and two-pass packers, value
    scales 2^-60 .. 2^39 with zero rows and large elements), and heal_split_f32's
    planes equal the oracle's plain split of the same values."""
    from test_gpu_gemm import unpack
    i, R, K, layout, e = case
    print(f"pack sweep {i}: R={R} K={K} {layout} scale=2^{e}", flush=True)
    g = WL.rng(9160 + i)
    X = (g.standard_normal((R, K)) * np.exp2(e)).astype(np.float32)
    X[g.random(R) < 0.05] = 0.0
    X[:, g.choice(K, size=min(K, 2), replace=False)] *= np.float32(300.0)
    src = X if layout == "nk" else np.ascontiguousarray(X.T)
    p = heal.heal_pack_w(torch.from_numpy(src).to(DEV), layout)
    h, r, ex = unpack(p.buf.cpu().numpy(), R, K)
    oh, orr, oe = oracle.split_rownorm(X)
    assert np.array_equal(ex, oe)
    assert np.array_equal(h[:, :K], oh) and np.array_equal(r[:, :K], orr)
    flat = X.reshape(-1)
    if flat.size <= 1 << 22 and np.all(np.abs(flat) < 65504.0):
        hi, lo = heal.heal_split_f32(torch.from_numpy(flat).to(DEV))
        oh2, ol2 = oracle.split_f16(flat)
        assert np.array_equal(hi.cpu().numpy().view(np.uint16), oh2)
        assert np.array_equal(lo.cpu().numpy().view(np.uint16), ol2)


# ---- the Q/K/V projection stored as INT16, bit for bit on exact operands ------------------

def _qkv_cases(n=16, seed=9170):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(g.choice([1, 2, 4]))
        out.append((i, int(g.choice([1, 3, 16, 17, 64, 65, 200, 513])), int(g.integers(1, 33)) * 32,
                    int(g.choice([1, 2, 4])) * Hkv, Hkv, str(g.choice(["fp32", "fp16", "packed16"]))))
    return out


@pytest.mark.parametrize("case", _qkv_cases(), ids=lambda c: f"{c[0]}-M{c[1]}-K{c[2]}-{c[3]}x{c[4]}-{c[5]}")
def test_qkv_proj_seeded_sweep(case):
    """heal_qkv_proj_quant_i16 on dyadic-grid operands (every partial sum exact in
    fp32): Q codes and scales, and the K/V rows scattered by slot (padding tokens
    write nothing, untouched slots keep their contents), equal the oracle's INT16
    quantization of the binary64 product, bit for bit."""
    from test_gpu_qkv_proj import _grid_operands, _slots, _run, _check_scatter
    i, M, K, Hq, Hkv, weight = case
    D = 128
    H = Hq + 2 * Hkv
    print(f"qkv sweep {i}: M={M} K={K} Hq={Hq} Hkv={Hkv} {weight}", flush=True)
    A, W = _grid_operands(M, K, H * D, seed=9180 + i)
    num_slots = 2 * M + 5
    slots = _slots(M, num_slots, seed=9190 + i)
    out = _run(A, W, Hq, Hkv, D, slots, num_slots, weight)
    codes, scales = oracle.quant_i16(oracle.gemm_f64(A, W).astype(np.float32).reshape(M, H, D))
    _check_scatter(codes, scales, out, slots, Hq, Hkv)
