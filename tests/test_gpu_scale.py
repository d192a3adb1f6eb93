"""The compensated GEMM at every activation scale, on every path.

FP16's dynamic range is narrow (HEAL paper, section 3, "Mitigating GEMM
Truncation via FP16 Promotion and Algebraic Compensation"): values far below
it lose bits when split, values above it overflow.  The library normalizes
each operand row by a power of two before the split and scales the product
back, so:
  * the tolerance against the binary64 oracle holds for activations of any
    magnitude (sigma from 1e-20 to 1e6 here, and rows of mixed scales);
  * scaling a row of A by 2^j scales that row of C by 2^j, bit for bit.
Paths: decode with the in-kernel split (M <= 16) and with split planes
(M > 16), fp32 and binary16 weights, streamed or packed; prefill with and
without its k split, packed weight, packed activation, binary16 weight; the
Q/K/V projection with INT16 output, fused and two-pass.
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

SCALES = [1.0, 1e-2, 1e-3, 1e-4, 1e-5, 1e-8, 1e-20, 1e6]

# (label, M, K, N, weight form): decode in-kernel split, decode split planes,
# prefill k-split grid, prefill grid without k split (144 tiles)
PATHS = [("decode_ink", 8, 1024, 384, "fp32"), ("decode_planes", 40, 1024, 384, "fp32"),
         ("decode_w16", 16, 1024, 256, "fp16"), ("prefill_ksplit", 300, 1024, 512, "fp32"),
         ("prefill", 2048, 256, 4608, "fp32"), ("prefill_packed", 300, 768, 640, "packed"),
         ("prefill_w16", 300, 768, 640, "fp16"), ("prefill_packed_a", 260, 512, 384, "packed_a"),
         ("decode_packed", 8, 1024, 384, "packed"), ("decode_packed_planes", 40, 1000, 384, "packed"),
         ("decode_packed_w16", 16, 1024, 256, "packed16")]


def _operands(M, K, N, sigma, seed):
    A, W = WL.decode_gemm(M, K, N, seed)
    with np.errstate(over="ignore", under="ignore"):
        A = (A.astype(np.float64) * sigma).astype(np.float32)
    return A, W


def _gpu(A, W, form):
    Ad = torch.from_numpy(A).to(DEV)
    if form in ("fp16", "packed16"):
        Wd = torch.from_numpy(W.astype(np.float16)).to(DEV)
    else:
        Wd = torch.from_numpy(W).to(DEV)
    if form in ("packed", "packed_a", "packed16"):
        Wd = heal.heal_pack_w(Wd)
    if form == "packed_a":
        Ad = heal.heal_pack_w(Ad)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = heal.heal_gemm_f32c(Ad, Wd, dev_status=st).cpu().numpy()
    assert st.item() == 0
    return C


def _rows(M):
    return np.arange(M) if M <= 64 else np.unique(np.r_[0, 1, M - 1, WL.rng(M).choice(M, size=29, replace=False)])


def _check(C, A, W, rows, label):
    K = A.shape[1]
    C64 = oracle.gemm_f64_rows(A, W, rows)
    C32 = oracle.gemm_f32_naive_rows(A, W, rows)
    e_gpu = gemm_normwise_error(C[rows], C64, A, W, rows=rows)
    e_naive = gemm_normwise_error(C32, C64, A, W, rows=rows)
    print(f"  {label}: e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert np.all(np.isfinite(C[rows]))
    assert e_gpu <= gemm_tolerance(e_naive, K), (label, e_gpu, e_naive)


@pytest.mark.parametrize("label,M,K,N,form", PATHS)
def test_gemm_tolerance_at_every_activation_scale(label, M, K, N, form):
    for i, sigma in enumerate(SCALES):
        print(f"scale {label} M={M} K={K} N={N} sigma={sigma:g}", flush=True)
        A, W = _operands(M, K, N, sigma, seed=9000 + 17 * i + M)
        Wref = W.astype(np.float16).astype(np.float32) if form in ("fp16", "packed16") else W
        C = _gpu(A, W, form)
        _check(C, A, Wref, _rows(M), f"sigma={sigma:g}")


@pytest.mark.parametrize("label,M,K,N,form", PATHS)
def test_gemm_row_scaling_is_exact(label, M, K, N, form):
    """Rows of A scaled by 2^j (j differing per row, from -60 to 40) give the rows
    of C scaled by 2^j, bit for bit."""
    print(f"row scaling {label} M={M}", flush=True)
    A, W = _operands(M, K, N, 1.0, seed=9500 + M)
    j = WL.rng(9501 + M).integers(-60, 41, size=M)
    A2 = np.ldexp(A, j[:, None]).astype(np.float32)
    C1 = _gpu(A, W, form)
    C2 = _gpu(A2, W, form)
    assert np.array_equal(np.ldexp(C1, j[:, None]).astype(np.float32), C2)


@pytest.mark.parametrize("label,M,K,N,form", PATHS)
def test_gemm_mixed_scales(label, M, K, N, form):
    """Rows of very different scales in one call (10^-12 .. 10^6), and rows whose
    channels span many decades (half the channels at 10^-6 of the rest)."""
    print(f"mixed scales {label} M={M}", flush=True)
    A, W = _operands(M, K, N, 1.0, seed=9600 + M)
    g = WL.rng(9601 + M)
    row_scale = 10.0 ** g.uniform(-12, 6, size=M)
    A = (A.astype(np.float64) * row_scale[:, None]).astype(np.float32)
    wide = g.random(M) < 0.5
    cols = g.random(K) < 0.5
    A[np.ix_(wide, cols)] *= np.float32(1e-6)
    Wref = W.astype(np.float16).astype(np.float32) if form in ("fp16", "packed16") else W
    C = _gpu(A, W, form)
    _check(C, A, Wref, _rows(M), "mixed")


@pytest.mark.parametrize("M,K", [(8, 512), (300, 200), (300, 512)])
@pytest.mark.parametrize("sigma", [1e-4, 1e-12, 1e5])
def test_qkv_projection_at_every_activation_scale(M, K, sigma):
    """The Q/K/V projection (decode path, the fused INT16 epilogue, the two-pass
    k-split form): each dequantized value is within half a step of its row's
    scale plus the GEMM tolerance of the binary64 product, at any scale."""
    Hq, Hkv, D = 4, 2, 128
    H = Hq + 2 * Hkv
    print(f"qkv scale M={M} K={K} sigma={sigma:g}", flush=True)
    A, W = _operands(M, K, H * D, sigma, seed=9700 + M + K)
    slots = np.arange(M, dtype=np.int64)
    kc = torch.zeros((M, Hkv, D), dtype=torch.int16, device=DEV)
    vc = torch.zeros_like(kc)
    ks = torch.zeros((M, Hkv), dtype=torch.float32, device=DEV)
    vs = torch.zeros_like(ks)
    qc, qs = heal.heal_qkv_proj_quant_i16(torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV), Hq, Hkv, D,
                                          torch.from_numpy(slots).to(DEV), kc, ks, vc, vs)
    codes = np.concatenate([qc.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy()], axis=1).astype(np.float64)
    scales = np.concatenate([qs.cpu().numpy(), ks.cpu().numpy(), vs.cpu().numpy()], axis=1).astype(np.float64)
    deq = codes * scales[:, :, None]
    C64 = oracle.gemm_f64(A, W).reshape(M, H, D)
    C32 = oracle.gemm_f32_naive(A, W)
    e_naive = gemm_normwise_error(C32, C64.reshape(M, H * D), A, W)
    tol = gemm_tolerance(e_naive, K)
    norm_a = np.linalg.norm(A.astype(np.float64), axis=1)[:, None, None]
    norm_b = np.linalg.norm(W.astype(np.float64), axis=1).reshape(1, H, D)
    bar = scales[:, :, None] / 2 * (1 + 2.0 ** -6) + tol * norm_a * norm_b
    assert np.all(np.abs(deq - C64) <= bar)
