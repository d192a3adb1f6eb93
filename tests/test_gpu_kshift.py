"""Per-channel power-of-two rescaling of massive activations (a_kshift).

Activation channels beyond FP16's range (|x| > 65504) make the split's high
part infinite.  With shifts from heal_kshift_from_absmax, the library
multiplies channel k of A by 2^-s_k inside its split, and the weight holds
row k multiplied by 2^+s_k (heal_scale_k, once).  Powers of two are exact, so
the product is unchanged and must meet the same tolerance against the
binary64 oracle of the unscaled A.B; and the result is bit for bit the one of
the activation scaled beforehand (host, exact).
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


def _case(M, K, N, seed):
    A, W = WL.overflow_gemm(M, K, N, seed)
    ks = heal.heal_kshift_from_absmax(np.abs(A).max(axis=0), 32768.0)
    assert ks.max() > 0 and np.abs(A).max() > 65504.0
    return A, W, ks


def _pow2(ks):
    return np.exp2(ks.astype(np.float64))


@pytest.mark.parametrize("M", [1, 8, 16, 17, 64, 300])
def test_kshift_gemm_within_tolerance_and_no_overflow(M):
    """Decode (in-kernel split, split pass) and prefill paths: with the shifts the
    range flag stays clear and the result meets the tolerance.  Without them the
    row normalization alone brings the rows into FP16's range: no flag either,
    and the tolerance holds too (the shifts keep more bits of the ordinary
    channels of those rows)."""
    K, N = 1024, 384
    print(f"kshift gemm M={M} K={K} N={N}", flush=True)
    A, W, ks = _case(M, K, N, seed=7000 + M)
    Ws = (W.astype(np.float64) * _pow2(ks)[None, :]).astype(np.float32)     # exact
    Ad, Wsd = torch.from_numpy(A).to(DEV), torch.from_numpy(Ws).to(DEV)
    ksd = torch.from_numpy(ks).to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = heal.heal_gemm_f32c(Ad, Wsd, a_kshift=ksd, dev_status=st).cpu().numpy()
    assert st.item() == 0
    assert np.all(np.isfinite(C))
    st0 = torch.zeros(1, dtype=torch.int32, device=DEV)
    C0 = heal.heal_gemm_f32c(Ad, torch.from_numpy(W).to(DEV), dev_status=st0).cpu().numpy()
    assert st0.item() == 0
    rows = np.arange(M) if M <= 64 else np.sort(WL.rng(M).choice(M, size=24, replace=False))
    C64 = oracle.gemm_f64_rows(A, W, rows)
    C32 = oracle.gemm_f32_naive_rows(A, W, rows)
    e_naive = gemm_normwise_error(C32, C64, A, W, rows=rows)
    for label, Cx in (("shifted", C), ("unshifted", C0)):
        e_gpu = gemm_normwise_error(Cx[rows], C64, A, W, rows=rows)
        print(f"  {label}: e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
        assert e_gpu <= gemm_tolerance(e_naive, K)


@pytest.mark.parametrize("M", [1, 16, 17, 64, 200])
def test_kshift_bit_equal_to_prescaled_activation(M):
    """The shift is applied exactly before the split: the same bits as the GEMM of
    A * 2^-s (scaled on the host) without shifts, on every path."""
    K, N = 640, 200
    A, W, ks = _case(M, K, N, seed=7100 + M)
    As = (A.astype(np.float64) / _pow2(ks)[None, :]).astype(np.float32)     # exact
    Ws = (W.astype(np.float64) * _pow2(ks)[None, :]).astype(np.float32)
    Wsd = torch.from_numpy(Ws).to(DEV)
    c1 = heal.heal_gemm_f32c(torch.from_numpy(A).to(DEV), Wsd, a_kshift=torch.from_numpy(ks).to(DEV)).cpu().numpy()
    c2 = heal.heal_gemm_f32c(torch.from_numpy(As).to(DEV), Wsd).cpu().numpy()
    assert np.array_equal(c1, c2)


def test_kshift_packed_activation_and_weight():
    """heal_pack_w takes the same shifts: an activation packed with them, and a
    weight packed with the negated shifts from the unscaled W, give the bits of
    the unpacked call."""
    M, K, N = 300, 1000, 260
    A, W, ks = _case(M, K, N, seed=7200)
    Ws = (W.astype(np.float64) * _pow2(ks)[None, :]).astype(np.float32)
    Ad, ksd = torch.from_numpy(A).to(DEV), torch.from_numpy(ks).to(DEV)
    ref = heal.heal_gemm_f32c(Ad, torch.from_numpy(Ws).to(DEV), a_kshift=ksd).cpu().numpy()
    Ap = heal.heal_pack_w(Ad, kshift=ksd)
    Wp = heal.heal_pack_w(torch.from_numpy(W).to(DEV), kshift=-ksd)
    got = heal.heal_gemm_f32c(Ap, Wp).cpu().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M", [1, 8, 17, 40, 64])
def test_kshift_decode_packed_weight(M):
    """Decode kernel on a weight packed once with the negated shifts: the shifted
    call equals, bit for bit, the call on the host-prescaled activation with the
    same packed weight (in-kernel split and split-pass forms), and meets the
    tolerance against the binary64 product of the unscaled operands."""
    K, N = 1000, 320
    print(f"kshift decode packed M={M}", flush=True)
    A, W, ks = _case(M, K, N, seed=7500 + M)
    ksd = torch.from_numpy(ks).to(DEV)
    Wp = heal.heal_pack_w(torch.from_numpy(W).to(DEV), kshift=-ksd)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    c1 = heal.heal_gemm_f32c(torch.from_numpy(A).to(DEV), Wp, a_kshift=ksd, dev_status=st).cpu().numpy()
    assert st.item() == 0
    As = (A.astype(np.float64) / _pow2(ks)[None, :]).astype(np.float32)
    c2 = heal.heal_gemm_f32c(torch.from_numpy(As).to(DEV), Wp).cpu().numpy()
    assert np.array_equal(c1, c2)
    rows = np.arange(M)
    C64 = oracle.gemm_f64_rows(A, W, rows)
    C32 = oracle.gemm_f32_naive_rows(A, W, rows)
    e_gpu = gemm_normwise_error(c1, C64, A, W, rows=rows)
    e_naive = gemm_normwise_error(C32, C64, A, W, rows=rows)
    assert e_gpu <= gemm_tolerance(e_naive, K)


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_scale_k_exact(dtype, layout):
    """heal_scale_k multiplies reduction index k by 2^-s exactly, out of place and in place."""
    K, rows = 300, 70
    g = WL.rng(7300)
    X = WL.normal(g, (rows, K) if layout == "nk" else (K, rows), std=0.02).astype(dtype)
    s = g.integers(-6, 7, size=K).astype(np.int8)
    f = np.exp2(-s.astype(np.float64))
    want = (X.astype(np.float64) * (f[None, :] if layout == "nk" else f[:, None])).astype(dtype)
    Xd = torch.from_numpy(X).to(DEV)
    sd = torch.from_numpy(s).to(DEV)
    out = heal.heal_scale_k(Xd, sd, layout).cpu().numpy()
    assert np.array_equal(out.view(np.uint16 if dtype == np.float16 else np.uint32),
                          want.view(np.uint16 if dtype == np.float16 else np.uint32))
    heal.heal_scale_k(Xd, sd, layout, out=Xd)
    assert np.array_equal(Xd.cpu().numpy(), want)


@pytest.mark.parametrize("M", [1, 64])
def test_kshift_fp16_weight(M):
    """Two-product form with a rescaled binary16 weight: the shifted call equals the
    call on the host-prescaled activation, and meets the tolerance."""
    K, N = 1024, 256
    A, W, ks = _case(M, K, N, seed=7400 + M)
    W16 = W.astype(np.float16)
    W16d = torch.from_numpy(W16).to(DEV)
    ksd = torch.from_numpy(ks).to(DEV)
    W16s = heal.heal_scale_k(W16d, -ksd)
    c1 = heal.heal_gemm_f32c(torch.from_numpy(A).to(DEV), W16s, a_kshift=ksd).cpu().numpy()
    As = (A.astype(np.float64) / _pow2(ks)[None, :]).astype(np.float32)
    c2 = heal.heal_gemm_f32c(torch.from_numpy(As).to(DEV), W16s).cpu().numpy()
    assert np.array_equal(c1, c2)
    W32 = W16.astype(np.float32)
    rows = np.arange(M)
    C64 = oracle.gemm_f64_rows(A, W32, rows)
    C32 = oracle.gemm_f32_naive_rows(A, W32, rows)
    e_gpu = gemm_normwise_error(c1, C64, A, W32, rows=rows)
    e_naive = gemm_normwise_error(C32, C64, A, W32, rows=rows)
    assert e_gpu <= gemm_tolerance(e_naive, K)
