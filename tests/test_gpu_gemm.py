"""GPU parity of the compensated GEMM against the CPU oracle.

Tolerance (normwise, see tests/metrics.py): at most 2x the error of a naive
FP32 GEMM against the binary64 reference, and at most 1e-5.  Exact cases
(binary16-representable operands with exact partial sums) must match the
binary64 reference bit for bit.
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


def _run(A, W, w_layout="nk", packed=False, C=None):
    Ad = torch.from_numpy(A).to(DEV)
    Wd = torch.from_numpy(W).to(DEV)
    if packed:
        Wd = heal.heal_pack_w(Wd, w_layout)
    out = heal.heal_gemm_f32c(Ad, Wd, w_layout=w_layout, C=C)
    torch.cuda.synchronize()
    return out


def _check(A, W, w_layout="nk", packed=False, rows=None, label=""):
    print(f"gemm {label} M={A.shape[0]} K={A.shape[1]} W={W.shape} {w_layout} packed={packed}", flush=True)
    C = _run(A, W, w_layout, packed).cpu().numpy()
    K = A.shape[1]
    if rows is None:
        C64 = oracle.gemm_f64(A, W, w_layout)
        C32 = oracle.gemm_f32_naive(A, W, w_layout)
        Cg = C
    else:
        C64 = oracle.gemm_f64_rows(A, W, rows, w_layout)
        C32 = oracle.gemm_f32_naive_rows(A, W, rows, w_layout)
        Cg = C[rows]
    e_gpu = gemm_normwise_error(Cg, C64, A, W, w_layout, rows)
    e_naive = gemm_normwise_error(C32, C64, A, W, w_layout, rows)
    bar = gemm_tolerance(e_naive, K)
    print(f"   e_gpu={e_gpu:.3e} e_naive={e_naive:.3e} ratio={e_gpu / max(e_naive, 1e-300):.3f}", flush=True)
    assert np.all(np.isfinite(Cg))
    assert e_gpu <= bar, (e_gpu, e_naive)
    return C


def test_gemm_smoke_case():
    A, W = WL.smoke_gemm()
    _check(A, W, label="smoke 16x256x256")


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (2, 33, 1), (17, 40, 31), (64, 100, 300), (65, 129, 33),
                                   (300, 200, 100), (257, 300, 1000), (513, 257, 129)])
@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_gemm_ragged_shapes(M, N, K, layout):
    g = WL.rng(M * 7 + N * 3 + K)
    A = WL.normal(g, (M, K))
    W = WL.normal(g, (N, K) if layout == "nk" else (K, N), std=0.02)
    _check(A, W, layout, label="ragged")


@pytest.mark.parametrize("M", [1, 8, 64, 200])
def test_gemm_packed_weight(M):
    A, W = WL.decode_gemm(M, 1024, 384, seed=77 + M)
    _check(A, W, "nk", packed=True, label="packed")


@pytest.mark.parametrize("M", [5, 300])
def test_gemm_packed_activation_reused(M):
    """One activation split once (HEAL_A_PACKED) feeding two GEMMs equals the unpacked calls."""
    g = WL.rng(900 + M)
    A = WL.normal(g, (M, 700))
    W1 = WL.normal(g, (130, 700), std=0.02)
    W2 = WL.normal(g, (64, 700), std=0.02)
    Ad = torch.from_numpy(A).to(DEV)
    Ap = heal.heal_pack_w(Ad)
    for W in (W1, W2):
        Wd = torch.from_numpy(W).to(DEV)
        Wp = heal.heal_pack_w(Wd)
        c1 = heal.heal_gemm_f32c(Ap, Wp).cpu().numpy()
        c2 = heal.heal_gemm_f32c(Ap, Wd).cpu().numpy()
        c3 = heal.heal_gemm_f32c(Ad, Wp).cpu().numpy()
        assert np.array_equal(c1, c2)
        if M > 64:       # an unpacked A of <= 64 rows takes the decode kernel
            assert np.array_equal(c1, c3)
        e32 = gemm_normwise_error(oracle.gemm_f32_naive(A, W), oracle.gemm_f64(A, W), A, W)
        for c in (c1, c3):
            assert gemm_normwise_error(c, oracle.gemm_f64(A, W), A, W) <= gemm_tolerance(e32, 700)


def test_gemm_strided_operands():
    g = WL.rng(5)
    A_big = WL.normal(g, (40, 520))
    W_big = WL.normal(g, (72, 516), std=0.02)
    A, W = A_big[:, :500], W_big[:, :500]          # lda = 520, ldw = 516
    Ad = torch.from_numpy(A_big).to(DEV)[:, :500]
    Wd = torch.from_numpy(W_big).to(DEV)[:, :500]
    Cbig = torch.full((40, 80), float("nan"), device=DEV)
    heal.heal_gemm_f32c(Ad, Wd, C=Cbig[:, :72])
    torch.cuda.synchronize()
    C = Cbig.cpu().numpy()
    assert np.all(np.isnan(C[:, 72:]))            # nothing written outside the view
    e = gemm_normwise_error(C[:, :72], oracle.gemm_f64(A, W), A, W)
    e32 = gemm_normwise_error(oracle.gemm_f32_naive(A, W), oracle.gemm_f64(A, W), A, W)
    assert e <= gemm_tolerance(e32, 500)


@pytest.mark.parametrize("M,K", [(16, 256), (100, 256), (64, 40)])
def test_gemm_exact_on_binary16_operands(M, K):
    g = WL.rng(M + K)
    A = (g.integers(-8, 9, size=(M, K)) / 8.0).astype(np.float32)
    W = (g.integers(-8, 9, size=(96, K)) / 8.0).astype(np.float32)
    C = _run(A, W).cpu().numpy()
    assert np.array_equal(C.astype(np.float64), oracle.gemm_f64(A, W))


def test_gemm_k_zero_and_empty():
    A = torch.zeros((5, 0), device=DEV)
    W = torch.zeros((7, 0), device=DEV)
    C = torch.full((5, 7), 3.0, device=DEV)
    heal.heal_gemm_f32c(A, W, C=C)
    assert torch.all(C == 0).item()
    out = heal.heal_gemm_f32c(torch.zeros((0, 8), device=DEV), torch.zeros((4, 8), device=DEV))
    assert out.shape == (0, 4)


@pytest.mark.parametrize("M", [4, 40, 100])
def test_gemm_activation_past_fp16_range_is_normalized(M):
    """An activation beyond 65504 is brought into FP16's range with its row (decode
    in-kernel split, split planes, prefill): no flag, and the tolerance holds."""
    g = WL.rng(60 + M)
    A = WL.normal(g, (M, 64))
    A[2, 5] = 70000.0
    A[M - 1, 7] = -3.0e9
    W = WL.normal(g, (8, 64), std=0.02)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = heal.heal_gemm_f32c(torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV), dev_status=st).cpu().numpy()
    assert st.item() == 0
    e = gemm_normwise_error(C, oracle.gemm_f64(A, W), A, W)
    e32 = gemm_normwise_error(oracle.gemm_f32_naive(A, W), oracle.gemm_f64(A, W), A, W)
    assert e <= gemm_tolerance(e32, 64)


def test_gemm_range_flag_on_streamed_weight():
    """The decode path splits an fp32 weight as it streams it, unnormalized: an
    element at or past 65520 has an infinite fp16 high part and sets the flag."""
    A = np.ones((4, 64), np.float32)
    W = np.ones((8, 64), np.float32)
    W[3, 9] = 70000.0
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    heal.heal_gemm_f32c(torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV), dev_status=st)
    assert st.item() == heal.HEAL_FLAG_F16_RANGE


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("K,N", WL.LLAMA3_8B_DECODE_KN)
def test_gemm_decode_shapes_and_batch_invariance(K, N, packed):
    """Decode-shaped Llama-3-8B-like layers, M = 1, 8, 32, 64, fp32 weight streamed
    or packed once: tolerance on every M, and row i of the product identical for
    every M (fixed K chunking; M = 16 and 17 straddle the switch from the
    in-kernel activation split to the pre-split copy)."""
    print(f"decode K={K} N={N} packed={packed}", flush=True)
    A, W = WL.decode_gemm(64, K, N, seed=2000 + K + N)
    Wd = torch.from_numpy(W).to(DEV)
    if packed:
        Wd = heal.heal_pack_w(Wd)
    Ad = torch.from_numpy(A).to(DEV)
    outs = {}
    Ms = sorted(set(WL.DECODE_M) | {16, 17})
    for M in Ms:
        outs[M] = heal.heal_gemm_f32c(Ad[:M], Wd).cpu().numpy()
    for M in Ms:
        assert np.array_equal(outs[M], outs[64][:M]), M
    rows = np.arange(64)            # every row of the M = 64 call against the oracle
    C64 = oracle.gemm_f64_rows(A, W, rows)
    C32 = oracle.gemm_f32_naive_rows(A, W, rows)
    e_gpu = gemm_normwise_error(outs[64][rows], C64, A, W, rows=rows)
    e_naive = gemm_normwise_error(C32, C64, A, W, rows=rows)
    print(f"decode K={K} N={N}: e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert e_gpu <= gemm_tolerance(e_naive, K)


@pytest.mark.parametrize("K,N", [(2048, 4100), (2000, 4100), (4096, 4096)])
@pytest.mark.parametrize("wkind", ["fp32", "f16", "packed", "kshift"])
def test_gemm_decode_chunks_as_waves(K, N, wkind):
    """M <= 16 with short k chunks (at most 4 blocks of 128) over at least 256 slices
    of 16 rows: the chunks are the waves of one workgroup and meet in LDS.  Every M
    gives the rows of the M = 17 call (chunks completed through memory) bit for bit,
    the allocation-free entry point gives the same bits, and the M = 16 result meets
    the tolerance on every row (ragged N; K = 2000 loads W element by element)."""
    print(f"decode chunks as waves K={K} N={N} {wkind}", flush=True)
    A, W = WL.decode_gemm(17, K, N, seed=2200 + K + N)
    ks = None
    if wkind == "kshift":     # two channels past FP16's range, rescaled per channel
        A[:, 3] *= 3.0e5
        A[:, K - 1] *= -7.0e5
        ks = np.zeros(K, np.int8)
        ks[3], ks[K - 1] = 6, 6
        W = W * np.exp2(ks.astype(np.float32))[None, :]
    if wkind == "f16":
        W = W.astype(np.float16)
    Ad, Wd = torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV)
    Wop = heal.heal_pack_w(Wd) if wkind == "packed" else Wd
    ksd = None if ks is None else torch.from_numpy(ks).to(DEV)
    outs = {M: heal.heal_gemm_f32c(Ad[:M], Wop, a_kshift=ksd).cpu().numpy() for M in (1, 3, 8, 16, 17)}
    for M in outs:
        assert np.array_equal(outs[M], outs[17][:M]), M
    C = torch.empty(16, N, dtype=torch.float32, device=DEV)
    heal.heal_gemm_f32c_noalloc(Ad[:16], Wop, C, a_kshift=ksd)
    assert np.array_equal(C.cpu().numpy(), outs[16])
    W64 = W.astype(np.float32)
    A16 = A[:16]
    if ks is not None:        # the product the rescaled operands stand for
        A16 = (A16.astype(np.float64) * np.exp2(-ks.astype(np.float64))[None, :]).astype(np.float32)
    rows = np.arange(16)
    C64 = oracle.gemm_f64_rows(A16, W64, rows)
    C32 = oracle.gemm_f32_naive_rows(A16, W64, rows)
    e_gpu = gemm_normwise_error(outs[16], C64, A16, W64, rows=rows)
    e_naive = gemm_normwise_error(C32, C64, A16, W64, rows=rows)
    print(f"  e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert e_gpu <= gemm_tolerance(e_naive, K)


@pytest.mark.parametrize("K,N", [(8192, 4096), (16384, 4096)])
def test_gemm_decode_aligned_long_rows(K, N):
    """Weight rows a multiple of 32 KiB apart, read in 8 chunks of 8 or more k
    blocks each: the rotated k order is on.  Tolerance on every row of the
    M = 64 call, and each row identical for every M."""
    print(f"decode aligned rows K={K} N={N}", flush=True)
    A, W = WL.decode_gemm(64, K, N, seed=2100 + K)
    Ad, Wd = torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV)
    outs = {M: heal.heal_gemm_f32c(Ad[:M], Wd).cpu().numpy() for M in (1, 8, 17, 64)}
    for M in outs:
        assert np.array_equal(outs[M], outs[64][:M]), M
    rows = np.arange(64)
    C64 = oracle.gemm_f64_rows(A, W, rows)
    e_gpu = gemm_normwise_error(outs[64], C64, A, W, rows=rows)
    e_naive = gemm_normwise_error(oracle.gemm_f32_naive_rows(A, W, rows), C64, A, W, rows=rows)
    print(f"decode aligned rows K={K}: e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert e_gpu <= gemm_tolerance(e_naive, K)


@pytest.mark.parametrize("M,N,K", [(1, 384, 1024), (8, 300, 1000), (40, 260, 700), (64, 512, 4096),
                                   (300, 384, 1024)])
@pytest.mark.parametrize("f16", [False, True])
def test_gemm_packed_weight_row_scaling_is_exact(M, N, K, f16):
    """A packed fp32 weight is normalized per row: rows of W scaled by 2^j (j from
    -40 to 40, per row) give the columns of C scaled by 2^j, bit for bit (decode
    kernel for M <= 64, prefill otherwise).  A packed binary16 weight keeps its
    values: its two-product result meets the tolerance."""
    print(f"packed weight scaling M={M} N={N} K={K} f16={f16}", flush=True)
    A, W = WL.decode_gemm(M, K, N, seed=2600 + M + K)
    Ad = torch.from_numpy(A).to(DEV)
    if f16:
        W16 = W.astype(np.float16)
        C = heal.heal_gemm_f32c(Ad, heal.heal_pack_w(torch.from_numpy(W16).to(DEV))).cpu().numpy()
        W32 = W16.astype(np.float32)
        e_gpu = gemm_normwise_error(C, oracle.gemm_f64(A, W32), A, W32)
        e_naive = gemm_normwise_error(oracle.gemm_f32_naive(A, W32), oracle.gemm_f64(A, W32), A, W32)
        assert e_gpu <= gemm_tolerance(e_naive, K)
        return
    j = WL.rng(2601 + N).integers(-40, 41, size=N)
    W2 = np.ldexp(W, j[:, None]).astype(np.float32)
    C1 = heal.heal_gemm_f32c(Ad, heal.heal_pack_w(torch.from_numpy(W).to(DEV))).cpu().numpy()
    C2 = heal.heal_gemm_f32c(Ad, heal.heal_pack_w(torch.from_numpy(W2).to(DEV))).cpu().numpy()
    assert np.array_equal(np.ldexp(C1, j[None, :]).astype(np.float32), C2)
    e_gpu = gemm_normwise_error(C1, oracle.gemm_f64(A, W), A, W)
    e_naive = gemm_normwise_error(oracle.gemm_f32_naive(A, W), oracle.gemm_f64(A, W), A, W)
    assert e_gpu <= gemm_tolerance(e_naive, K)


@pytest.mark.parametrize("K,N", WL.PREFILL_KN)
def test_gemm_prefill_full_size_sampled_rows(K, N):
    """Prefill shape M = 2048 with massive-activation channels, packed weight as
    the benchmark times it; 256 sampled rows (all N columns) against the oracle."""
    A, W = WL.prefill_gemm(WL.PREFILL_M, K, N, seed=3000 + K)
    rows = np.sort(WL.rng(K).choice(WL.PREFILL_M, size=256, replace=False))
    _check(A, W, "nk", packed=True, rows=rows, label="prefill")


# ---- the packed operand layout -------------------------------------------------------------

def unpack(buf, R, K, hi_only=False):
    """Read a heal_pack_w buffer (test code): rows padded to 256, k to 32; per row
    and 32-wide k block 32 hi then 32 residual fp16 (hi parts alone in the
    hi-only form), each row followed by 256 unused bytes; then one int32
    exponent per padded row.  Returns (hi, res, e) for the R real rows, k padded."""
    Rp, Kp = -(-R // 256) * 256, -(-K // 32) * 32
    planes = 1 if hi_only else 2
    rb = Kp * 2 * planes + 256                       # bytes per packed row
    rows = buf[: Rp * rb].reshape(Rp, rb)[:, : Kp * 2 * planes]
    data = np.frombuffer(rows.tobytes(), np.uint16).reshape(Rp, Kp // 32, planes, 32)
    e = np.frombuffer(buf[Rp * rb: Rp * rb + Rp * 4].tobytes(), np.int32)
    hi = data[:, :, 0, :].reshape(Rp, Kp)
    res = data[:, :, 1, :].reshape(Rp, Kp) if not hi_only else np.zeros_like(hi)
    assert not hi[R:].any() and not res[R:].any() and not e[R:].any()      # zero padding rows
    assert not hi[:, K:].any() and not res[:, K:].any()                    # zero padding k
    return hi[:R], res[:R], e[:R]


@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("R,K,sigma", [(1, 7, 1.0), (300, 1000, 1e-6), (100, 4096, 3e4), (257, 14336, 1.0),
                                       (64, 20000, 1e-3)])
def test_pack_bit_exact_against_oracle(R, K, sigma, layout):
    """heal_pack_w on fp32 values: hi parts, residuals and row exponents equal the
    oracle's split of the normalized rows, bit for bit (the fused one-pass kernel
    for K <= 16384 in the NK layout, the two-pass form otherwise)."""
    print(f"pack R={R} K={K} sigma={sigma:g} {layout}", flush=True)
    g = WL.rng(R + K)
    X = (WL.normal(g, (R, K)) * np.float32(sigma))
    X[:, g.choice(K, size=min(K, 3), replace=False)] *= np.float32(40.0)
    X[R // 2] = 0.0                                   # a zero row: exponent 0
    src = X if layout == "nk" else np.ascontiguousarray(X.T)
    p = heal.heal_pack_w(torch.from_numpy(src).to(DEV), layout)
    h, r, e = unpack(p.buf.cpu().numpy(), R, K)
    oh, orr, oe = oracle.split_rownorm(X)
    assert np.array_equal(e, oe)
    assert np.array_equal(h[:, :K], oh) and np.array_equal(r[:, :K], orr)


# ---- 16-bit weights (HEAL_W_F16): the two-product form -------------------------------------

def _f16_weight(W):
    """Round a weight to binary16 (what an FP16 checkpoint holds); input data, not the method."""
    return W.astype(np.float16)


@pytest.mark.parametrize("K,N", [(4096, 1024), (14336, 4096)])
def test_gemm_f16_weight_decode_equals_fp32_path(K, N):
    """With fp16 weights the residual plane is zero, so the two-product path must give
    bit for bit what the three-product path gives on the same values held in fp32
    (the dropped product adds exact zeros), for every M; and it meets the tolerance."""
    A, W = WL.decode_gemm(64, K, N, seed=5000 + K + N)
    W16 = _f16_weight(W)
    W32 = W16.astype(np.float32)            # the same values, exactly
    Ad = torch.from_numpy(A).to(DEV)
    W16d = torch.from_numpy(W16).to(DEV)
    W32d = torch.from_numpy(W32).to(DEV)
    outs = {}
    for M in WL.DECODE_M:
        c16 = heal.heal_gemm_f32c(Ad[:M], W16d).cpu().numpy()
        c32 = heal.heal_gemm_f32c(Ad[:M], W32d).cpu().numpy()
        assert np.array_equal(c16, c32), M
        outs[M] = c16
    for M in WL.DECODE_M:
        assert np.array_equal(outs[M], outs[64][:M]), M
    rows = np.array([0, 3, 40, 63])
    C64 = oracle.gemm_f64_rows(A, W32, rows)
    C32 = oracle.gemm_f32_naive_rows(A, W32, rows)
    e_gpu = gemm_normwise_error(outs[64][rows], C64, A, W32, rows=rows)
    e_naive = gemm_normwise_error(C32, C64, A, W32, rows=rows)
    print(f"f16 weight K={K} N={N}: e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert e_gpu <= gemm_tolerance(e_naive, K)


@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("M,N,K", [(3, 40, 31), (100, 130, 300), (64, 100, 33)])
def test_gemm_f16_weight_ragged_and_packed(M, N, K, layout):
    """Ragged shapes on both paths and layouts: the fp16 weight gives the same bits as
    its fp32 copy, its packed form is byte-identical to the packed fp32 copy, and the
    result meets the tolerance."""
    print(f"gemm f16 weight M={M} N={N} K={K} {layout}", flush=True)
    A, W = WL.decode_gemm(M, K, N, seed=5100 + M + N + K)
    W16 = _f16_weight(W if layout == "nk" else np.ascontiguousarray(W.T))
    W32 = W16.astype(np.float32)
    Ad = torch.from_numpy(A).to(DEV)
    W16d, W32d = torch.from_numpy(W16).to(DEV), torch.from_numpy(W32).to(DEV)
    c16 = heal.heal_gemm_f32c(Ad, W16d, w_layout=layout).cpu().numpy()
    c32 = heal.heal_gemm_f32c(Ad, W32d, w_layout=layout).cpu().numpy()
    assert np.array_equal(c16, c32)
    p16 = heal.heal_pack_w(W16d, layout)
    p32 = heal.heal_pack_w(W32d, layout)
    torch.cuda.synchronize()
    # the fp16 weight packs its binary16 values alone, not normalized (exponents 0);
    # the fp32 copy packs normalized rows whose residuals are all zero
    Wnk = W32 if layout == "nk" else np.ascontiguousarray(W32.T)
    h16, r16, e16 = unpack(p16.buf.cpu().numpy(), N, K, hi_only=True)
    assert np.array_equal(h16[:, :K], Wnk.astype(np.float16).view(np.uint16)) and not e16.any()
    h32, r32, e32 = unpack(p32.buf.cpu().numpy(), N, K)
    oh, orr, oe = oracle.split_rownorm(Wnk)
    assert np.array_equal(h32[:, :K], oh) and np.array_equal(e32, oe) and not r32.any()
    cp = heal.heal_gemm_f32c(Ad, p16).cpu().numpy()
    if M > 64:   # both through the prefill kernel's two-product form
        assert np.array_equal(cp, c16)
    C64 = oracle.gemm_f64(A, W32, layout)
    C32 = oracle.gemm_f32_naive(A, W32, layout)
    for C in (c16, cp):
        e_gpu = gemm_normwise_error(C, C64, A, W32, layout)
        e_naive = gemm_normwise_error(C32, C64, A, W32, layout)
        assert e_gpu <= gemm_tolerance(e_naive, K), (e_gpu, e_naive)


@pytest.mark.parametrize("M,N,K", [(512, 1024, 4096), (4096, 4096, 256)])
def test_gemm_f16_weight_prefill_two_products(M, N, K):
    """Prefill shapes (the k-split grid and the plain one): with fp16 weights the kernel
    skips the A_hi.B_lo product; its result equals, bit for bit, the three-product
    kernel's on the same values held in fp32 (whose B_lo is zero), packed or not,
    and meets the tolerance on sampled rows."""
    print(f"gemm f16 weight prefill M={M} N={N} K={K}", flush=True)
    A, W = WL.decode_gemm(M, K, N, seed=5200 + M + N + K)
    W16 = _f16_weight(W)
    W32 = W16.astype(np.float32)
    Ad = torch.from_numpy(A).to(DEV)
    W16d, W32d = torch.from_numpy(W16).to(DEV), torch.from_numpy(W32).to(DEV)
    c16 = heal.heal_gemm_f32c(Ad, W16d).cpu().numpy()
    c32 = heal.heal_gemm_f32c(Ad, W32d).cpu().numpy()
    cp = heal.heal_gemm_f32c(Ad, heal.heal_pack_w(W16d)).cpu().numpy()
    assert np.array_equal(c16, c32)
    assert np.array_equal(cp, c16)
    rows = np.array([0, 1, M // 2, M - 1])
    C64 = oracle.gemm_f64_rows(A, W32, rows)
    C32 = oracle.gemm_f32_naive_rows(A, W32, rows)
    e_gpu = gemm_normwise_error(c16[rows], C64, A, W32, rows=rows)
    e_naive = gemm_normwise_error(C32, C64, A, W32, rows=rows)
    print(f"  e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert e_gpu <= gemm_tolerance(e_naive, K)


# ---- one-product mode (plain FP16, HEAL_ONE_PRODUCT) -----------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 384, 1024), (17, 300, 700), (64, 130, 4096), (300, 260, 1000),
                                   (2048, 1024, 512)])
@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_gemm_one_product_against_plain_f16_oracle(M, N, K, layout):
    """Decode and prefill grids: the one-product result against the oracle's exact
    product of the fp16-rounded operands, to the fp32-accumulation bar on those
    operands; and bit-equal to the three-product kernels when the operands are
    binary16 (their correction products are exact zeros)."""
    print(f"gemm one product M={M} N={N} K={K} {layout}", flush=True)
    A, W = WL.decode_gemm(M, K, N, seed=5300 + M + N + K)
    if layout == "kn":
        W = np.ascontiguousarray(W.T)
    Ad, Wd = torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV)
    C = heal.heal_gemm_f32c(Ad, Wd, w_layout=layout, one_product=True).cpu().numpy()
    rows = np.arange(M) if M <= 64 else np.sort(WL.rng(M + K).choice(M, size=24, replace=False))
    C64, C32 = oracle.gemm_f16_plain_rows(A, W, rows, layout)
    Ah, Wh = oracle.round_f16(A), oracle.round_f16(W)
    e_gpu = gemm_normwise_error(C[rows], C64, Ah, Wh, layout, rows)
    e_naive = gemm_normwise_error(C32, C64, Ah, Wh, layout, rows)
    print(f"  e_gpu={e_gpu:.3e} e_naive={e_naive:.3e}", flush=True)
    assert e_gpu <= gemm_tolerance(e_naive, K)
    # binary16 operands: the compensation adds zeros, so one product gives the same bits
    c1 = heal.heal_gemm_f32c(torch.from_numpy(Ah).to(DEV), torch.from_numpy(Wh).to(DEV), w_layout=layout,
                             one_product=True).cpu().numpy()
    c3 = heal.heal_gemm_f32c(torch.from_numpy(Ah).to(DEV), torch.from_numpy(Wh).to(DEV),
                             w_layout=layout).cpu().numpy()
    assert np.array_equal(c1, c3)


def test_gemm_one_product_fp16_and_packed_weight():
    """With an fp16 weight (packed or not) the one-product mode is the plain FP16 GEMM too."""
    M, N, K = 200, 256, 768
    A, W = WL.decode_gemm(M, K, N, seed=5400)
    W16d = torch.from_numpy(W.astype(np.float16)).to(DEV)
    Ad = torch.from_numpy(A).to(DEV)
    c = heal.heal_gemm_f32c(Ad, W16d, one_product=True).cpu().numpy()
    cp = heal.heal_gemm_f32c(Ad, heal.heal_pack_w(W16d), one_product=True).cpu().numpy()
    assert np.array_equal(c, cp)
    rows = np.arange(0, M, 9)
    C64, C32 = oracle.gemm_f16_plain_rows(A, W.astype(np.float16).astype(np.float32), rows)
    Ah, Wh = oracle.round_f16(A), W.astype(np.float16).astype(np.float32)
    e_gpu = gemm_normwise_error(c[rows], C64, Ah, Wh, rows=rows)
    e_naive = gemm_normwise_error(C32, C64, Ah, Wh, rows=rows)
    assert e_gpu <= gemm_tolerance(e_naive, K)
