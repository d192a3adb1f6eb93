"""GPU parity of the BF16 three-way precision mode (HEAL_BF16X3).

The packed operand is compared bit for bit with the oracle's split; GEMM
results are held to the compensated GEMM's bar against the binary64 product
(at most 2x the naive FP32 error and 1e-5, normwise), and to the fp32
accumulation of the oracle's six-product model.  Exact cases (bf16 small
integers with exact partial sums) match the binary64 product bit for bit.
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


def _packed_planes(buf, rows, K):
    """The packed buffer as planes [3, rows, K] of bf16 values (float64): per row
    and 32-wide k block, 32 b0 then 32 b1 then 32 b2 (the documented layout)."""
    Kp = (K + 31) // 32 * 32
    u = buf.cpu().numpy().view(np.uint16)[: ((rows + 255) // 256 * 256) * Kp * 3]
    u = u.reshape(-1, Kp // 32, 3, 32)[:rows]
    f = (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.stack([f[:, :, p, :].reshape(rows, Kp)[:, :K] for p in range(3)]), u


@pytest.mark.parametrize("rows,K,layout", [(1, 1, "nk"), (5, 33, "nk"), (300, 70, "nk"), (257, 100, "kn"),
                                           (64, 512, "kn")])
def test_bf16x3_pack_bit_exact(rows, K, layout):
    print(f"bf16x3 pack rows={rows} K={K} {layout}", flush=True)
    g = WL.rng(rows * 31 + K)
    X = (g.standard_normal((rows, K)) * np.exp2(g.integers(-60, 60, (rows, K)))).astype(np.float32)
    X.flat[:: 7] = 0.0
    src = X if layout == "nk" else np.ascontiguousarray(X.T)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    P = heal.heal_pack_w(torch.from_numpy(src).to(DEV), layout, bf16x3=True, dev_status=st)
    planes, u = _packed_planes(P.buf, rows, K)
    ref = oracle.split_bf16x3(X)
    for p in range(3):
        assert np.array_equal(planes[p], ref[p]), p
    Kp = (K + 31) // 32 * 32
    full = P.buf.cpu().numpy().view(np.uint16).reshape(-1, Kp // 32, 3, 32)
    pad_k = full.reshape(full.shape[0], Kp // 32, 3, 32).transpose(0, 2, 1, 3).reshape(full.shape[0], 3, Kp)[:, :, K:]
    assert not pad_k.any() and not full[rows:].any()     # zero padding in k and in rows
    assert int(st.item()) == 0


def _check(A, W, layout="nk", packed_w=False, packed_a=False, rows=None, label=""):
    print(f"bf16x3 gemm {label} M={A.shape[0]} K={A.shape[1]} W={W.shape} {layout} pw={packed_w} pa={packed_a}",
          flush=True)
    Ad = torch.from_numpy(A).to(DEV)
    Wd = torch.from_numpy(W).to(DEV)
    if packed_w:
        Wd = heal.heal_pack_w(Wd, layout, bf16x3=True)
    if packed_a:
        Ad = heal.heal_pack_w(Ad, "nk", bf16x3=True)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = heal.heal_gemm_f32c(Ad, Wd, w_layout=layout, bf16x3=True, dev_status=st).cpu().numpy()
    K = A.shape[1]
    if rows is None:
        C64 = oracle.gemm_f64(A, W, layout)
        C32 = oracle.gemm_f32_naive(A, W, layout)
        Cm = oracle.gemm_bf16x3_model(A, W, layout)
        Cg = C
    else:
        C64 = oracle.gemm_f64_rows(A, W, rows, layout)
        C32 = oracle.gemm_f32_naive_rows(A, W, rows, layout)
        Cm = oracle.gemm_bf16x3_model(A[rows], W, layout)
        Cg = C[rows]
    e_gpu = gemm_normwise_error(Cg, C64, A, W, layout, rows)
    e_naive = gemm_normwise_error(C32, C64, A, W, layout, rows)
    e_model = gemm_normwise_error(Cg, Cm, A, W, layout, rows)
    print(f"   e_gpu={e_gpu:.3e} e_naive={e_naive:.3e} e_model={e_model:.3e}", flush=True)
    assert np.all(np.isfinite(Cg))
    assert e_gpu <= gemm_tolerance(e_naive, K), (e_gpu, e_naive)
    assert e_model <= 2 * e_naive + 2.0 ** -24, (e_model, e_naive)   # fp32 accumulation of the model
    assert int(st.item()) == 0
    return C


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 40, 31), (64, 100, 300), (65, 129, 33),
                                   (300, 200, 100), (513, 257, 129)])
@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_bf16x3_ragged_shapes(M, N, K, layout):
    g = WL.rng(M * 5 + N * 11 + K)
    A = WL.normal(g, (M, K))
    W = WL.normal(g, (N, K) if layout == "nk" else (K, N), std=0.02)
    _check(A, W, layout, label="ragged")


@pytest.mark.parametrize("M", [1, 64, 300])
def test_bf16x3_packed_operands(M):
    g = WL.rng(600 + M)
    A = WL.normal(g, (M, 777))
    W = WL.normal(g, (190, 777), std=0.02)
    C1 = _check(A, W, packed_w=True, label="packed W")
    C2 = _check(A, W, packed_w=True, packed_a=True, label="packed A and W")
    assert np.array_equal(C1, C2)


def test_bf16x3_exact_on_bf16_integers():
    """bf16 small integers with exact fp32 partial sums: bit-equal to binary64."""
    g = WL.rng(7)
    A = g.integers(-100, 101, (70, 256)).astype(np.float32)
    W = g.integers(-100, 101, (90, 256)).astype(np.float32)
    C = heal.heal_gemm_f32c(torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV), bf16x3=True).cpu().numpy()
    assert np.array_equal(C.astype(np.float64), oracle.gemm_f64(A, W))


def test_bf16x3_values_beyond_fp16_range():
    """Massive activations (0.5% of channels scaled by 2e5) and a wide spread of
    magnitudes: no rescaling needed, no flag, the bar holds."""
    A, W = WL.overflow_gemm(200, 1024, 300, seed=8)
    g = WL.rng(9)
    A = (A * np.exp2(g.integers(-20, 20, A.shape[1]))[None, :]).astype(np.float32)
    assert np.abs(A).max() > 65504
    _check(A, W, label="beyond fp16 range")


def test_bf16x3_flag_on_bf16_overflow():
    A = np.ones((4, 64), np.float32)
    A[1, 3] = np.float32(3.4e38)     # finite in fp32, rounds past bf16's largest value
    W = np.ones((8, 64), np.float32)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    heal.heal_gemm_f32c(torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV), bf16x3=True, dev_status=st)
    assert int(st.item()) & heal.HEAL_FLAG_F16_RANGE


@pytest.mark.parametrize("N,K", [(14336, 4096), (4096, 14336)])
def test_bf16x3_full_prefill_shapes_sampled_rows(N, K):
    """The measured prefill shapes (both grid forms: plain and k-split), sampled rows."""
    A, W = WL.prefill_gemm(WL.PREFILL_M, K, N, seed=40 + N)
    rows = np.sort(WL.rng(N).choice(A.shape[0], 6, replace=False))
    _check(A, W, packed_w=True, rows=rows, label="prefill")
