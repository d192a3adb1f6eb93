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
