"""heal_gemm_f32c_noalloc: the decode-path GEMM with the library's own scratch
memory, called through the C ABI, against heal_gemm_f32c with a workspace.

The kernels are the same, so the outputs must be equal bit for bit: two calls
in a row, the second on a smaller input (the scratch keeps the first call's
contents), for fp32, binary16 and packed weights and a shape with split planes.
"""
import ctypes

import numpy as np
import pytest
import torch

import error_compensated_gemm_heal_amd as heal
import heal_workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _noalloc(A, W, f16=False):
    M, K = A.shape
    if isinstance(W, heal.PackedOperand):
        N, wbuf, ldw, flags = W.rows, W.buf, 0, heal.HEAL_W_PACKED | (heal.HEAL_W_F16 if W.f16 else 0)
    else:
        N, wbuf, ldw, flags = W.shape[0], W, K, heal.HEAL_W_F16 if f16 else 0
    C = torch.full((M, N), float("nan"), device=DEV)
    st = heal.lib().heal_gemm_f32c_noalloc(ctypes.c_void_p(A.data_ptr()), K, ctypes.c_void_p(wbuf.data_ptr()), ldw,
                                           ctypes.c_void_p(C.data_ptr()), N, M, N, K, flags, None, None,
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, heal.heal_status_str(st)
    return C


@pytest.mark.parametrize("form", ["fp32", "fp16", "packed"])
def test_noalloc_equals_workspace_entry_point_two_calls(form):
    f16 = form == "fp16"
    for (M, K, N, seed) in [(64, 14336, 4096, 11), (40, 4096, 1024, 12), (5, 1000, 300, 13)]:
        print(f"noalloc M={M} K={K} N={N} {form}", flush=True)
        A, W = WL.decode_gemm(M, K, N, seed=seed)
        Ad = torch.from_numpy(A).to(DEV)
        Wd = torch.from_numpy(W.astype(np.float16) if f16 else W).to(DEV)
        if form == "packed":
            Wd = heal.heal_pack_w(Wd)
        ref = heal.heal_gemm_f32c(Ad, Wd).cpu().numpy()
        got = _noalloc(Ad, Wd, f16).cpu().numpy()
        torch.cuda.synchronize()
        assert np.array_equal(ref, got)


def test_noalloc_binding_and_limits():
    A, W = WL.decode_gemm(8, 512, 256, seed=14)
    Ad, Wd = torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV)
    C = torch.empty((8, 256), device=DEV)
    heal.heal_gemm_f32c_noalloc(Ad, Wd, C)
    assert np.array_equal(C.cpu().numpy(), heal.heal_gemm_f32c(Ad, Wd).cpu().numpy())


@pytest.mark.parametrize("M,K,N,form", [(8, 4096, 1024, "fp32"), (40, 4096, 4096, "fp32"),
                                        (64, 14336, 4096, "packed"), (1, 4096, 14336, "fp16"),
                                        (8, 4096, 4096, "fp32")])   # the last: k chunks as waves
def test_noalloc_graph_replays(M, K, N, form):
    """Captured once in a HIP graph and replayed with new activations (copied into
    the captured input between replays): every replay equals the workspace entry
    point's eager result, bit for bit.  The split-K counters are left zero by each
    call, so each replay starts from the state the capture saw."""
    print(f"noalloc graph M={M} K={K} N={N} {form}", flush=True)
    A0, W = WL.decode_gemm(M, K, N, seed=20 + M)
    Wd = torch.from_numpy(W.astype(np.float16) if form == "fp16" else W).to(DEV)
    if form == "packed":
        Wd = heal.heal_pack_w(Wd)
    Ad = torch.from_numpy(A0).to(DEV)
    C = torch.full((M, N), float("nan"), device=DEV)
    heal.heal_gemm_f32c_noalloc(Ad, Wd, C)          # eager first call: the scratch array's address
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        heal.heal_gemm_f32c_noalloc(Ad, Wd, C)
    for r in range(3):
        Ar, _ = WL.decode_gemm(M, K, N, seed=30 + 7 * r + M)
        Ad.copy_(torch.from_numpy(Ar).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        ref = heal.heal_gemm_f32c(Ad, Wd).cpu().numpy()
        torch.cuda.synchronize()
        assert np.array_equal(got, ref), r
