"""heal_gemm_f32c and HIP graph capture.

On the decode path with a k split, the workspace entry point marks its
split-K flags with a per-call epoch taken on the host; a captured call would
replay that epoch and read the previous replay's flags as its own.  So under
capture it refuses such shapes (HEAL_ERR_UNSUPPORTED, before any launch), and
heal_gemm_f32c_noalloc is the form to capture.  Shapes without a k split, and
the prefill path, capture and replay normally.
"""
import ctypes

import numpy as np
import pytest
import torch

import error_compensated_gemm_heal_amd as heal
import heal_workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _raw_call(A, W, C, ws):
    M, K = A.shape
    N = W.shape[0]
    return heal.lib().heal_gemm_f32c(ctypes.c_void_p(A.data_ptr()), K, ctypes.c_void_p(W.data_ptr()), K,
                                     ctypes.c_void_p(C.data_ptr()), N, M, N, K, 0, None,
                                     ctypes.c_void_p(ws.data_ptr()), ws.numel(), None,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_capture_refused_with_split_k():
    M, K, N = 8, 4096, 1024
    A, W = WL.decode_gemm(M, K, N, seed=41)
    Ad, Wd = torch.from_numpy(A).to(DEV), torch.from_numpy(W).to(DEV)
    C = torch.empty((M, N), device=DEV)
    ws = torch.empty(heal.heal_gemm_f32c_workspace(M, N, K, 0), dtype=torch.uint8, device=DEV)
    assert _raw_call(Ad, Wd, C, ws) == 0            # eager: fine
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = _raw_call(Ad, Wd, C, ws)
    assert st == 5, heal.heal_status_str(st)        # HEAL_ERR_UNSUPPORTED


@pytest.mark.parametrize("M,K,N", [(4, 256, 192), (300, 512, 384), (8, 4096, 4096), (1, 2048, 4100)])
def test_capture_and_replay_without_split_k(M, K, N):
    """A decode shape with one k chunk, a prefill shape, and decode shapes whose k
    chunks are the waves of one workgroup (no flags in the workspace): replays
    with new activations equal the eager calls, bit for bit."""
    print(f"graph M={M} K={K} N={N}", flush=True)
    A0, W = WL.decode_gemm(M, K, N, seed=42 + M)
    Wd = torch.from_numpy(W).to(DEV)
    Ad = torch.from_numpy(A0).to(DEV)
    C = torch.empty((M, N), device=DEV)
    ws = torch.empty(max(heal.heal_gemm_f32c_workspace(M, N, K, 0), 1), dtype=torch.uint8, device=DEV)
    heal.heal_gemm_f32c(Ad, Wd, C=C, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        heal.heal_gemm_f32c(Ad, Wd, C=C, workspace=ws)
    for r in range(3):
        Ar, _ = WL.decode_gemm(M, K, N, seed=50 + 5 * r + M)
        Ad.copy_(torch.from_numpy(Ar).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        ref = heal.heal_gemm_f32c(Ad, Wd).cpu().numpy()
        assert np.array_equal(got, ref), r
