"""Host-side checks of the C ABI (no GPU needed).

* libheal.so loads and exports every entry point declared in include/heal.h;
* the binding declares a signature for each of them;
* argument validation returns the documented HEAL_ERR_* code before any HIP
  call (pointers below are never dereferenced: every case fails validation or
  is a documented no-op);
* workspace-size queries are pure host arithmetic.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import error_compensated_gemm_heal_amd as heal

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "heal.h")

OK, NULL, SHAPE, STRIDE, ALIGN, UNSUP, WS = 0, 1, 2, 3, 4, 5, 6
FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x10004)    # 4-byte aligned only
NULLP = None


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(heal_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported_and_bound():
    L = heal.lib()
    syms = declared_symbols()
    assert len(syms) >= 11
    for s in syms:
        assert hasattr(L, s), s
        assert s in heal.SIGNATURES, s


def test_status_strings_and_version():
    for code in range(8):
        assert heal.heal_status_str(code).startswith("HEAL")
    assert heal.heal_version() >> 16 == 1 and (heal.heal_version() >> 8) & 0xff >= 1


def test_split_validation():
    L = heal.lib()
    assert L.heal_split_f32(FAKE, -1, FAKE, FAKE, None, None) == SHAPE
    assert L.heal_split_f32(NULLP, 0, NULLP, NULLP, None, None) == OK
    assert L.heal_split_f32(NULLP, 8, FAKE, FAKE, None, None) == NULL
    assert L.heal_split_f32(FAKE_ODD, 8, FAKE, FAKE, None, None) == ALIGN
    assert L.heal_split_f32(FAKE, 8, ctypes.c_void_p(0x10002), FAKE, None, None) == ALIGN


def _gemm(A=FAKE, lda=4096, W=FAKE, ldw=4096, C=FAKE, ldc=4096, M=8, N=4096, K=4096, flags=0, ws=FAKE,
          wsb=1 << 30, st=None, ks=None):
    return heal.lib().heal_gemm_f32c(A, lda, W, ldw, C, ldc, M, N, K, flags, ks, ws, wsb, st, None)


def test_gemm_validation():
    assert _gemm(M=-1) == SHAPE
    assert _gemm(K=1 << 31) == SHAPE
    # launches past the 32-bit grid size (in threads): prefill tiles, then decode row groups
    assert _gemm(M=1 << 20, N=1 << 20, K=64, lda=64, ldw=64, ldc=1 << 20) == UNSUP
    assert _gemm(M=1, N=1 << 30, K=64, lda=64, ldw=64, ldc=1 << 30) == UNSUP
    assert _gemm(flags=heal.HEAL_W_F16 | heal.HEAL_W_PACKED, W=ctypes.c_void_p(0x10010)) == ALIGN  # packed: 256 B
    assert _gemm(flags=64) == UNSUP
    X3 = heal.HEAL_BF16X3
    assert _gemm(flags=X3, C=None) == NULL                            # a valid flag: validation goes on
    assert _gemm(flags=X3 | heal.HEAL_W_F16) == UNSUP                 # fp32 operands only
    assert _gemm(flags=X3 | heal.HEAL_ONE_PRODUCT) == UNSUP
    assert _gemm(flags=X3, ks=FAKE) == UNSUP                          # no range shifts in this mode
    assert _gemm(flags=heal.HEAL_ONE_PRODUCT, C=None) == NULL          # a valid flag: validation goes on
    assert _gemm(M=0, A=None, W=None, C=None) == OK
    assert _gemm(N=0, A=None, W=None, C=None) == OK
    assert _gemm(C=None) == NULL
    assert _gemm(ldc=4095) == STRIDE
    assert _gemm(A=None) == NULL
    assert _gemm(W=None) == NULL
    assert _gemm(lda=4095) == STRIDE
    assert _gemm(ldw=4095) == STRIDE
    assert _gemm(flags=heal.HEAL_W_KN, N=8192, ldc=8192) == STRIDE   # KN needs ldw >= N
    assert _gemm(A=ctypes.c_void_p(0x10002)) == ALIGN
    assert _gemm(W=ctypes.c_void_p(0x10001)) == ALIGN
    assert _gemm(W=ctypes.c_void_p(0x10002)) == ALIGN                          # fp32 W: 4-byte aligned
    assert _gemm(flags=heal.HEAL_W_F16, W=ctypes.c_void_p(0x10001)) == ALIGN   # fp16 W: 2-byte aligned
    assert _gemm(flags=heal.HEAL_W_PACKED, W=ctypes.c_void_p(0x10010)) == ALIGN
    assert _gemm(flags=heal.HEAL_A_PACKED, A=ctypes.c_void_p(0x10010)) == ALIGN
    assert _gemm(flags=heal.HEAL_A_PACKED, A=ctypes.c_void_p(0x10100), ks=FAKE) == UNSUP   # packed A: shift at pack time
    assert heal.heal_gemm_f32c_workspace(8, 4096, 4096, 0) > 0     # split-K partials
    assert _gemm(ws=None) == WS
    assert _gemm(wsb=16) == WS
    assert _gemm(ws=ctypes.c_void_p(0x10010)) == ALIGN
    assert _gemm(st=ctypes.c_void_p(0x10002)) == ALIGN


def test_gemm_noalloc_validation():
    """heal_gemm_f32c_noalloc: decode path only, and shapes whose scratch would
    pass the library's 16 MiB array are rejected; both before any HIP call."""
    f = heal.lib().heal_gemm_f32c_noalloc
    args = lambda M=8, N=64, K=256, flags=0: (FAKE, K, FAKE, K, FAKE, N, M, N, K, flags, None, None, None)
    assert f(*args(M=-1)) == SHAPE
    assert f(*args(M=65)) == UNSUP                       # the prefill path allocates its packed operands
    assert f(*args(flags=heal.HEAL_A_PACKED)) == UNSUP
    assert f(*args(flags=heal.HEAL_W_KN)) == UNSUP
    assert f(*args(flags=heal.HEAL_BF16X3)) == UNSUP
    assert f(*args(N=(1 << 19) + 64)) == UNSUP           # one split-K counter per 64 rows of W, 8192 at most
    assert heal.heal_gemm_f32c_workspace(64, 256, 1 << 20, 0) > 16 << 20
    assert f(*args(M=64, N=256, K=1 << 20)) == WS       # split blocks past 16 MiB
    assert heal.heal_gemm_f32c_workspace(64, 4096, 14336, 0) <= 16 << 20   # the Llama-3-8B-like layers fit
    assert heal.heal_gemm_f32c_workspace(64, 14336, 4096, 0) <= 16 << 20
    assert heal.heal_gemm_f32c_workspace(64, 1024, 4096, 0) <= 16 << 20
    assert f(*args(M=0)) == OK


def test_gemm_workspace_sizes():
    ws = heal.heal_gemm_f32c_workspace
    assert ws(0, 64, 64, 0) == 0 and ws(8, 64, -1, 0) == 0
    # decode path (M <= 64, fp32 NK weight): split-K partials only, fixed by (N, K)
    for M in (1, 8, 32, 64):
        b = ws(M, 4096, 4096, 0)
        assert b % 256 == 0
    assert ws(64, 4096, 4096, 0) >= 64 * 4096 * 4
    # prefill path: packed A (rows padded to 256, k to 32, 4 bytes per element
    # and 256 bytes more per row, then one int32 row exponent per padded row)
    # + packed W
    pk = lambda R, Kp, b: R * (Kp * b + 256) + R * 4
    assert ws(2048, 4096, 14336, 0) == pk(2048, 14336, 4) + pk(4096, 14336, 4)
    assert ws(2048, 4096, 14336, heal.HEAL_W_PACKED) == pk(2048, 14336, 4)
    assert ws(2048, 4096, 14336, heal.HEAL_W_PACKED | heal.HEAL_A_PACKED) == 0
    assert ws(8, 4096, 4096, heal.HEAL_A_PACKED) == pk(4096, 4096, 4)   # packed A -> prefill path
    for M in (1, 8, 64):      # a packed weight keeps the decode path and its workspace
        assert ws(M, 4096, 4096, heal.HEAL_W_PACKED) == ws(M, 4096, 4096, 0)
        assert ws(M, 4096, 4096, heal.HEAL_W_PACKED | heal.HEAL_W_F16) == ws(M, 4096, 4096, 0)
    assert ws(65, 100, 33, 0) == pk(256, 64, 4) + pk(256, 64, 4)
    assert heal.heal_pack_w_bytes(100, 33) == pk(256, 64, 4)
    assert heal.heal_pack_w_bytes(100, 33, heal.HEAL_W_F16) == pk(256, 64, 2)      # hi parts only
    assert ws(2048, 4096, 14336, heal.HEAL_W_F16) == pk(2048, 14336, 4) + pk(4096, 14336, 2)
    # BF16 three-way mode: 6 bytes per padded element, every M on the prefill path
    X3 = heal.HEAL_BF16X3
    assert heal.heal_pack_w_bytes(100, 33, X3) == 256 * 64 * 6
    assert ws(1, 4096, 4096, X3) == 256 * 4096 * 6 + 4096 * 4096 * 6
    assert ws(2048, 4096, 14336, X3 | heal.HEAL_W_PACKED) == 2048 * 14336 * 6
    assert ws(2048, 4096, 14336, X3 | heal.HEAL_W_PACKED | heal.HEAL_A_PACKED) == 0


def test_pack_validation():
    L = heal.lib()
    assert L.heal_pack_w(FAKE, 64, -1, 64, 0, None, FAKE, 1 << 30, None, None) == SHAPE
    assert L.heal_pack_w(FAKE, 64, 64, 64, 4, None, FAKE, 1 << 30, None, None) == UNSUP
    assert L.heal_pack_w(FAKE, 64, 0, 64, 0, None, None, 0, None, None) == OK
    assert L.heal_pack_w(None, 64, 64, 64, 0, None, FAKE, 1 << 30, None, None) == NULL
    assert L.heal_pack_w(FAKE, 32, 64, 64, 0, None, FAKE, 1 << 30, None, None) == STRIDE
    assert L.heal_pack_w(FAKE, 64, 64, 64, 0, None, ctypes.c_void_p(0x10080), 1 << 30, None, None) == ALIGN
    assert L.heal_pack_w(ctypes.c_void_p(0x10002), 64, 64, 64, 0, None, FAKE, 1 << 30, None, None) == ALIGN
    assert L.heal_pack_w(ctypes.c_void_p(0x10001), 64, 64, 64, heal.HEAL_W_F16, None, FAKE, 1 << 30, None, None) == ALIGN
    assert L.heal_pack_w(FAKE, 64, 64, 64, heal.HEAL_W_F16 | 16, None, FAKE, 1 << 30, None, None) == UNSUP
    assert L.heal_pack_w(FAKE, 64, 64, 64, 0, None, FAKE, 100, None, None) == WS
    X3 = heal.HEAL_BF16X3
    assert L.heal_pack_w(FAKE, 64, 64, 64, X3 | heal.HEAL_W_F16, None, FAKE, 1 << 30, None, None) == UNSUP
    assert L.heal_pack_w(FAKE, 64, 64, 64, X3, FAKE, FAKE, 1 << 30, None, None) == UNSUP      # no kshift
    assert L.heal_pack_w(FAKE, 64, 64, 64, X3, None, FAKE, 256 * 64 * 4, None, None) == WS  # needs 6 B/elem
    assert L.heal_pack_w(None, 64, 64, 64, X3, None, FAKE, 1 << 30, None, None) == NULL


def test_scale_k_validation():
    L = heal.lib()
    sk = L.heal_scale_k
    assert sk(FAKE, 64, -1, 64, 0, FAKE, FAKE, 64, None) == SHAPE
    assert sk(FAKE, 64, 64, 64, 2, FAKE, FAKE, 64, None) == UNSUP          # only HEAL_W_KN / HEAL_W_F16
    assert sk(None, 64, 0, 64, 0, None, None, 64, None) == OK
    assert sk(FAKE, 64, 64, 64, 0, None, FAKE, 64, None) == NULL          # the shifts are required
    assert sk(FAKE, 63, 64, 64, 0, FAKE, FAKE, 64, None) == STRIDE
    assert sk(FAKE, 64, 100, 64, heal.HEAL_W_KN, FAKE, FAKE, 100, None) == STRIDE   # [K, rows]: ld >= rows
    assert sk(FAKE, 64, 64, 64, 0, FAKE, FAKE, 32, None) == STRIDE
    assert sk(ctypes.c_void_p(0x10002), 64, 64, 64, 0, FAKE, FAKE, 64, None) == ALIGN
    assert sk(FAKE, 64, 64, 64, heal.HEAL_W_F16, FAKE, ctypes.c_void_p(0x10001), 64, None) == ALIGN


def test_kshift_from_absmax():
    """Host arithmetic: the smallest s >= 0 with absmax * 2^-s < limit."""
    f = heal.heal_kshift_from_absmax
    a = np.array([0.0, 1.0, 32767.99, 32768.0, 65535.0, 65536.0, 1e6, 2.0 ** 40, 3e38], np.float32)
    s = f(a, 32768.0)
    assert s.dtype == np.int8
    assert s.tolist() == [0, 0, 0, 1, 1, 2, 5, 26, 113]
    for ai, si in zip(a.astype(np.float64), s.astype(int)):   # the definition, checked exactly
        assert ai * 2.0 ** -si < 32768.0 and (si == 0 or ai * 2.0 ** -(si - 1) >= 32768.0)
    assert f(np.array([1.0, 3.0], np.float32), 1.0).tolist() == [1, 2]
    L = heal.lib()
    out = np.full(3, 7, np.int8)
    P = ctypes.c_void_p
    for bad in (np.array([1.0, np.nan, 2.0], np.float32), np.array([1.0, np.inf, 2.0], np.float32),
                np.array([1.0, -1.0, 2.0], np.float32)):
        assert L.heal_kshift_from_absmax(bad.ctypes.data_as(P), 3, 32768.0, out.ctypes.data_as(P)) == UNSUP
        assert out.tolist() == [7, 7, 7]      # nothing written on failure
    good = np.ones(3, np.float32)
    assert L.heal_kshift_from_absmax(good.ctypes.data_as(P), 3, 0.5, out.ctypes.data_as(P)) == UNSUP
    assert L.heal_kshift_from_absmax(good.ctypes.data_as(P), 3, 70000.0, out.ctypes.data_as(P)) == UNSUP
    assert L.heal_kshift_from_absmax(None, 3, 32768.0, out.ctypes.data_as(P)) == NULL
    assert L.heal_kshift_from_absmax(None, 0, 32768.0, None) == OK
    assert L.heal_kshift_from_absmax(good.ctypes.data_as(P), -1, 32768.0, out.ctypes.data_as(P)) == SHAPE


def test_quant_dequant_validation():
    L = heal.lib()
    q = L.heal_qkv_quant_i16
    assert q(FAKE, -1, 128, 128, FAKE, 128, FAKE, None) == SHAPE
    assert q(None, 0, 128, 128, None, 128, None, None) == OK
    for D in (0, 2, 6, 4100):
        assert q(FAKE, 4, D, 4104, FAKE, 4104, FAKE, None) == SHAPE
    assert q(None, 4, 128, 128, FAKE, 128, FAKE, None) == NULL
    assert q(FAKE, 4, 128, 124, FAKE, 128, FAKE, None) == STRIDE
    assert q(FAKE, 4, 128, 128, FAKE, 124, FAKE, None) == STRIDE
    assert q(FAKE_ODD, 4, 128, 128, FAKE, 128, FAKE, None) == ALIGN
    assert q(FAKE, 4, 128, 130, FAKE, 128, FAKE, None) == ALIGN
    assert q(FAKE, 4, 128, 128, ctypes.c_void_p(0x10002), 128, FAKE, None) == ALIGN
    d = L.heal_kv_dequant_i16
    assert d(FAKE, 4, 128, 128, FAKE, 7, FAKE, None, 128, None) == UNSUP
    assert d(FAKE, 4, 128, 128, None, heal.HEAL_DQ_F32, FAKE, None, 128, None) == NULL
    assert d(FAKE, 4, 128, 128, None, heal.HEAL_DQ_F16X2, FAKE, None, 128, None) == NULL
    assert d(FAKE, 4, 128, 128, FAKE, heal.HEAL_DQ_F32, FAKE_ODD, None, 128, None) == ALIGN
    assert d(FAKE, 4, 128, 120, FAKE, heal.HEAL_DQ_F32, FAKE, None, 128, None) == STRIDE


def _qkv(M=8, K=256, Hq=4, Hkv=2, D=128, flags=0, q=FAKE, sl=FAKE, kc=FAKE, ns=16, ws=FAKE, wsb=1 << 30):
    return heal.lib().heal_qkv_proj_quant_i16(FAKE, K, FAKE, K, M, K, Hq, Hkv, D, flags, None, q, FAKE, sl, ns, kc,
                                              FAKE, FAKE, FAKE, ws, wsb, None, None)


def test_qkv_proj_validation():
    assert _qkv(M=-1) == SHAPE
    assert _qkv(Hkv=0) == SHAPE
    assert _qkv(D=6) == SHAPE
    assert _qkv(flags=heal.HEAL_W_KN) == UNSUP
    assert _qkv(M=0, q=None, sl=None) == OK
    assert _qkv(q=None) == NULL
    assert _qkv(sl=None) == NULL
    assert _qkv(kc=ctypes.c_void_p(0x10004)) == ALIGN
    assert _qkv(sl=ctypes.c_void_p(0x10004)) == ALIGN
    assert _qkv(ws=None) == WS
    assert _qkv(wsb=16) == WS
    n = heal.heal_qkv_proj_quant_workspace(8, 256, 4, 2, 128, 0)
    assert n >= 8 * 1024 * 4 and n % 256 == 0
    # quantized in the GEMM epilogue (heads of 128, no k split): packed operands only
    wsq, wsg = heal.heal_qkv_proj_quant_workspace, heal.heal_gemm_f32c_workspace
    assert wsq(2048, 4096, 32, 8, 128, 0) == wsg(2048, 6144, 4096, 0)
    assert wsq(300, 200, 4, 2, 128, 0) == wsg(300, 1024, 200, 0)
    # two passes (the fp32 product lands in the workspace first): k split, D != 128, decode sizes
    assert wsq(300, 512, 4, 2, 128, 0) == 300 * 1024 * 4 + wsg(300, 1024, 512, 0)
    assert wsq(2048, 4096, 32, 8, 64, 0) == 2048 * 48 * 64 * 4 + wsg(2048, 48 * 64, 4096, 0)
    assert wsq(2048, 4096, 32, 8, 128, heal.HEAL_ONE_PRODUCT) == \
        2048 * 6144 * 4 + wsg(2048, 6144, 4096, heal.HEAL_ONE_PRODUCT)
    # K == 0: a zero product, staged and quantized to zero codes; the workspace
    # holds it, so a missing or short one is rejected before any launch
    assert wsq(8, 0, 4, 2, 128, 0) == 8 * 1024 * 4
    assert _qkv(K=0, ws=None) == WS
    assert _qkv(K=0, wsb=8 * 1024 * 4 - 256) == WS


def _attn(B=2, T=16, Hq=8, Hkv=2, D=128, ws=FAKE, wsb=1 << 30, q=FAKE):
    return heal.lib().heal_attn_decode_i16(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, T, Hq, Hkv, D, ws, wsb, None)


def test_attention_prefill_validation():
    f = heal.lib().heal_attn_prefill_i16
    args = lambda q=FAKE, B=1, T=64, Hq=8, Hkv=2, D=128, o=FAKE: (q, FAKE, FAKE, FAKE, FAKE, FAKE, o, B, T, Hq, Hkv,
                                                                   D, None)
    assert f(*args(B=-1)) == SHAPE
    assert f(*args(T=0, q=None)) == OK
    assert f(*args(Hkv=3)) == SHAPE
    assert f(*args(D=64)) == UNSUP
    assert f(*args(T=262145)) == UNSUP
    assert f(*args(q=None)) == NULL
    assert f(*args(q=ctypes.c_void_p(0x10008))) == ALIGN
    assert f(*args(o=ctypes.c_void_p(0x10002))) == ALIGN
    assert f(*args(Hq=1 << 40, Hkv=1 << 40)) == SHAPE
    # 2^14 batches x 64 heads x 2048 query blocks x 512 threads: past the 32-bit grid size
    assert f(*args(B=1 << 14, T=262144, Hq=64, Hkv=1)) == UNSUP
    assert f(*args(B=1 << 14, T=64, Hq=64, Hkv=1, q=None)) == NULL   # the same heads at T = 64 fit


def test_attention_validation():
    assert _attn(B=-1) == SHAPE
    assert _attn(B=0, q=None) == OK
    assert _attn(Hkv=3) == SHAPE
    assert _attn(T=0) == SHAPE
    assert _attn(D=64) == UNSUP
    assert _attn(Hq=18, Hkv=1) == UNSUP
    assert _attn(T=262145) == UNSUP
    assert _attn(T=131072, Hq=128, Hkv=128) == UNSUP   # K block of one batch past 4 GiB
    assert _attn(Hq=1 << 40, Hkv=1 << 40) == SHAPE
    # launch sizes past the 32-bit grid size: the range kernel, then the merge
    assert _attn(B=1 << 20, T=8192, Hq=8, Hkv=8) == UNSUP
    assert _attn(B=1 << 24, T=1, Hq=1, Hkv=1) == UNSUP
    assert _attn(B=1 << 12, T=8192, Hq=8, Hkv=8, q=None) == NULL   # within both
    assert _attn(q=None) == NULL
    assert _attn(q=ctypes.c_void_p(0x10008)) == ALIGN
    assert _attn(ws=None) == WS
    assert _attn(wsb=8) == WS
    assert heal.heal_attn_decode_workspace(16, 8192, 32, 8, 128) > 0
