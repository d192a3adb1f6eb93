"""Python binding of libheal: the HEAL hot path on MI355X (gfx950).

Thin ctypes wrappers with the same names as the C ABI in include/heal.h.
They only marshal arguments: every step of the computation runs in the HIP
kernels of libheal.so.  PyTorch supplies device memory (tensors, workspaces)
and the stream (the current torch stream).  There is no CPU fallback: if the
library is missing the binding raises.
"""
import ctypes
import os

import torch

__all__ = [
    "HealError", "lib", "heal_status_str", "heal_version", "heal_split_f32", "heal_gemm_f32c",
    "heal_gemm_f32c_workspace", "heal_gemm_f32c_noalloc", "heal_pack_w", "heal_pack_w_bytes", "heal_qkv_quant_i16",
    "heal_kv_dequant_i16", "heal_attn_decode_i16", "heal_attn_decode_workspace", "PackedOperand",
    "heal_scale_k", "heal_kshift_from_absmax",
    "PackedWeight", "HEAL_W_NK", "HEAL_W_KN", "HEAL_W_PACKED", "HEAL_A_PACKED", "HEAL_W_F16", "HEAL_ONE_PRODUCT", "HEAL_BF16X3",
    "HEAL_FLAG_F16_RANGE", "HEAL_FLAG_SLOT_RANGE", "heal_qkv_proj_quant_i16", "heal_qkv_proj_quant_workspace",
    "heal_attn_prefill_i16", "heal_calib_mfma_f16", "heal_calib_read",
    "HEAL_DQ_F32", "HEAL_DQ_F16X2",
    "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libheal.so")

HEAL_OK = 0
HEAL_W_NK, HEAL_W_KN, HEAL_W_PACKED, HEAL_A_PACKED, HEAL_W_F16, HEAL_ONE_PRODUCT = 0, 1, 2, 4, 8, 16
HEAL_BF16X3 = 32
HEAL_FLAG_F16_RANGE = 1
HEAL_FLAG_SLOT_RANGE = 2
HEAL_DQ_F32, HEAL_DQ_F16X2 = 0, 1

# (name, argtypes, restype) of every exported entry point
_I64, _P, _SZ, _U32, _INT = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_int
SIGNATURES = {
    "heal_status_str": ([_INT], ctypes.c_char_p),
    "heal_version": ([], _INT),
    "heal_split_f32": ([_P, _I64, _P, _P, _P, _P], _INT),
    "heal_gemm_f32c": ([_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _U32, _P, _P, _SZ, _P, _P], _INT),
    "heal_gemm_f32c_workspace": ([_I64, _I64, _I64, _U32], _SZ),
    "heal_gemm_f32c_noalloc": ([_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _U32, _P, _P, _P], _INT),
    "heal_pack_w": ([_P, _I64, _I64, _I64, _U32, _P, _P, _SZ, _P, _P], _INT),
    "heal_scale_k": ([_P, _I64, _I64, _I64, _U32, _P, _P, _I64, _P], _INT),
    "heal_kshift_from_absmax": ([_P, _I64, ctypes.c_float, _P], _INT),
    "heal_pack_w_bytes": ([_I64, _I64, _U32], _SZ),
    "heal_qkv_quant_i16": ([_P, _I64, _I64, _I64, _P, _I64, _P, _P], _INT),
    "heal_kv_dequant_i16": ([_P, _I64, _I64, _I64, _P, _INT, _P, _P, _I64, _P], _INT),
    "heal_attn_decode_i16": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "heal_attn_decode_workspace": ([_I64, _I64, _I64, _I64, _I64], _SZ),
    "heal_qkv_proj_quant_i16": ([_P, _I64, _P, _I64, _I64, _I64, _I64, _I64, _I64, _U32, _P, _P, _P, _P, _I64,
                                 _P, _P, _P, _P, _P, _SZ, _P, _P], _INT),
    "heal_qkv_proj_quant_workspace": ([_I64, _I64, _I64, _I64, _I64, _U32], _SZ),
    "heal_attn_prefill_i16": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P], _INT),
    "heal_calib_mfma_f16": ([_I64, _I64, _P, _P], _INT),
    "heal_calib_read": ([_P, _I64, _I64, _P, _P], _INT),
}

_LIB = None


class HealError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {heal_status_str(status)}")
        self.status = status


def lib():
    """The loaded libheal.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with error_compensated_gemm_heal_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        for name, (argtypes, restype) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _LIB = L
    return _LIB


def heal_status_str(status: int) -> str:
    return lib().heal_status_str(int(status)).decode()


def heal_version() -> int:
    return lib().heal_version()


def _check(fn: str, status: int):
    if status != HEAL_OK:
        raise HealError(fn, status)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _rowmajor_ld(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a 2-D row-major view (unit stride along rows)."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its rows")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None
    # 256-byte alignment: torch's caching allocator returns blocks aligned far beyond that
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ---- operand split ------------------------------------------------------------

def heal_split_f32(X: torch.Tensor, hi=None, lo=None, dev_status=None):
    """x -> (hi, lo) fp16 with x ~= hi + lo / 2^10 (elementwise, contiguous)."""
    _dev(X, "X", torch.float32)
    X = X.contiguous()
    hi = torch.empty(X.shape, dtype=torch.float16, device=X.device) if hi is None else hi
    lo = torch.empty(X.shape, dtype=torch.float16, device=X.device) if lo is None else lo
    _check("heal_split_f32", lib().heal_split_f32(_ptr(X), X.numel(), _ptr(hi), _ptr(lo),
                                                  _ptr(dev_status), _stream()))
    return hi, lo


# ---- compensated GEMM ------------------------------------------------------------

class PackedOperand:
    """An operand of `rows` x K split once into the GEMM's packed dual-FP16 form
    (opaque buffer): a weight (rows = N) or an activation (rows = M)."""

    def __init__(self, buf: torch.Tensor, rows: int, K: int, f16: bool = False, bf16x3: bool = False):
        # f16: packed from binary16 weights (zero lo planes): GEMMs take the
        # two-product form (HEAL_W_PACKED | HEAL_W_F16).  bf16x3: the BF16
        # three-way form, for GEMMs in that mode only.
        self.buf, self.rows, self.K, self.f16, self.bf16x3 = buf, rows, K, f16, bf16x3

    @property
    def N(self):
        return self.rows


PackedWeight = PackedOperand


def heal_pack_w_bytes(N: int, K: int, flags: int = 0) -> int:
    return lib().heal_pack_w_bytes(N, K, flags)


def _weight_dtype_flag(W: torch.Tensor) -> int:
    """fp32 weights, or float16 ones (binary16 values: the two-product form)."""
    if W.dtype == torch.float16:
        return HEAL_W_F16
    if W.dtype != torch.float32:
        raise TypeError(f"W must be float32 or float16, got {W.dtype}")
    return 0


def _kshift(kshift, K: int, name: str):
    """A per-channel shift vector: a device int8 tensor of K entries, or None."""
    if kshift is None:
        return None
    _dev(kshift, name, torch.int8)
    if kshift.numel() != K or (K > 1 and kshift.stride(-1) != 1):
        raise ValueError(f"{name} must be a contiguous int8 vector of K = {K} entries")
    return kshift


def heal_pack_w(W: torch.Tensor, w_layout: str = "nk", dev_status=None, out=None, kshift=None,
                bf16x3: bool = False) -> PackedOperand:
    """Split an operand once into the packed form.  kshift (int8 [K], optional):
    element (r, k) is multiplied by 2^-kshift[k] first (an activation takes the
    shifts given to heal_gemm_f32c as a_kshift, a weight their negation).
    bf16x3: the BF16 three-way form (fp32 input, no kshift)."""
    _dev(W, "W")
    flags = (HEAL_W_KN if w_layout == "kn" else HEAL_W_NK) | _weight_dtype_flag(W) | (HEAL_BF16X3 if bf16x3 else 0)
    if w_layout == "kn":
        K, N = W.shape
    else:
        N, K = W.shape
    ldw = _rowmajor_ld(W, "W")
    nbytes = heal_pack_w_bytes(N, K, flags)
    if out is None:
        buf = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=W.device)
    else:
        buf = out.buf
        if buf.numel() < nbytes:
            raise ValueError("packed buffer too small")
    ks = _kshift(kshift, K, "kshift")
    _check("heal_pack_w", lib().heal_pack_w(_ptr(W), ldw, N, K, flags, _ptr(ks), _ptr(buf), nbytes,
                                            _ptr(dev_status), _stream()))
    return PackedOperand(buf, N, K, f16=bool(flags & HEAL_W_F16), bf16x3=bool(bf16x3))


def heal_gemm_f32c_workspace(M: int, N: int, K: int, flags: int) -> int:
    return lib().heal_gemm_f32c_workspace(M, N, K, flags)


def heal_gemm_f32c(A, W, w_layout: str = "nk", C=None, workspace=None, dev_status=None, a_kshift=None,
                   one_product: bool = False, bf16x3: bool = False):
    """C = A . B with B = W^T ('nk', W [N,K]) or B = W ('kn', W [K,N]).
    A and/or W may be PackedOperand buffers from heal_pack_w.  a_kshift (int8
    [K], optional): A's element (m, k) is multiplied by 2^-a_kshift[k] before
    its split; W must hold reduction index k multiplied by 2^+a_kshift[k].
    one_product: plain FP16, C = A_hi.B_hi (no compensation).  bf16x3: the
    BF16 three-way split with six products (packed operands must be packed in
    that form)."""
    for X, name in ((A, "A"), (W, "W")):
        if isinstance(X, PackedOperand) and X.bf16x3 != bool(bf16x3):
            raise ValueError(f"packed {name} was packed {'with' if X.bf16x3 else 'without'} bf16x3")
    aflags = 0
    if isinstance(A, PackedOperand):
        M, K, lda, aptr, adev, aflags = A.rows, A.K, 0, _ptr(A.buf), A.buf.device, HEAL_A_PACKED
    else:
        _dev(A, "A", torch.float32)
        M, K = A.shape
        lda, aptr, adev = _rowmajor_ld(A, "A"), _ptr(A), A.device
    if isinstance(W, PackedOperand):
        if W.K != K:
            raise ValueError("packed weight has a different K")
        N, flags, wptr, ldw = W.rows, HEAL_W_PACKED | (HEAL_W_F16 if W.f16 else 0), _ptr(W.buf), 0
    else:
        _dev(W, "W")
        if w_layout == "kn":
            K2, N = W.shape
            flags = HEAL_W_KN
        else:
            N, K2 = W.shape
            flags = HEAL_W_NK
        flags |= _weight_dtype_flag(W)
        if K2 != K:
            raise ValueError("inner dimensions differ")
        wptr, ldw = _ptr(W), _rowmajor_ld(W, "W")
    flags |= aflags | (HEAL_ONE_PRODUCT if one_product else 0) | (HEAL_BF16X3 if bf16x3 else 0)
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=adev)
    ldc = _rowmajor_ld(C, "C") if M > 0 and N > 0 else N
    nbytes = heal_gemm_f32c_workspace(M, N, K, flags)
    if workspace is None:
        workspace = _workspace(nbytes, adev)
    elif workspace.numel() < nbytes:
        raise ValueError("workspace too small")
    ks = _kshift(a_kshift, K, "a_kshift")
    _check("heal_gemm_f32c", lib().heal_gemm_f32c(aptr, lda, wptr, ldw, _ptr(C), ldc, M, N, K, flags, _ptr(ks),
                                                  _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                                  _ptr(dev_status), _stream()))
    return C


def heal_gemm_f32c_noalloc(A: torch.Tensor, W, C: torch.Tensor, dev_status=None, a_kshift=None):
    """C = A . W^T on the decode path with the library's own scratch memory:
    no allocation anywhere in the call (C is the caller's).  A fp32 [M, K]
    with M <= 64, W fp32 or float16 [N, K], or a PackedOperand of it."""
    _dev(A, "A", torch.float32)
    _dev(C, "C", torch.float32)
    M, K = A.shape
    if isinstance(W, PackedOperand):
        if W.bf16x3:
            raise ValueError("a weight packed with bf16x3 takes the prefill path")
        N, K2, wptr, ldw = W.rows, W.K, _ptr(W.buf), 0
        flags = HEAL_W_PACKED | (HEAL_W_F16 if W.f16 else 0)
    else:
        _dev(W, "W")
        N, K2 = W.shape
        wptr, ldw = _ptr(W), _rowmajor_ld(W, "W") if N > 0 else K
        flags = HEAL_W_NK | _weight_dtype_flag(W)
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError("shapes of A, W and C do not match")
    ks = _kshift(a_kshift, K, "a_kshift")
    ldc = _rowmajor_ld(C, "C") if M > 0 and N > 0 else N
    _check("heal_gemm_f32c_noalloc",
           lib().heal_gemm_f32c_noalloc(_ptr(A), _rowmajor_ld(A, "A") if M > 0 else K, wptr, ldw, _ptr(C), ldc,
                                        M, N, K, flags, _ptr(ks), _ptr(dev_status), _stream()))
    return C


def heal_calib_mfma_f16(iters: int, workgroups: int = 256, out=None):
    """Register-only 16-bit MFMA loop (roofline calibration); returns out and
    the flops it performs."""
    if out is None:
        out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    _check("heal_calib_mfma_f16", lib().heal_calib_mfma_f16(iters, workgroups, _ptr(out), _stream()))
    return out, workgroups * 4 * iters * 16 * 32768


def heal_calib_read(buf: torch.Tensor, workgroups: int = 2048, out=None):
    """Streaming read of a device buffer (roofline calibration)."""
    _dev(buf, "buf")
    if out is None:
        out = torch.empty(workgroups * 256, dtype=torch.float32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check("heal_calib_read", lib().heal_calib_read(_ptr(buf), nbytes, workgroups, _ptr(out), _stream()))
    return out


def heal_scale_k(X: torch.Tensor, kshift: torch.Tensor, w_layout: str = "nk", out=None):
    """out = X with element (r, k) multiplied by 2^-kshift[k] (fp32 or fp16, layout
    'nk' = [rows, K] or 'kn' = [K, rows]); out may be X for an in-place update."""
    _dev(X, "X")
    flags = (HEAL_W_KN if w_layout == "kn" else HEAL_W_NK) | _weight_dtype_flag(X)
    if w_layout == "kn":
        K, rows = X.shape
    else:
        rows, K = X.shape
    ks = _kshift(kshift, K, "kshift")
    if ks is None:
        raise ValueError("kshift is required")
    out = torch.empty_like(X) if out is None else out
    if out.shape != X.shape or out.dtype != X.dtype:
        raise ValueError("out must match X in shape and dtype")
    _check("heal_scale_k", lib().heal_scale_k(_ptr(X), _rowmajor_ld(X, "X"), rows, K, flags, _ptr(ks), _ptr(out),
                                              _rowmajor_ld(out, "out"), _stream()))
    return out


def heal_kshift_from_absmax(absmax, limit: float = 32768.0):
    """Host call: per-channel shifts (int8 numpy array) from calibration maxima
    max|A[:, k]|: the smallest s >= 0 with absmax[k] * 2^-s < limit."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(absmax, dtype=np.float32).reshape(-1))
    out = np.zeros(a.size, dtype=np.int8)
    _check("heal_kshift_from_absmax", lib().heal_kshift_from_absmax(
        a.ctypes.data_as(ctypes.c_void_p), a.size, float(limit), out.ctypes.data_as(ctypes.c_void_p)))
    return out


# ---- INT16 quant / dequant -------------------------------------------------------------

def heal_qkv_proj_quant_workspace(M: int, K: int, Hq: int, Hkv: int, D: int, flags: int = 0) -> int:
    return lib().heal_qkv_proj_quant_workspace(M, K, Hq, Hkv, D, flags)


def heal_qkv_proj_quant_i16(A, W, Hq: int, Hkv: int, D: int, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                            k_scales: torch.Tensor, v_cache: torch.Tensor, v_scales: torch.Tensor, q_codes=None,
                            q_scales=None, workspace=None, dev_status=None, a_kshift=None,
                            one_product: bool = False, bf16x3: bool = False):
    """Fused Q/K/V projection stored as INT16: C = A . W^T (W [(Hq + 2 Hkv) D, K], or a
    packed weight), Q rows -> (q_codes [M, Hq, D], q_scales [M, Hq]) returned, K/V rows
    -> k/v_cache [num_slots, Hkv, D] and k/v_scales [num_slots, Hkv] at slot_mapping[m].
    one_product / bf16x3: the GEMM's precision modes, as in heal_gemm_f32c."""
    _dev(A, "A", torch.float32)
    M, K = A.shape
    N = (Hq + 2 * Hkv) * D
    if isinstance(W, PackedOperand):
        if W.K != K or W.rows != N:
            raise ValueError("packed weight does not match (K, (Hq + 2 Hkv) D)")
        if W.bf16x3 != bool(bf16x3):
            raise ValueError(f"packed W was packed {'with' if W.bf16x3 else 'without'} bf16x3")
        flags, wptr, ldw = HEAL_W_PACKED | (HEAL_W_F16 if W.f16 else 0), _ptr(W.buf), 0
    else:
        _dev(W, "W")
        if tuple(W.shape) != (N, K):
            raise ValueError("W must be [(Hq + 2 Hkv) D, K]")
        flags, wptr, ldw = _weight_dtype_flag(W), _ptr(W), _rowmajor_ld(W, "W")
    flags |= (HEAL_ONE_PRODUCT if one_product else 0) | (HEAL_BF16X3 if bf16x3 else 0)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    for t, name, dt in ((k_cache, "k_cache", torch.int16), (v_cache, "v_cache", torch.int16),
                        (k_scales, "k_scales", torch.float32), (v_scales, "v_scales", torch.float32)):
        _dev(t, name, dt)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    num_slots = k_cache.numel() // (Hkv * D)
    if (k_cache.numel() != num_slots * Hkv * D or v_cache.numel() != k_cache.numel()
            or k_scales.numel() != num_slots * Hkv or v_scales.numel() != k_scales.numel()):
        raise ValueError("cache shapes must be [num_slots, Hkv, D] and scales [num_slots, Hkv]")
    if slot_mapping.numel() != M or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 vector of M entries")
    if q_codes is None:
        q_codes = torch.empty((M, Hq, D), dtype=torch.int16, device=A.device)
    if q_scales is None:
        q_scales = torch.empty((M, Hq), dtype=torch.float32, device=A.device)
    nbytes = heal_qkv_proj_quant_workspace(M, K, Hq, Hkv, D, flags)
    if workspace is None:
        workspace = _workspace(nbytes, A.device)
    elif workspace.numel() < nbytes:
        raise ValueError("workspace too small")
    ks = _kshift(a_kshift, K, "a_kshift")
    _check("heal_qkv_proj_quant_i16", lib().heal_qkv_proj_quant_i16(
        _ptr(A), _rowmajor_ld(A, "A"), wptr, ldw, M, K, Hq, Hkv, D, flags, _ptr(ks), _ptr(q_codes), _ptr(q_scales),
        _ptr(slot_mapping), num_slots, _ptr(k_cache), _ptr(k_scales), _ptr(v_cache), _ptr(v_scales),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _ptr(dev_status), _stream()))
    return q_codes, q_scales


def heal_qkv_quant_i16(X: torch.Tensor, codes=None, scales=None):
    """X [..., D] fp32 -> (codes int16 [..., D], scales fp32 [...]), one scale per row of D."""
    _dev(X, "X", torch.float32)
    X = X.contiguous()
    D = X.shape[-1]
    rows = X.numel() // D if D else 0
    codes = torch.empty(X.shape, dtype=torch.int16, device=X.device) if codes is None else codes
    scales = torch.empty(X.shape[:-1], dtype=torch.float32, device=X.device) if scales is None else scales
    _check("heal_qkv_quant_i16", lib().heal_qkv_quant_i16(_ptr(X), rows, D, D, _ptr(codes), D, _ptr(scales),
                                                          _stream()))
    return codes, scales


def heal_kv_dequant_i16(codes: torch.Tensor, scales=None, fmt: str = "f32", out=None):
    """codes [..., D] int16 (+ scales [...]) -> fp32 values, or (hi, lo) fp16 planes for fmt='f16x2'."""
    _dev(codes, "codes", torch.int16)
    codes = codes.contiguous()
    D = codes.shape[-1]
    rows = codes.numel() // D if D else 0
    if fmt == "f32":
        out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device) if out is None else out
        _check("heal_kv_dequant_i16", lib().heal_kv_dequant_i16(_ptr(codes), rows, D, D, _ptr(scales), HEAL_DQ_F32,
                                                                _ptr(out), None, D, _stream()))
        return out
    hi = torch.empty(codes.shape, dtype=torch.float16, device=codes.device)
    lo = torch.empty(codes.shape, dtype=torch.float16, device=codes.device)
    _check("heal_kv_dequant_i16", lib().heal_kv_dequant_i16(_ptr(codes), rows, D, D, _ptr(scales), HEAL_DQ_F16X2,
                                                            _ptr(hi), _ptr(lo), D, _stream()))
    return hi, lo


# ---- decode attention over INT16 Q/K/V -----------------------------------------------------

def heal_attn_decode_workspace(B, T, Hq, Hkv, D) -> int:
    return lib().heal_attn_decode_workspace(B, T, Hq, Hkv, D)


def heal_attn_prefill_i16(q, q_scale, k, k_scale, v, v_scale, out=None):
    """Causal self-attention of a prompt: q [B,T,Hq,D] int16 + [B,T,Hq]; k, v [B,T,Hkv,D]
    int16 + [B,T,Hkv] -> out [B,T,Hq,D] fp32 (query t sees keys 0 .. t)."""
    for name, t, dt in (("q", q, torch.int16), ("k", k, torch.int16), ("v", v, torch.int16),
                        ("q_scale", q_scale, torch.float32), ("k_scale", k_scale, torch.float32),
                        ("v_scale", v_scale, torch.float32)):
        _dev(t, name, dt)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, T, Hkv, D) or tuple(v.shape) != (B, T, Hkv, D):
        raise ValueError("k and v must be [B, T, Hkv, D] with q's B, T, D")
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q.device) if out is None else out
    _check("heal_attn_prefill_i16", lib().heal_attn_prefill_i16(
        _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(v), _ptr(v_scale), _ptr(out), B, T, Hq, Hkv, D,
        _stream()))
    return out


def heal_attn_decode_i16(q, q_scale, k, k_scale, v, v_scale, out=None, workspace=None):
    """q [B,Hq,D] int16 + [B,Hq]; k, v [B,T,Hkv,D] int16 + [B,T,Hkv] -> out [B,Hq,D] fp32."""
    for name, t, dt in (("q", q, torch.int16), ("k", k, torch.int16), ("v", v, torch.int16),
                        ("q_scale", q_scale, torch.float32), ("k_scale", k_scale, torch.float32),
                        ("v_scale", v_scale, torch.float32)):
        _dev(t, name, dt)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, Hq, D = q.shape
    _, T, Hkv, _ = k.shape
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device) if out is None else out
    nbytes = heal_attn_decode_workspace(B, T, Hq, Hkv, D)
    if workspace is None:
        workspace = _workspace(nbytes, q.device)
    _check("heal_attn_decode_i16", lib().heal_attn_decode_i16(
        _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(v), _ptr(v_scale), _ptr(out), B, T, Hq, Hkv, D,
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream()))
    return out
