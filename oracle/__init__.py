"""CPU oracle for the HEAL hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU baseline leg may
import this package.  The GPU library and its Python binding never import it.

The arithmetic lives in heal_oracle.c (plain C, binary64 / naive binary32);
this module only marshals numpy arrays through ctypes.  See heal_oracle.c
for the passage of the HEAL paper each function follows and what pins it.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_c_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def lib():
    """Load the oracle library, building it first only if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        sigs = {
            "oracle_f32_to_f16": [_p, _c_i64, _p],
            "oracle_f16_to_f64": [_p, _c_i64, _p],
            "oracle_split_f16": [_p, _c_i64, _p, _p],
            "oracle_gemm_f64": [_p, _c_i64, _p, _c_i64, ctypes.c_int, _p, _c_i64, _c_i64, _c_i64, _c_i64],
            "oracle_gemm_f32_naive": [_p, _c_i64, _p, _c_i64, ctypes.c_int, _p, _c_i64, _c_i64, _c_i64, _c_i64],
            "oracle_gemm_comp_model": [_p, _c_i64, _p, _c_i64, ctypes.c_int, _p, _c_i64, _c_i64, _c_i64, _c_i64],
            "oracle_row_exponent": [_p, _c_i64, _c_i64, _c_i64, _p],
            "oracle_split_rownorm": [_p, _c_i64, _c_i64, _c_i64, _p, _p, _p],
            "oracle_gemm_f64_rows": [_p, _c_i64, _p, _c_i64, ctypes.c_int, _p, _c_i64, _p, _c_i64, _c_i64, _c_i64],
            "oracle_gemm_f32_naive_rows": [_p, _c_i64, _p, _c_i64, ctypes.c_int, _p, _c_i64, _p, _c_i64, _c_i64, _c_i64],
            "oracle_quant_i16": [_p, _c_i64, _c_i64, _c_i64, _p, _c_i64, _p],
            "oracle_dequant_f32": [_p, _c_i64, _c_i64, _c_i64, _p, _p, _c_i64],
            "oracle_dequant_f16x2": [_p, _c_i64, _c_i64, _c_i64, _p, _p, _c_i64],
            "oracle_attn_decode_f64": [_p] * 6 + [_p] + [_c_i64] * 5,
            "oracle_attn_decode_weight_norm": [_p] * 6 + [_p] + [_c_i64] * 5,
            "oracle_attn_decode_f32_naive": [_p] * 6 + [_p] + [_c_i64] * 5,
        }
        for name, argtypes in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = argtypes
            fn.restype = None
        L.oracle_abi_version.restype = ctypes.c_int
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        _LIB = L
    return _LIB


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Set the OpenMP threads of the oracle's parallel loops (for CPU timings)."""
    lib().oracle_set_num_threads(int(n))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --- binary16 -----------------------------------------------------------------

def f32_to_f16_bits(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_f16(_ptr(x), x.size, _ptr(out))
    return out


def f16_bits_to_f64(h):
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().oracle_f16_to_f64(_ptr(h), h.size, _ptr(out))
    return out


# --- split ----------------------------------------------------------------------

def split_f16(x):
    """x (float32, any shape) -> (hi, lo) binary16 bit patterns, x ~= hi + lo/2^10."""
    x = _c(x, np.float32)
    hi = np.empty(x.shape, np.uint16)
    lo = np.empty(x.shape, np.uint16)
    lib().oracle_split_f16(_ptr(x), x.size, _ptr(hi), _ptr(lo))
    return hi, lo


# --- row normalization ------------------------------------------------------------

def row_exponent(X):
    """X float32 [rows, K] -> int32 [rows]: e with 2^14 <= max_k |x_k| 2^e < 2^15
    (0 for a zero row).  HEAL paper, section 3, "Mitigating GEMM Truncation via
    FP16 Promotion and Algebraic Compensation" (FP16's narrow range, handled by
    targeted power-of-two rescaling)."""
    X = _c(X, np.float32)
    rows, K = X.shape
    e = np.empty(rows, np.int32)
    lib().oracle_row_exponent(_ptr(X), rows, K, K, _ptr(e))
    return e


def split_rownorm(X):
    """X float32 [rows, K] -> (hi, res) binary16 bit patterns of x' = x 2^e_r and
    e int32 [rows]: hi = fp16(x'), res = fp16(x' - hi)."""
    X = _c(X, np.float32)
    rows, K = X.shape
    hi = np.empty((rows, K), np.uint16)
    res = np.empty((rows, K), np.uint16)
    e = np.empty(rows, np.int32)
    lib().oracle_split_rownorm(_ptr(X), rows, K, K, _ptr(hi), _ptr(res), _ptr(e))
    return hi, res, e


def gemm_rownorm_model(A, W, w_layout="nk", norm_w=True):
    """Representation model of the compensated GEMM on row-normalized operands
    (diagnostic): (A'_hi.B'_hi + A'_hi.B'_res + A'_res.B'_hi) 2^-(e_a + e_b) in
    binary64, the three 16-bit products of the paper's expansion.  norm_w =
    False leaves B unnormalized (e_b = 0), as for a weight held in binary16."""
    A = _c(A, np.float32)
    Wn = _c(W, np.float32) if w_layout == "nk" else np.ascontiguousarray(np.asarray(W, np.float32).T)
    ah, ar, ea = split_rownorm(A)
    if norm_w:
        bh, br, eb = split_rownorm(Wn)
    else:
        bh, br = split_f16(Wn)
        br = np.zeros_like(br)
        eb = np.zeros(Wn.shape[0], np.int32)
    f = f16_bits_to_f64
    C = f(ah) @ f(bh).T + f(ah) @ f(br).T + f(ar) @ f(bh).T
    return np.ldexp(C, -(ea[:, None] + eb[None, :]).astype(np.int64))


# --- GEMM -----------------------------------------------------------------------

def _gemm_args(A, W, w_layout):
    A = _c(A, np.float32)
    W = _c(W, np.float32)
    M, K = A.shape
    if w_layout == "nk":
        N, K2 = W.shape
        w_kn = 0
    elif w_layout == "kn":
        K2, N = W.shape
        w_kn = 1
    else:
        raise ValueError(w_layout)
    if K2 != K:
        raise ValueError("inner dimensions differ")
    return A, W, M, N, K, w_kn


def gemm_f64(A, W, w_layout="nk"):
    """C64 = A . B in binary64, B = W^T for W [N,K] ('nk') or B = W for W [K,N] ('kn')."""
    A, W, M, N, K, w_kn = _gemm_args(A, W, w_layout)
    C = np.empty((M, N), np.float64)
    lib().oracle_gemm_f64(_ptr(A), K, _ptr(W), W.shape[1], w_kn, _ptr(C), N, M, N, K)
    return C


def gemm_f32_naive(A, W, w_layout="nk"):
    A, W, M, N, K, w_kn = _gemm_args(A, W, w_layout)
    C = np.empty((M, N), np.float32)
    lib().oracle_gemm_f32_naive(_ptr(A), K, _ptr(W), W.shape[1], w_kn, _ptr(C), N, M, N, K)
    return C


def gemm_comp_model(A, W, w_layout="nk"):
    A, W, M, N, K, w_kn = _gemm_args(A, W, w_layout)
    C = np.empty((M, N), np.float64)
    lib().oracle_gemm_comp_model(_ptr(A), K, _ptr(W), W.shape[1], w_kn, _ptr(C), N, M, N, K)
    return C


def gemm_f64_rows(A, W, rows, w_layout="nk"):
    """Rows `rows` of the binary64 product (for shapes too large to do whole)."""
    A, W, M, N, K, w_kn = _gemm_args(A, W, w_layout)
    rows = _c(rows, np.int64)
    C = np.empty((rows.size, N), np.float64)
    lib().oracle_gemm_f64_rows(_ptr(A), K, _ptr(W), W.shape[1], w_kn, _ptr(rows), rows.size,
                               _ptr(C), N, N, K)
    return C


def gemm_f32_naive_rows(A, W, rows, w_layout="nk"):
    A, W, M, N, K, w_kn = _gemm_args(A, W, w_layout)
    rows = _c(rows, np.int64)
    C = np.empty((rows.size, N), np.float32)
    lib().oracle_gemm_f32_naive_rows(_ptr(A), K, _ptr(W), W.shape[1], w_kn, _ptr(rows), rows.size,
                                     _ptr(C), N, N, K)
    return C


def round_f16(x):
    """Operands rounded to binary16 (the oracle's own conversion), held exactly in float32."""
    return f16_bits_to_f64(f32_to_f16_bits(x)).astype(np.float32)


def gemm_f16_plain_rows(A, W, rows, w_layout="nk"):
    """Plain FP16 GEMM (one product): rows of fp16(A) . fp16(B) in binary64.
    HEAL paper, section 3, "Mitigating GEMM Truncation via FP16 Promotion and
    Algebraic Compensation": the single FP16 product that the compensation
    extends.  Products of binary16 values are exact, so this is the exact
    result of that product; a GPU run differs from it by its fp32 accumulation
    only.  Returns (C64 rows, naive-fp32 rows of the same rounded operands)."""
    Ah, Wh = round_f16(A), round_f16(W)
    return gemm_f64_rows(Ah, Wh, rows, w_layout), gemm_f32_naive_rows(Ah, Wh, rows, w_layout)


# --- BF16 three-way split (precision mode) ---------------------------------------
#
# A precision-mode variant of the same compensation (HEAL paper, section 3,
# "Mitigating GEMM Truncation via FP16 Promotion and Algebraic Compensation":
# an fp32 operand written as a sum of 16-bit parts, products accumulated in
# fp32).  bfloat16 keeps fp32's exponent range with 8 significant bits, so three
# parts are needed to hold an fp32 significand.

def round_bf16(x):
    """Values rounded to bfloat16 (8 significant bits, exponent range of
    binary32, subnormal quantum 2^-133), to nearest with ties to even; returned
    exactly as float64.  From the format's definition: the value is scaled by a
    power of two so that its kept bits form the integer part, rounded by
    numpy's rint (ties to even) and scaled back; results at or above 2^128 in
    magnitude overflow to infinity."""
    x = np.asarray(x, np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)                    # |x| in [2^(e-1), 2^e)
    q = np.maximum(e - 8, -133)            # quantum of 8 significant bits, or the subnormal one
    y = np.ldexp(np.rint(np.ldexp(xf, -q)), q)
    y = np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, xf), y)
    out[fin] = y
    return out


def split_bf16x3(x):
    """x (float32) -> (b0, b1, b2) float64 with b0 = bf16(x), b1 = bf16(x - b0),
    b2 = bf16(x - b0 - b1); the residuals are exact, and the parts sum to x
    exactly while the last one stays a normal bf16 (|x| above about 2^-110)."""
    x = np.asarray(x, np.float32).astype(np.float64)
    b0 = round_bf16(x)
    r1 = x - b0
    b1 = round_bf16(r1)
    b2 = round_bf16(r1 - b1)
    return b0, b1, b2


def gemm_bf16x3_model(A, W, w_layout="nk"):
    """The six-product BF16 GEMM: sum over i + j <= 2 of A_i . B_j, in binary64
    (products of bf16 parts are exact).  A GPU run differs from it by its fp32
    accumulation only.  B = W^T ('nk') or W ('kn')."""
    A = np.asarray(A, np.float32)
    B = np.asarray(W, np.float32)
    B = B.T if w_layout == "nk" else B
    a = split_bf16x3(A)
    b = split_bf16x3(B)
    C = np.zeros((A.shape[0], B.shape[1]), np.float64)
    for i in range(3):
        for j in range(3 - i):
            C += a[i] @ b[j]
    return C


# --- INT16 quant / dequant ----------------------------------------------------

def quant_i16(X):
    """X float32 [..., D] -> (codes int16 [..., D], scales float32 [...]), one scale per row."""
    X = _c(X, np.float32)
    D = X.shape[-1]
    rows = X.size // D if D else 0
    codes = np.empty(X.shape, np.int16)
    scales = np.empty(X.shape[:-1], np.float32)
    lib().oracle_quant_i16(_ptr(X), rows, D, D, _ptr(codes), D, _ptr(scales))
    return codes, scales


def dequant_f32(codes, scales):
    codes = _c(codes, np.int16)
    scales = _c(scales, np.float32)
    D = codes.shape[-1]
    rows = codes.size // D if D else 0
    out = np.empty(codes.shape, np.float32)
    lib().oracle_dequant_f32(_ptr(codes), rows, D, D, _ptr(scales), _ptr(out), D)
    return out


def dequant_f16x2(codes):
    codes = _c(codes, np.int16)
    D = codes.shape[-1]
    rows = codes.size // D if D else 0
    hi = np.empty(codes.shape, np.uint16)
    lo = np.empty(codes.shape, np.uint16)
    lib().oracle_dequant_f16x2(_ptr(codes), rows, D, D, _ptr(hi), _ptr(lo), D)
    return hi, lo


# --- decode attention -----------------------------------------------------------

def _attn_args(q, qs, k, ks, v, vs):
    q = _c(q, np.int16); qs = _c(qs, np.float32)
    k = _c(k, np.int16); ks = _c(ks, np.float32)
    v = _c(v, np.int16); vs = _c(vs, np.float32)
    B, Hq, D = q.shape
    B2, T, Hkv, D2 = k.shape
    if B2 != B or D2 != D or v.shape != k.shape or Hq % Hkv:
        raise ValueError("attention shapes")
    return q, qs, k, ks, v, vs, B, T, Hq, Hkv, D


def attn_decode_f64(q, qs, k, ks, v, vs):
    """q [B,Hq,D] int16 + qs [B,Hq]; k, v [B,T,Hkv,D] int16 + [B,T,Hkv] -> o [B,Hq,D] float64."""
    q, qs, k, ks, v, vs, B, T, Hq, Hkv, D = _attn_args(q, qs, k, ks, v, vs)
    out = np.empty((B, Hq, D), np.float64)
    lib().oracle_attn_decode_f64(_ptr(q), _ptr(qs), _ptr(k), _ptr(ks), _ptr(v), _ptr(vs),
                                 _ptr(out), B, T, Hq, Hkv, D)
    return out


def attn_decode_weight_norm(q, qs, k, ks, v, vs):
    q, qs, k, ks, v, vs, B, T, Hq, Hkv, D = _attn_args(q, qs, k, ks, v, vs)
    out = np.empty((B, Hq, D), np.float64)
    lib().oracle_attn_decode_weight_norm(_ptr(q), _ptr(qs), _ptr(k), _ptr(ks), _ptr(v), _ptr(vs),
                                         _ptr(out), B, T, Hq, Hkv, D)
    return out


def attn_decode_f32_naive(q, qs, k, ks, v, vs):
    q, qs, k, ks, v, vs, B, T, Hq, Hkv, D = _attn_args(q, qs, k, ks, v, vs)
    out = np.empty((B, Hq, D), np.float32)
    lib().oracle_attn_decode_f32_naive(_ptr(q), _ptr(qs), _ptr(k), _ptr(ks), _ptr(v), _ptr(vs),
                                       _ptr(out), B, T, Hq, Hkv, D)
    return out


def _prefill_positions(q, qs, k, ks, v, vs, positions, fn):
    """Causal prefill attention = decode attention of query t over keys 0 .. t:
    q [B,T,Hq,D] + qs [B,T,Hq]; k, v [B,T,Hkv,D] + [B,T,Hkv] -> [B, len(positions), Hq, D]."""
    q, k, v = _c(q, np.int16), _c(k, np.int16), _c(v, np.int16)
    qs, ks, vs = _c(qs, np.float32), _c(ks, np.float32), _c(vs, np.float32)
    outs = []
    for t in positions:
        outs.append(fn(q[:, t], qs[:, t], k[:, :t + 1], ks[:, :t + 1], v[:, :t + 1], vs[:, :t + 1]))
    return np.stack(outs, axis=1)


def attn_prefill_f64(q, qs, k, ks, v, vs, positions):
    """Causal self-attention of a prompt at query positions `positions` (binary64):
    HEAL paper, section 3, "Mitigating QKV Truncation Error via INT16 Quantization",
    applied to every prefix; each position is the decode reference over keys 0 .. t."""
    return _prefill_positions(q, qs, k, ks, v, vs, positions, attn_decode_f64)


def attn_prefill_f32_naive(q, qs, k, ks, v, vs, positions):
    return _prefill_positions(q, qs, k, ks, v, vs, positions, attn_decode_f32_naive)


def attn_prefill_weight_norm(q, qs, k, ks, v, vs, positions):
    return _prefill_positions(q, qs, k, ks, v, vs, positions, attn_decode_weight_norm)
