"""Error measures used by the parity tests (test code, no method arithmetic)."""
import numpy as np


def gemm_normwise_error(C, C64, A, W, w_layout="nk", rows=None):
    """max_ij |C_ij - C64_ij| / (||a_i||_2 ||b_j||_2), b_j = column j of B.

    This is the error a GEMM commits relative to the Cauchy-Schwarz bound of its
    output; unlike the elementwise relative error it stays finite under
    cancellation.  `rows` selects the rows of A that C and C64 hold.
    """
    A64 = np.asarray(A, np.float64)
    if rows is not None:
        A64 = A64[np.asarray(rows)]
    W64 = np.asarray(W, np.float64)
    bn = np.linalg.norm(W64, axis=1) if w_layout == "nk" else np.linalg.norm(W64, axis=0)
    an = np.linalg.norm(A64, axis=1)
    denom = an[:, None] * bn[None, :]
    err = np.abs(np.asarray(C, np.float64) - C64)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(denom > 0, err / np.where(denom > 0, denom, 1.0), np.where(err > 0, np.inf, 0.0))
    return float(r.max()) if r.size else 0.0


def gemm_tolerance(e_naive, K):
    """Pass bar for the compensated GEMM against the binary64 reference.

    * at most 2x the error of a naive FP32 GEMM on the same data, and at most
      1e-5 (normwise);
    * for K < 64 the naive FP32 error is essentially one rounded product
      (2^-24), which no two-part fp16 split (22 significant bits, plus the
      dropped lo.lo term) can match: there the bar adds the split's own
      representation bound 3 * 2^-22 per product.
    """
    bar = 2.0 * e_naive + (3.0 * 2.0 ** -22 if K < 64 else 0.0)
    return min(bar, 1e-5)


def attn_normwise_error(o, o64, weight_norm):
    """max |o - o64| / (sum_t P_t |v_t[d]|), the scale of a positively weighted sum."""
    err = np.abs(np.asarray(o, np.float64) - o64)
    return float((err / np.maximum(weight_norm, 1e-300)).max())
