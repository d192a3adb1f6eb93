"""Seeded synthetic inputs for the HEAL hot path (no method arithmetic here).

Both the CPU oracle side and the GPU side of every test, and the benchmark,
draw their inputs from these functions; nothing here quantizes, splits or
multiplies the way the method does.  Generator: numpy PCG64 with an explicit
seed; by convention seed = 1000 * workload number + shape index.

The HEAL paper measures on MedQA, MCR-Bench and ShareGPT with trained
Qwen3 / Llama weights.  None of those are used: these synthetic tensors
stand in for them with the model shapes and value distributions below
(outlier activation channels, small Gaussian weights, per-head magnitude
spread for Q/K/V).
"""
import numpy as np

# Model shapes the workloads take their sizes from.
LLAMA3_8B_DECODE_KN = [(4096, 4096), (4096, 1024), (4096, 14336), (14336, 4096)]
DECODE_M = [1, 8, 32, 64]
PREFILL_M = 2048
PREFILL_KN = [(4096, 14336), (14336, 4096)]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(g: np.random.Generator, shape, std=1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def activations(M: int, K: int, seed: int, n_outlier: int, outlier_gain: float) -> np.ndarray:
    """A [M, K] ~ N(0, 1) with `n_outlier` randomly chosen channels (columns)
    multiplied by `outlier_gain` (outlier / massive-activation channels)."""
    g = rng(seed)
    A = normal(g, (M, K))
    if n_outlier:
        cols = g.choice(K, size=n_outlier, replace=False)
        A[:, cols] *= np.float32(outlier_gain)
    return A


def weights_nk(N: int, K: int, seed: int, std: float = 0.02) -> np.ndarray:
    """Linear-layer weight W [N, K] ~ N(0, std^2) (row n holds output n)."""
    return normal(rng(seed), (N, K), std)


def overflow_gemm(M: int, K: int, N: int, seed: int):
    """Linear layer whose activation has massive channels beyond FP16's range:
    round(0.005 K) channels (the pages report 0.1-1% of fixed channels) x 2e5,
    so |x| reaches ~1e6 > 65504; W ~ N(0, 0.02^2)."""
    n_out = max(1, int(round(0.005 * K)))
    A = activations(M, K, seed, n_outlier=n_out, outlier_gain=2.0e5)
    W = weights_nk(N, K, seed + 500)
    return A, W


def smoke_gemm(seed: int = 1000):
    """Small case: A 16x256 ~ N(0,1) with 2 channels x100; W [256,256] ~ N(0, 0.02)."""
    A = activations(16, 256, seed, n_outlier=2, outlier_gain=100.0)
    W = weights_nk(256, 256, seed + 500)
    return A, W


def smoke_quant(seed: int = 1001):
    """Small case: a 16 x 256 tensor ~ N(0,1), one scale per row of 256."""
    return normal(rng(seed), (16, 256))


def decode_gemm(M: int, K: int, N: int, seed: int):
    """Decode-shaped linear layer: activations with round(0.001 K) channels x50."""
    n_out = int(round(0.001 * K))
    A = activations(M, K, seed, n_outlier=n_out, outlier_gain=50.0)
    W = weights_nk(N, K, seed + 500)
    return A, W


def prefill_gemm(M: int, K: int, N: int, seed: int):
    """Prefill-shaped linear layer: 4 massive-activation channels x1000."""
    A = activations(M, K, seed, n_outlier=4, outlier_gain=1000.0)
    W = weights_nk(N, K, seed + 500)
    return A, W


def qkv(tokens: int, Hq: int, Hkv: int, D: int, seed: int):
    """Q [tokens, Hq, D], K and V [tokens, Hkv, D], ~ N(0,1) times a factor per
    (tensor, head) drawn log-uniformly in [0.1, 30] and shared by all tokens."""
    g = rng(seed)
    out = []
    for H in (Hq, Hkv, Hkv):
        gain = np.exp(g.uniform(np.log(0.1), np.log(30.0), size=H)).astype(np.float32)
        X = normal(g, (tokens, H, D))
        X *= gain[None, :, None]
        out.append(X)
    return tuple(out)


def attention_prefill_fp32(B: int, T: int, Hq: int, Hkv: int, D: int, seed: int):
    """Prefill attention inputs before quantization: q [B,T,Hq,D], k and v
    [B,T,Hkv,D], all ~ N(0,1)."""
    g = rng(seed)
    q = normal(g, (B, T, Hq, D))
    k = normal(g, (B, T, Hkv, D))
    v = normal(g, (B, T, Hkv, D))
    return q, k, v


def attention_fp32(B: int, T: int, Hq: int, Hkv: int, D: int, seed: int):
    """Decode attention inputs before quantization: q [B,Hq,D], k and v
    [B,T,Hkv,D], all ~ N(0,1)."""
    g = rng(seed)
    q = normal(g, (B, Hq, D))
    k = normal(g, (B, T, Hkv, D))
    v = normal(g, (B, T, Hkv, D))
    return q, k, v
