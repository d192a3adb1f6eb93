/*
 * heal_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU model of what the HEAL hot path
 * computes.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg may load this library; the GPU library never links, calls or
 * includes anything from here, and nothing here comes from the GPU library.
 *
 * Source of the method: "Demystifying Numerical Instability in LLM Inference:
 * Achieving Reproducible Inference for Mission-Critical Tasks with HEAL"
 * (arXiv 2606.21023), cited below as [HEAL <section>, "<paragraph title>"].
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 * -ffp-contract=off keeps every a*b+c as two correctly rounded binary32
 * operations; x86-64 evaluates float arithmetic in SSE registers, so every
 * float operation below is one IEEE-754 binary32 rounding (round to nearest
 * even), and every double operation one binary64 rounding.
 *
 * Parity status of each function (what pins it) is stated at the function.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16, written from the format's definition.                 */
/* ------------------------------------------------------------------------ */

/* Round a binary32 value to the nearest binary16 value, ties to even, keeping
 * subnormals (no flush to zero); values whose rounded magnitude reaches 2^16
 * become infinity.  Returns the 16-bit encoding.
 *
 * binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.  Around
 * a magnitude a in [2^E, 2^(E+1)) with E >= -14 the representable values are
 * spaced 2^(E-10); below 2^-14 (subnormals) they are spaced 2^-24.  Rounding
 * is therefore "divide by the spacing, round to an integer (ties to even),
 * multiply back" -- all exact in binary64 except the integer rounding, which
 * rint() performs in the default round-to-nearest-even mode.
 * Pinned against numpy's float32->float16 conversion and the format's
 * boundary values.                                                          */
static uint16_t f32_to_f16_bits(float xf)
{
    double x = (double)xf;                       /* exact widening */
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isnan(a)) return (uint16_t)(sign | 0x7e00u);
    if (isinf(a)) return (uint16_t)(sign | 0x7c00u);
    if (a == 0.0) return sign;

    int e2;
    (void)frexp(a, &e2);                         /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < -14) E = -14;                        /* subnormal spacing 2^-24 */
    double spacing = ldexp(1.0, E - 10);
    double m = rint(a / spacing);                /* integer multiple of spacing */
    double r = m * spacing;                      /* the rounded magnitude */
    if (r >= 65536.0) return (uint16_t)(sign | 0x7c00u);   /* overflow */

    if (r < ldexp(1.0, -14)) {
        /* subnormal: fraction = r / 2^-24, exponent field 0 */
        return (uint16_t)(sign | (uint16_t)m);
    }
    /* normal: r = (1 + f/1024) * 2^Er with Er in [-14, 15] */
    int er2;
    (void)frexp(r, &er2);
    int Er = er2 - 1;
    double frac = r / ldexp(1.0, Er) - 1.0;      /* in [0, 1), a multiple of 2^-10 */
    uint16_t f = (uint16_t)(frac * 1024.0);
    return (uint16_t)(sign | (uint16_t)((Er + 15) << 10) | f);
}

/* Value of a binary16 encoding (exact in binary64). */
static double f16_bits_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)       v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else              v = ldexp(1024.0 + (double)f, e - 25);
    return s ? -v : v;
}

ORACLE_API void oracle_f32_to_f16(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16_bits(x[i]);
}

ORACLE_API void oracle_f16_to_f64(const uint16_t* h, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = f16_bits_to_f64(h[i]);
}

/* ------------------------------------------------------------------------ */
/* Operand split: x ~= hi + lo / 2^10, both parts binary16.                 */
/* [HEAL §3, "Mitigating GEMM Truncation via FP16 Promotion and Algebraic   */
/*  Compensation"]: the FP32 input h is decomposed as h_hi + h_lo/2^10.     */
/* [HEAL §3, "Mitigating QKV Truncation Error via INT16 Quantization"]: the */
/*  same dual-FP16 pairing, lower part shifted by 2^10.                      */
/* The pages give the decomposition, not its rounding; the plain reading   */
/* taken here: hi is x rounded to binary16, the residual x - hi is formed   */
/* in binary32 (exact: it needs at most 12 significant bits), scaled by     */
/* 2^10 (exact) and rounded to binary16.                                    */
/* Pinned by the closed-form bound |x - (hi + lo/2^10)| <= 2^-22|x| + 2^-35 */
/* (|x| < 65504) and by lo == 0 whenever x is binary16-representable.       */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_split_f16(const float* x, int64_t n, uint16_t* hi, uint16_t* lo)
{
    for (int64_t i = 0; i < n; ++i) {
        uint16_t h = f32_to_f16_bits(x[i]);
        float hv = (float)f16_bits_to_f64(h);    /* exact: binary16 fits binary32 */
        float r = x[i] - hv;                     /* one binary32 rounding (exact for finite, in-range x) */
        float rs = r * 1024.0f;                  /* exact power-of-two scaling */
        hi[i] = h;
        lo[i] = f32_to_f16_bits(rs);
    }
}

/* ------------------------------------------------------------------------ */
/* GEMM references.  C[M,N] = A[M,K] . B[K,N] where B is given either as    */
/* W[N,K] (w_kn == 0, the layout of a linear layer's weight: B = W^T) or    */
/* as W[K,N] (w_kn == 1).  Leading dimensions are in elements.              */
/* ------------------------------------------------------------------------ */
static inline float wget(const float* W, int64_t ldw, int w_kn, int64_t k, int64_t j)
{
    return w_kn ? W[k * ldw + j] : W[j * ldw + k];
}

/* FP64-accumulated GEMM: the reference answer.  Each product of two binary32
 * values is exact in binary64 (24 + 24 <= 53 significant bits); only the
 * sums round, so |C64 - exact| <= K * 2^-53 * sum_k |a_ik b_kj| (to first
 * order).  Pinned against exact rational arithmetic on small shapes.       */
ORACLE_API void oracle_gemm_f64(const float* A, int64_t lda, const float* W, int64_t ldw,
                                int w_kn, double* C, int64_t ldc,
                                int64_t M, int64_t N, int64_t K)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += (double)A[i * lda + k] * (double)wget(W, ldw, w_kn, k, j);
            C[i * ldc + j] = s;
        }
    }
}

/* Same contraction on a subset of rows: C[r, :] = A[rows[r], :] . B.
 * Used where the full product is too slow for a CPU (large prefill shapes). */
ORACLE_API void oracle_gemm_f64_rows(const float* A, int64_t lda, const float* W, int64_t ldw,
                                     int w_kn, const int64_t* rows, int64_t nrows,
                                     double* C, int64_t ldc, int64_t N, int64_t K)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const float* a = A + rows[r] * lda;
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += (double)a[k] * (double)wget(W, ldw, w_kn, k, j);
            C[r * ldc + j] = s;
        }
    }
}

/* Naive FP32 GEMM: sequential k, a separate binary32 multiply and add per
 * term, no fused multiply-add.  It defines the error level of a plain FP32
 * pipeline, against which the compensated GEMM's tolerance is set.
 * Pinned: equals the FP64 GEMM bit-for-bit when every partial sum is
 * exact (small integers), and a three-term case that fixes the order.      */
ORACLE_API void oracle_gemm_f32_naive(const float* A, int64_t lda, const float* W, int64_t ldw,
                                      int w_kn, float* C, int64_t ldc,
                                      int64_t M, int64_t N, int64_t K)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            float s = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                float p = A[i * lda + k] * wget(W, ldw, w_kn, k, j);
                s = s + p;
            }
            C[i * ldc + j] = s;
        }
    }
}

ORACLE_API void oracle_gemm_f32_naive_rows(const float* A, int64_t lda, const float* W, int64_t ldw,
                                           int w_kn, const int64_t* rows, int64_t nrows,
                                           float* C, int64_t ldc, int64_t N, int64_t K)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const float* a = A + rows[r] * lda;
        for (int64_t j = 0; j < N; ++j) {
            float s = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                float p = a[k] * wget(W, ldw, w_kn, k, j);
                s = s + p;
            }
            C[r * ldc + j] = s;
        }
    }
}

/* Representation model of the compensated GEMM (diagnostic): split both
 * operands as above, then form hi.hi + 2^-10 (hi.lo + lo.hi) with every
 * product and sum in binary64.  It carries the method's representation
 * error but none of a device's accumulation order, so a device result far
 * from this model points at the kernel, not at the split.
 * [HEAL §3, "Mitigating GEMM Truncation via FP16 Promotion and Algebraic
 *  Compensation"] expands the product into 16-bit products; with both
 * operands in FP32 the expansion has the three terms used here.           */
ORACLE_API void oracle_gemm_comp_model(const float* A, int64_t lda, const float* W, int64_t ldw,
                                       int w_kn, double* C, int64_t ldc,
                                       int64_t M, int64_t N, int64_t K)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double hh = 0.0, cc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                float a = A[i * lda + k], b = wget(W, ldw, w_kn, k, j);
                uint16_t ah, al, bh, bl;
                oracle_split_f16(&a, 1, &ah, &al);
                oracle_split_f16(&b, 1, &bh, &bl);
                double ahv = f16_bits_to_f64(ah), alv = f16_bits_to_f64(al);
                double bhv = f16_bits_to_f64(bh), blv = f16_bits_to_f64(bl);
                hh += ahv * bhv;
                cc += ahv * blv + alv * bhv;
            }
            C[i * ldc + j] = hh + cc / 1024.0;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Row normalization by a power of two, and the split of a normalized row.  */
/* [HEAL §3, "Mitigating GEMM Truncation via FP16 Promotion and Algebraic   */
/*  Compensation"]: FP16's narrow dynamic range is the method's weak point  */
/*  (values beyond it overflow, values below it lose bits), and the pages   */
/*  answer it by targeted rescaling.  Reading taken: every operand row is   */
/*  multiplied by the power of two 2^e that brings its largest magnitude    */
/*  into [2^14, 2^15) -- the top binade that cannot round past 65504 --     */
/*  before its split, and the product is multiplied back by 2^-(e_a + e_b). */
/*  Powers of two are exact in binary floating point, so the product is    */
/*  unchanged; the split then sees every significant element of the row in  */
/*  FP16's normal range, whatever the row's own scale.                      */
/* ------------------------------------------------------------------------ */

/* e = 14 - floor(log2(max_k |x_k|)), so that 2^14 <= max * 2^e < 2^15;
 * e = 0 for a row of zeros.  frexp gives max = f * 2^p with f in [0.5, 1),
 * i.e. floor(log2(max)) = p - 1, exactly, subnormal binary32 included.
 * Pinned by the defining inequality on rows spanning binary32's range.    */
static int32_t row_exponent(const float* x, int64_t K)
{
    double m = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double a = fabs((double)x[k]);
        if (a > m) m = a;
    }
    if (m == 0.0) return 0;
    int p;
    (void)frexp(m, &p);
    return 14 - (p - 1);
}

ORACLE_API void oracle_row_exponent(const float* X, int64_t rows, int64_t K, int64_t ldx, int32_t* e)
{
    for (int64_t r = 0; r < rows; ++r) e[r] = row_exponent(X + r * ldx, K);
}

/* Split of a normalized row: x' = x * 2^e (binary32, rounded once: exact
 * unless it falls below binary32's subnormal quantum), hi = rne16(x'),
 * res = rne16(x' - hi) with x' - hi exact in binary32.  This is the dual-FP16
 * pair of the pages with the residual kept at its own scale: res equals
 * lo / 2^10 of oracle_split_f16(x') whenever that is a normal binary16, which
 * on a normalized row holds for every element above 2^-17 of the row's
 * largest.  Pinned against numpy's binary16 conversion and against
 * oracle_split_f16.                                                        */
ORACLE_API void oracle_split_rownorm(const float* X, int64_t rows, int64_t K, int64_t ldx,
                                     uint16_t* hi, uint16_t* res, int32_t* e)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float* x = X + r * ldx;
        int32_t er = row_exponent(x, K);
        e[r] = er;
        for (int64_t k = 0; k < K; ++k) {
            float xs = (float)ldexp((double)x[k], er);
            uint16_t h = f32_to_f16_bits(xs);
            float rr = xs - (float)f16_bits_to_f64(h);
            hi[r * K + k] = h;
            res[r * K + k] = f32_to_f16_bits(rr);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* INT16 quantizer.                                                         */
/* [HEAL §3, "Mitigating QKV Truncation Error via INT16 Quantization"]:     */
/*  Q_INT16(X) = Round((2^15 - 1) X / max|X|), step Delta = M / (2^15 - 1). */
/* Readings where the pages are silent (each listed in the design notes):   */
/*  - one max per contiguous row of length D (per token, per head);         */
/*  - Round is round-half-to-even (the pages state unbiased RNE hardware);  */
/*  - the formula's order: t = fl(32767 * x), then u = fl(t / M), then RNE; */
/*  - a row of zeros (M == 0) gives scale 0 and codes 0;                    */
/*  - the stored scale is s = fl(M / 32767) (binary32).                     */
/* Codes lie in [-32767, 32767]; -32768 is never produced on finite input.  */
/* Pinned: absmax -> +-32767, odd symmetry, exact rational rounding away    */
/* from ties, the error bounds, and the uniform-error MSE Delta^2/12.      */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_quant_i16(const float* X, int64_t rows, int64_t D, int64_t ldx,
                                 int16_t* codes, int64_t ldq, float* scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* x = X + r * ldx;
        int16_t* q = codes + r * ldq;
        float M = 0.0f;
        for (int64_t d = 0; d < D; ++d) {
            float a = fabsf(x[d]);
            if (a > M) M = a;
        }
        if (M == 0.0f) {
            scales[r] = 0.0f;
            for (int64_t d = 0; d < D; ++d) q[d] = 0;
            continue;
        }
        scales[r] = M / 32767.0f;
        for (int64_t d = 0; d < D; ++d) {
            float t = 32767.0f * x[d];
            float u = t / M;
            q[d] = (int16_t)rintf(u);
        }
    }
}

/* Dequant to binary32: x^ = fl(q * s).                                     */
ORACLE_API void oracle_dequant_f32(const int16_t* codes, int64_t rows, int64_t D, int64_t ldq,
                                   const float* scales, float* out, int64_t ldo)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t d = 0; d < D; ++d)
            out[r * ldo + d] = (float)codes[r * ldq + d] * scales[r];
}

/* Dequant to the dual-FP16 pair of [HEAL §3, "Mitigating QKV Truncation
 * Error via INT16 Quantization"]: the integer code q is written as
 * hi + lo / 2^10 with hi = fp16(q) and lo = fp16((q - hi) * 2^10); both
 * conversions are exact for every int16 code (|q - hi| <= 8, |lo| <= 8192),
 * so the pair carries the code without loss.  The scale is applied later. */
ORACLE_API void oracle_dequant_f16x2(const int16_t* codes, int64_t rows, int64_t D, int64_t ldq,
                                     uint16_t* hi, uint16_t* lo, int64_t ldo)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t d = 0; d < D; ++d) {
            float qv = (float)codes[r * ldq + d];
            uint16_t h = f32_to_f16_bits(qv);
            float rs = (qv - (float)f16_bits_to_f64(h)) * 1024.0f;
            hi[r * ldo + d] = h;
            lo[r * ldo + d] = f32_to_f16_bits(rs);
        }
}

/* ------------------------------------------------------------------------ */
/* Decode attention over INT16 operands.                                    */
/* [HEAL §3, "Mitigating QKV Truncation Error via INT16 Quantization"]:     */
/*  Q, K, V are held as INT16 codes with a scale per row; attention runs on */
/*  the dequantized values.  One query token per sequence; grouped-query    */
/*  attention maps query head h to KV head h / (Hq / Hkv).                  */
/* Layouts: q [B, Hq, D] codes + [B, Hq] scales; k, v [B, T, Hkv, D] codes  */
/*  + [B, T, Hkv] scales; out [B, Hq, D].  Softmax scale 1/sqrt(D).        */
/* FP64 version: operands x~ = (double)q * (double)s (exact), scores,       */
/*  max-subtracted softmax and the weighted sum all in binary64.            */
/* Pinned: T = 1 gives o = v~ exactly; equal scores give the mean of v~.    */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_attn_decode_f64(const int16_t* q, const float* qs,
                                       const int16_t* k, const float* ks,
                                       const int16_t* v, const float* vs,
                                       double* out, int64_t B, int64_t T,
                                       int64_t Hq, int64_t Hkv, int64_t D)
{
    int64_t group = Hq / Hkv;
    double inv_sqrt_d = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < Hq; ++h) {
            int64_t g = h / group;
            const int16_t* qc = q + (b * Hq + h) * D;
            double qscale = (double)qs[b * Hq + h];
            double m = -INFINITY;
            /* pass 1: the maximum score */
            for (int64_t t = 0; t < T; ++t) {
                int64_t row = (b * T + t) * Hkv + g;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += ((double)qc[d] * qscale) * ((double)k[row * D + d] * (double)ks[row]);
                double sc = dot * inv_sqrt_d;
                if (sc > m) m = sc;
            }
            /* pass 2: weights, normaliser and weighted sum */
            double l = 0.0;
            double* o = out + (b * Hq + h) * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                int64_t row = (b * T + t) * Hkv + g;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += ((double)qc[d] * qscale) * ((double)k[row * D + d] * (double)ks[row]);
                double p = exp(dot * inv_sqrt_d - m);
                l += p;
                for (int64_t d = 0; d < D; ++d)
                    o[d] += p * ((double)v[row * D + d] * (double)vs[row]);
            }
            for (int64_t d = 0; d < D; ++d) o[d] /= l;
        }
    }
}

/* Weight statistics for the attention tolerance: for each (b, h, d),
 * norm[b,h,d] = sum_t P_t |v~_t[d]| with P the FP64 softmax weights.  A
 * weighted sum with these positive weights has an absolute rounding error
 * proportional to this quantity, so errors are measured relative to it.   */
ORACLE_API void oracle_attn_decode_weight_norm(const int16_t* q, const float* qs,
                                               const int16_t* k, const float* ks,
                                               const int16_t* v, const float* vs,
                                               double* norm, int64_t B, int64_t T,
                                               int64_t Hq, int64_t Hkv, int64_t D)
{
    int64_t group = Hq / Hkv;
    double inv_sqrt_d = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < Hq; ++h) {
            int64_t g = h / group;
            const int16_t* qc = q + (b * Hq + h) * D;
            double qscale = (double)qs[b * Hq + h];
            double m = -INFINITY;
            for (int64_t t = 0; t < T; ++t) {
                int64_t row = (b * T + t) * Hkv + g;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += ((double)qc[d] * qscale) * ((double)k[row * D + d] * (double)ks[row]);
                double sc = dot * inv_sqrt_d;
                if (sc > m) m = sc;
            }
            double l = 0.0;
            double* o = norm + (b * Hq + h) * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                int64_t row = (b * T + t) * Hkv + g;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += ((double)qc[d] * qscale) * ((double)k[row * D + d] * (double)ks[row]);
                double p = exp(dot * inv_sqrt_d - m);
                l += p;
                for (int64_t d = 0; d < D; ++d)
                    o[d] += p * fabs((double)v[row * D + d] * (double)vs[row]);
            }
            for (int64_t d = 0; d < D; ++d) o[d] /= l;
        }
    }
}

/* Naive FP32 decode attention on the FP32-dequantized operands fl(q * s):
 * sequential loops, a separate binary32 multiply and add per term, expf.
 * It is what a plain FP32 pipeline holding these operands computes, and it
 * sets the error level for the attention tolerance.                        */
ORACLE_API void oracle_attn_decode_f32_naive(const int16_t* q, const float* qs,
                                             const int16_t* k, const float* ks,
                                             const int16_t* v, const float* vs,
                                             float* out, int64_t B, int64_t T,
                                             int64_t Hq, int64_t Hkv, int64_t D)
{
    int64_t group = Hq / Hkv;
    float inv_sqrt_d = 1.0f / sqrtf((float)D);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < Hq; ++h) {
            int64_t g = h / group;
            const int16_t* qc = q + (b * Hq + h) * D;
            float qscale = qs[b * Hq + h];
            float m = -INFINITY;
            for (int64_t t = 0; t < T; ++t) {
                int64_t row = (b * T + t) * Hkv + g;
                float dot = 0.0f;
                for (int64_t d = 0; d < D; ++d) {
                    float p = ((float)qc[d] * qscale) * ((float)k[row * D + d] * ks[row]);
                    dot = dot + p;
                }
                float sc = dot * inv_sqrt_d;
                if (sc > m) m = sc;
            }
            float l = 0.0f;
            float* o = out + (b * Hq + h) * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0f;
            for (int64_t t = 0; t < T; ++t) {
                int64_t row = (b * T + t) * Hkv + g;
                float dot = 0.0f;
                for (int64_t d = 0; d < D; ++d) {
                    float p = ((float)qc[d] * qscale) * ((float)k[row * D + d] * ks[row]);
                    dot = dot + p;
                }
                float p = expf(dot * inv_sqrt_d - m);
                l = l + p;
                for (int64_t d = 0; d < D; ++d) {
                    float pv = p * ((float)v[row * D + d] * vs[row]);
                    o[d] = o[d] + pv;
                }
            }
            for (int64_t d = 0; d < D; ++d) o[d] = o[d] / l;
        }
    }
}

ORACLE_API int oracle_abi_version(void) { return 1; }

/* Threads the OpenMP loops above run on (for reporting CPU timings). */
ORACLE_API int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Set the OpenMP thread count of the loops above (CPU timings on 1 core). */
ORACLE_API void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
