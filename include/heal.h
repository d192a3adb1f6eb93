/*
 * heal.h -- C ABI of the HEAL hot path on AMD Instinct MI355X (gfx950).
 *
 * HEAL ("Hybrid Error ALleviation") comes from the paper "Demystifying
 * Numerical Instability in LLM Inference: Achieving Reproducible Inference
 * for Mission-Critical Tasks with HEAL" (arXiv 2606.21023).  Citations
 * below name its sections and paragraph titles:
 *   [INT16]  section 3, "Mitigating QKV Truncation Error via INT16 Quantization"
 *   [GEMM]   section 3, "Mitigating GEMM Truncation via FP16 Promotion and
 *            Algebraic Compensation"
 *
 * The library gives FP32-grade linear-layer products without an FP32
 * pipeline, and FP32-grade attention operands without doubling the KV cache
 * (section 1, "Key Insight"; section 3 opening).
 *
 * Conventions shared by every call
 *  - Pointers named as device pointers are device memory owned by the caller.
 *    The library never allocates, frees or synchronizes.  Scratch memory is
 *    the caller's `workspace`, sized by the matching *_workspace call, except
 *    for heal_gemm_f32c_noalloc, whose scratch is a fixed device array of the
 *    library (one per GPU, 16 MiB).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Each call enqueues its kernels on that stream and returns at once.
 *  - Matrices are row-major.  Leading dimensions (ld*) count elements.
 *  - Arguments are validated on the host before any HIP call.  A failed check
 *    returns its code and touches no device state.  A dimension of 0 is
 *    valid and makes the call a no-op, except where a call says otherwise.
 *  - Conditions that depend on the data never fail a call.  They set bits in
 *    an optional device status word (HEAL_FLAG_*) with an atomic OR.
 *  - NaN and Inf inputs are outside the numerical contract.  They never
 *    crash a call, and their results follow IEEE-754.
 *  - Calls are thread-safe.  Concurrent calls must use distinct output and
 *    workspace buffers, or the calls race.
 */
#ifndef HEAL_H
#define HEAL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum heal_status {
    HEAL_OK = 0,
    HEAL_ERR_NULL = 1,        /* a required pointer is NULL                              */
    HEAL_ERR_SHAPE = 2,       /* a dimension is negative or outside the supported range  */
    HEAL_ERR_STRIDE = 3,      /* a leading dimension is smaller than its row length      */
    HEAL_ERR_ALIGN = 4,       /* a pointer or leading dimension breaks required alignment */
    HEAL_ERR_UNSUPPORTED = 5, /* unknown flag bits or an unsupported combination         */
    HEAL_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the *_workspace size     */
    HEAL_ERR_HIP = 7          /* the HIP runtime rejected a kernel launch                */
} heal_status;

/* Flags of heal_gemm_f32c / heal_pack_w. */
enum {
    HEAL_W_NK = 0u,     /* W is fp32 [N, K] (a linear layer's weight, B = W^T)          */
    HEAL_W_KN = 1u,     /* W is fp32 [K, N] (B = W)                                     */
    HEAL_W_PACKED = 2u, /* W is a buffer written by heal_pack_w (ldw and layout ignored) */
    HEAL_A_PACKED = 4u, /* A is a buffer written by heal_pack_w for A's M rows (lda ignored) */
    HEAL_W_F16 = 8u,    /* W holds binary16 values (2 bytes each), layout per HEAL_W_KN   */
    HEAL_ONE_PRODUCT = 16u, /* plain FP16: C = A_hi.B_hi only (heal_gemm_f32c)            */
    HEAL_BF16X3 = 32u   /* BF16 three-way split, six products (heal_gemm_f32c, heal_pack_w) */
};

/* Bits of the optional device status word. */
enum {
    HEAL_FLAG_F16_RANGE = 1u, /* a value split as it is (not normalized) has an infinite
                                 16-bit high part: |x| >= 65520 (fp16), or |x| beyond
                                 bf16's largest value (HEAL_BF16X3)                     */
    HEAL_FLAG_SLOT_RANGE = 2u /* a K/V cache slot was >= num_slots: that row was skipped */
};

/* Formats of heal_kv_dequant_i16. */
enum {
    HEAL_DQ_F32 = 0,   /* out: fp32 values fl(q * s)                                  */
    HEAL_DQ_F16X2 = 1  /* out: fp16 hi plane, out_lo: fp16 lo plane, q = hi + lo/2^10 */
};

/* Text for a status code (static storage, never NULL). */
const char* heal_status_str(heal_status s);

/* Library version, (major << 16) | minor. */
int heal_version(void);

/* ------------------------------------------------------------------------
 * heal_split_f32 -- operand split into a dual-FP16 pair.   [GEMM], [INT16]
 *
 * For each of the n fp32 values x:
 *   hi = fp16(x)                      round to nearest even, subnormals kept
 *   lo = fp16((x - hi) * 2^10)        the residual is exact in fp32
 * so that x ~= hi + lo / 2^10, with |x - (hi + lo/2^10)| <= 2^-22|x| + 2^-35
 * for |x| < 65504.
 *   X      device, n fp32 values, 16-byte aligned
 *   hi, lo device, n fp16 bit patterns each, 8-byte aligned
 *   dev_status  device, nullable.  HEAL_FLAG_F16_RANGE is set when some
 *          |x| >= 65520 (hi is then inf, lo is -inf/+inf/NaN per IEEE).
 * Errors: NULL X/hi/lo (when n > 0), n < 0, misalignment.
 * ------------------------------------------------------------------------ */
heal_status heal_split_f32(const float* X, int64_t n, uint16_t* hi, uint16_t* lo,
                           uint32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * heal_gemm_f32c -- FP32-accurate GEMM by algebraic error compensation on
 * 16-bit matrix cores.   [GEMM]
 *
 *   C[M,N] = A[M,K] . B[K,N]      B = W^T (HEAL_W_NK) or B = W (HEAL_W_KN)
 *
 * Both fp32 operands are split as in heal_split_f32.  The product expands to
 *   C = A_hi.B_hi + 2^-10 (A_hi.B_lo + A_lo.B_hi)
 * with the three 16-bit products on fp16 MFMA and fp32 accumulation.  The
 * output stays fp32, so no downcast happens at the kernel boundary.  The
 * lo.lo term (2^-20) is dropped.  FP16's narrow range (the same paragraph:
 * handled by targeted rescaling) is met by exact powers of two: before its
 * split, each row of a packed operand, and each 128-wide k block of each
 * activation row on the M <= 64 path, is multiplied by the 2^e that puts its
 * largest magnitude in [2^14, 2^15), and the product is multiplied back by
 * 2^-e in fp32.  The result does not depend on the activation's scale:
 * scaling a row of A by a power of two scales that row of C by the same
 * power, bit for bit, and the accuracy below holds for activations of any
 * magnitude in fp32's normal range.  With HEAL_W_F16 the weight is already
 * 16-bit (exact in fp16, e.g. an FP16 checkpoint or a BF16 one converted
 * exactly), B_lo is zero and two products remain,
 *   C = A_hi.B + 2^-10 A_lo.B,
 * the paper's own form (section 3, "Mitigating GEMM Truncation via FP16
 * Promotion and Algebraic Compensation"), reading 2 bytes per weight.
 * HEAL_ONE_PRODUCT keeps the first product alone, C = A_hi.B_hi: plain FP16
 * with fp32 accumulation, for layers run without compensation (the paper's
 * HEAL++ upcasts only selected layers; the per-layer choice is the
 * caller's).  Its error is that of FP16 operands, not the bar below.
 * HEAL_BF16X3 is a precision mode for operands FP16's range cannot hold
 * without rescaling: each fp32 operand is split in BF16 (fp32's exponent
 * range) as x = b0 + b1 + b2, b0 = bf16(x), b1 = bf16(x - b0),
 * b2 = bf16(x - b0 - b1), round to nearest even (the sum is exact for
 * |x| above about 2^-110, where the last part is still a normal bf16), and
 *   C = sum over i + j <= 2 of A_i.B_j
 * (six BF16 products, fp32 accumulation; the three dropped terms are below
 * 2^-23 of |a||b|).  fp32 operands only: not with HEAL_W_F16,
 * HEAL_ONE_PRODUCT or a_kshift (UNSUPPORTED); packed operands must come from
 * heal_pack_w with HEAL_BF16X3.  Every M runs the prefill kernel.
 * Accuracy: normwise error max_ij |C - C_exact| / (|a_i| |b_j|)
 * within 2x that of a naive FP32 GEMM and below 1e-5.  The summation order
 * depends on (M, N, K) but not on the data.  For M <= 64 (NK layout or a
 * packed W, A not packed, K < 2^23) it also does not depend on M, so
 * decode-sized results do not change with batch size.
 *
 *   A      device fp32, lda >= K, 4-byte aligned (rows that are 16-byte
 *          aligned, lda % 4 == 0, take 16-byte vector loads)
 *   W      device fp32: [N, K] with ldw >= K (NK) or [K, N] with ldw >= N
 *          (KN), 4-byte aligned (16-byte aligned rows vectorize as for A).
 *          With HEAL_W_F16 the same layouts hold binary16 values (uint16
 *          bit patterns), 2-byte aligned.  With HEAL_W_PACKED it is a
 *          heal_pack_w buffer for the same (N, K), 256-byte aligned.
 *   C      device fp32 [M, N], ldc >= N.  C must not overlap A or W.
 *   flags  one of HEAL_W_NK / HEAL_W_KN, optionally | HEAL_W_F16 and/or
 *          | HEAL_W_PACKED (both: W is a buffer that heal_pack_w packed with
 *          HEAL_W_F16, whose lo planes are zero, and the A_hi.B_lo product
 *          is skipped; a buffer packed from fp32 values must not carry
 *          HEAL_W_F16, or its lo planes are ignored), and/or | HEAL_A_PACKED,
 *          and/or | HEAL_ONE_PRODUCT, or | HEAL_BF16X3 (see above)
 *          (A then is heal_pack_w(A, lda, M, K, HEAL_W_NK)'s buffer: an
 *          activation split once can feed several GEMMs)
 *   a_kshift  device int8 [K], nullable.  Per-channel power-of-two
 *          rescaling of massive activations ([GEMM], the paragraph on FP16
 *          overflow: values beyond FP16's range sit in a small fixed set of
 *          channels, and rescaling those channels, e.g. on the weight side,
 *          removes the overflow at no cost).  Element (m, k) of A is
 *          multiplied by 2^-a_kshift[k] before its split, exactly; the caller
 *          holds W with reduction index k multiplied by 2^+a_kshift[k]
 *          (prepared once: heal_scale_k, or heal_pack_w with the negated
 *          shifts), so C = A.B is unchanged.  Shifts come from
 *          heal_kshift_from_absmax.  Not with HEAL_A_PACKED (UNSUPPORTED): a
 *          packed activation takes its shifts in heal_pack_w.
 *   workspace  device, >= heal_gemm_f32c_workspace(M, N, K, flags) bytes,
 *          256-byte aligned (NULL allowed when that size is 0)
 *   dev_status  device, nullable.  HEAL_FLAG_F16_RANGE is set on the M <= 64
 *          path when an fp32 W (streamed and split as it is, not
 *          normalized) holds an element with |w| >= 65520: pack such a
 *          weight (heal_pack_w normalizes its rows).  The normalized
 *          operands never set it.
 * Layout note: in the M <= 64 case W streams from HBM row by row; rows whose
 * byte stride is a multiple of 16 KB (K = 4096 fp32, ldw = K) start in the
 * same memory channels.  The kernel visits k in a rotated order per group
 * of rows where that helps, and a packed W pads its rows, which is faster
 * still (K = 4096, N = 14336 at M = 1: 52.0 us streamed, 47.7 us packed).
 * Graph capture: on the M <= 64 path with a k split (chosen from N and K)
 * completed through memory, the call marks its split-K flags in the
 * workspace with a per-call value taken on the host, which a captured graph
 * would replay; under stream capture such a call returns
 * HEAL_ERR_UNSUPPORTED before any launch.  heal_gemm_f32c_noalloc captures
 * and replays correctly.  Other shapes capture normally, among them the
 * k splits whose chunks meet in LDS (M <= 16, N >= 4081, no a_kshift, and
 * 2 to 8 chunks of at most 512 k, e.g. K = N = 4096).
 * Limits: M, N, K < 2^31.  K == 0 writes zeros.  In the M <= 64 case above,
 * ldw < 2^26 and lda < 2^24 (each 16-row slice of W, and A, are addressed
 * with 32-bit byte offsets), else HEAL_ERR_UNSUPPORTED.  The launches'
 * thread counts must fit 32 bits: ceil(M/256) ceil(N/256) 512 and
 * ceil(N/64) 256 + 2^18 below 2^32 (M N below about 2^39, N below about
 * 2^30), else HEAL_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------ */
heal_status heal_gemm_f32c(const float* A, int64_t lda, const void* W, int64_t ldw,
                           float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                           uint32_t flags, const int8_t* a_kshift, void* workspace,
                           size_t workspace_bytes, uint32_t* dev_status, void* stream);

/* Workspace bytes heal_gemm_f32c needs for this shape and flags. */
size_t heal_gemm_f32c_workspace(int64_t M, int64_t N, int64_t K, uint32_t flags);

/* ------------------------------------------------------------------------
 * heal_gemm_f32c_noalloc -- heal_gemm_f32c without a workspace argument, for
 * callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.
 *  Same arguments, results and kernels as heal_gemm_f32c (bit for bit), on
 *  the decode path only: M <= 64, W fp32 or binary16 (HEAL_W_F16) in the
 *  [N, K] layout or packed by heal_pack_w (HEAL_W_PACKED), A not packed,
 *  not HEAL_BF16X3, K < 2^23, N <= 2^19 (else HEAL_ERR_UNSUPPORTED).  Its
 *  scratch memory is a 16 MiB array of device memory that the library owns,
 *  one per GPU, held until the process ends: 64 KiB of split-K counters,
 *  then the workspace; shapes whose heal_gemm_f32c_workspace exceeds
 *  16 MiB - 64 KiB get HEAL_ERR_WORKSPACE (the Llama-3-8B-like decode
 *  layers need at most 12.1 MB at M = 64).  No call allocates or frees
 *  memory.  The counters start at zero and every call leaves them zero, so
 *  the call can be captured into a HIP graph and replayed (it records
 *  kernel launches only); nothing in the array needs clearing.  Calls that
 *  overlap on one GPU (other streams or threads, or replays on several
 *  streams) share the array and race: serialize them.
 * ------------------------------------------------------------------------ */
heal_status heal_gemm_f32c_noalloc(const float* A, int64_t lda, const void* W, int64_t ldw,
                                   float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                   uint32_t flags, const int8_t* a_kshift, uint32_t* dev_status,
                                   void* stream);

/* ------------------------------------------------------------------------
 * heal_pack_w -- split an operand once into the GEMM's packed dual-FP16 form.
 *  [GEMM]  Weights are fixed across calls, so their split can be done once
 *  and reused (HEAL_W_PACKED); an activation read by several GEMMs can be
 *  split once as well (HEAL_A_PACKED, with N := M rows of A and HEAL_W_NK).
 *  The packed form is internal and opaque: each fp32 row r is multiplied by
 *  the power of two 2^e[r] that puts its largest magnitude in [2^14, 2^15)
 *  (e[r] = 0 for a zero row), then holds, for every 32-wide block of k, the
 *  32 fp16 hi parts then the 32 fp16 residuals fp16(x' - hi), each at its
 *  own scale (the residual equals heal_split_f32's lo / 2^10 wherever that
 *  is a normal fp16).  With HEAL_W_F16 a row holds its binary16 values
 *  alone, not normalized (e = 0), half the bytes; with HEAL_BF16X3, the 32
 *  bf16 b0, then the 32 b1, then the 32 b2 of the three-way split, not
 *  normalized.  Rows are padded to a multiple of 256 and k to a multiple of
 *  32 with zeros; in the fp16 forms each row is followed by 256 unused bytes
 *  (so rows are never a power-of-two number of bytes apart), and the int32
 *  exponents of the padded rows follow the rows.  An activation is packed
 *  without HEAL_W_F16 (with HEAL_BF16X3 when the GEMM uses that mode).
 *  HEAL_BF16X3 takes fp32 input and no kshift.
 *   W      as in heal_gemm_f32c (flags HEAL_W_NK or HEAL_W_KN, optionally
 *          | HEAL_W_F16: binary16 input, its lo parts are zero), 4-byte
 *          aligned (2-byte with HEAL_W_F16).  Normalized rows cannot
 *          overflow fp16; dev_status is set only by HEAL_BF16X3 (a value
 *          beyond bf16's largest).
 *   kshift device int8 [K], nullable: element (r, k) is multiplied by
 *          2^-kshift[k] before its split (exact; an activation takes the
 *          shifts of heal_gemm_f32c's a_kshift, a weight their negation)
 *   packed device, >= heal_pack_w_bytes(N, K, flags) bytes, 256-byte aligned
 * ------------------------------------------------------------------------ */
heal_status heal_pack_w(const void* W, int64_t ldw, int64_t N, int64_t K, uint32_t flags,
                        const int8_t* kshift, void* packed, size_t packed_bytes,
                        uint32_t* dev_status, void* stream);

/* Bytes of heal_pack_w's buffer for these flags: per padded row, 4 bytes per
 * element of the padded K (hi and residual), or 2 with HEAL_W_F16 (the hi
 * parts alone: a 16-bit weight's residuals are zero and are not stored), plus
 * 256, plus 4 for the row's exponent; or 6 per element with HEAL_BF16X3. */
size_t heal_pack_w_bytes(int64_t N, int64_t K, uint32_t flags);

/* ------------------------------------------------------------------------
 * heal_scale_k -- per-channel power-of-two rescaling of an operand.  [GEMM]
 *  out = X with element (r, k) multiplied by 2^-kshift[k]: the weight-side
 *  half of heal_gemm_f32c's a_kshift (pass the negated shifts to scale a
 *  weight up).  Exact while results stay in the format's normal range.
 *   X, out device, rows x K in the layout of flags (HEAL_W_NK: [rows, K];
 *          HEAL_W_KN: [K, rows]), fp32, or binary16 with HEAL_W_F16; 4-byte
 *          (2-byte) aligned; ldx and ldo >= the row length.  out may be X
 *          (same ld) for an in-place update.
 *   kshift device int8 [K]
 * ------------------------------------------------------------------------ */
heal_status heal_scale_k(const void* X, int64_t ldx, int64_t rows, int64_t K, uint32_t flags,
                         const int8_t* kshift, void* out, int64_t ldo, void* stream);

/* ------------------------------------------------------------------------
 * heal_kshift_from_absmax -- channel shifts from calibration maxima.  [GEMM]
 *  Host call on host arrays: kshift[k] = the smallest s >= 0 with
 *  absmax[k] * 2^-s < limit (exact), so channels inside the limit keep
 *  s = 0 and only outlier channels are rescaled.  With limit <= 32768 the
 *  scaled activations split with a finite fp16 high part.
 *   absmax host fp32 [K]: max |A[:, k]| over calibration data (finite, >= 0)
 *   limit  in [1, 65504]
 *   kshift host int8 [K], written only when the call succeeds
 * Errors: UNSUPPORTED for a limit out of range, an absmax that is negative,
 * NaN or inf, or a shift above 127.
 * ------------------------------------------------------------------------ */
heal_status heal_kshift_from_absmax(const float* absmax, int64_t K, float limit, int8_t* kshift);

/* ------------------------------------------------------------------------
 * heal_qkv_quant_i16 -- INT16 symmetric absmax quantization.   [INT16]
 *
 * Q_INT16(X) = Round((2^15 - 1) X / max|X|), applied per row of D values
 * (one row = one token of one head).  Per row:
 *   M = max_d |x_d|
 *   M == 0 :  s = 0, every code 0
 *   else   :  s = fl(M / 32767),  q_d = rne( fl( fl(32767 * x_d) / M ) )
 * using correctly rounded fp32 multiply and divide, then rounding half to
 * even.  Codes lie in [-32767, 32767].  Domain: finite x with
 * |x| <= 1.0e34 (above FLT_MAX / 32767 the product 32767 * x overflows; such
 * rows are outside the contract like NaN and Inf).  The results are bit-exact: the same
 * on every run and equal to the scalar CPU definition above.
 *   X      device fp32 [rows, D] with ldx >= D.  16-byte aligned, ldx % 4 == 0.
 *   codes  device int16 [rows, D] with ldq >= D.  8-byte aligned, ldq % 4 == 0.
 *   scales device fp32 [rows], 4-byte aligned
 * Limits: D % 4 == 0, 4 <= D <= 4096 (when rows > 0).
 * ------------------------------------------------------------------------ */
heal_status heal_qkv_quant_i16(const float* X, int64_t rows, int64_t D, int64_t ldx,
                               int16_t* codes, int64_t ldq, float* scales, void* stream);

/* ------------------------------------------------------------------------
 * heal_qkv_proj_quant_i16 -- Q/K/V projection with INT16 output.  [GEMM]+[INT16]
 *  The fused Q/K/V linear layer, C = A . W^T with W [(Hq + 2 Hkv) D, K]
 *  (Q heads, then K heads, then V heads, D rows each), computed as
 *  heal_gemm_f32c does, then stored only as INT16 (the pages keep Q, K and
 *  V in INT16; fp32 K/V would double the cache): each (token m, head h) row
 *  of D values is quantized as heal_qkv_quant_i16 does, bit for bit.  Q
 *  rows go to q_codes [M, Hq, D] / q_scales [M, Hq]; K and V rows go to the
 *  cache slot slot_mapping[m] of k_cache / v_cache [num_slots, Hkv, D] and
 *  k_scales / v_scales [num_slots, Hkv] (a paged cache of blocks of B
 *  tokens is this layout with slot = block * B + offset).  A negative slot
 *  writes no K/V row (a padding token); a slot >= num_slots writes none and
 *  sets HEAL_FLAG_SLOT_RANGE in dev_status.  Slots of distinct tokens must
 *  differ, or their rows race.
 *   A, lda, W, ldw, flags, a_kshift  as in heal_gemm_f32c with N = (Hq + 2 Hkv) D
 *          (HEAL_W_KN not supported)
 *   q_codes, k_cache, v_cache  device int16, 8-byte aligned
 *   q_scales, k_scales, v_scales  device fp32, 4-byte aligned
 *   slot_mapping  device int64 [M], 8-byte aligned
 *   workspace  device, >= heal_qkv_proj_quant_workspace(...) bytes, 256-byte
 *          aligned.  With D = 128, fp32 or fp16 weights (not HEAL_ONE_PRODUCT
 *          or HEAL_BF16X3) and a shape the prefill GEMM runs without its k
 *          split (M > 64 with more than 128 output tiles of 256 x 256, or
 *          K <= 224), the GEMM quantizes in its epilogue and the workspace
 *          holds only its packed operands; otherwise it also holds the fp32
 *          product, quantized by a second pass.  The codes are the same.
 * Limits: Hq, Hkv >= 1; D % 4 == 0, 4 <= D <= 4096; (Hq + 2 Hkv) D < 2^31.
 * ------------------------------------------------------------------------ */
heal_status heal_qkv_proj_quant_i16(const float* A, int64_t lda, const void* W, int64_t ldw, int64_t M,
                                    int64_t K, int64_t Hq, int64_t Hkv, int64_t D, uint32_t flags,
                                    const int8_t* a_kshift, int16_t* q_codes, float* q_scales,
                                    const int64_t* slot_mapping, int64_t num_slots, int16_t* k_cache,
                                    float* k_scales, int16_t* v_cache, float* v_scales, void* workspace,
                                    size_t workspace_bytes, uint32_t* dev_status, void* stream);

size_t heal_qkv_proj_quant_workspace(int64_t M, int64_t K, int64_t Hq, int64_t Hkv, int64_t D,
                                     uint32_t flags);

/* ------------------------------------------------------------------------
 * heal_kv_dequant_i16 -- INT16 dequantization.   [INT16]
 *   fmt HEAL_DQ_F32:   out fp32 [rows, D], x^ = fl(q * s)  (out_lo unused)
 *   fmt HEAL_DQ_F16X2: out / out_lo fp16 [rows, D] planes with
 *          hi = fp16(q), lo = fp16((q - hi) * 2^10).  Both are exact for
 *          every int16 code, so q = hi + lo / 2^10 holds exactly (the
 *          pages' dual-FP16 unpack).  The scale is applied by the consumer.
 *   codes  device int16 [rows, D], ldq >= D, 8-byte aligned, ldq % 4 == 0
 *   scales device fp32 [rows] (may be NULL for HEAL_DQ_F16X2)
 *   out    device, ldo >= D, 16-byte aligned (F32) / 8-byte (F16X2), ldo % 4 == 0
 * Limits: D % 4 == 0, 4 <= D <= 4096 (when rows > 0).  Bit-exact.
 * ------------------------------------------------------------------------ */
heal_status heal_kv_dequant_i16(const int16_t* codes, int64_t rows, int64_t D, int64_t ldq,
                                const float* scales, int fmt, void* out, void* out_lo,
                                int64_t ldo, void* stream);

/* ------------------------------------------------------------------------
 * heal_attn_decode_i16 -- one decode step of grouped-query attention over
 * INT16 Q/K/V, with the INT16 -> dual-FP16 unpack fused into the operand
 * load.   [INT16]
 *
 *   o[b,h,:] = softmax_t( q~[b,h] . k~[b,t,g] / sqrt(D) ) . v~[b,t,g,:]
 *   x~ = code * scale,  g = h / (Hq / Hkv)
 *
 * q.k uses an exact split of each code into two fp16 parts (64 (q >> 6)
 * and q & 63) and all four 16-bit products.  The scales are applied in fp32.
 * Softmax is fp32 with a running maximum.  For P.V, the scale of token t is
 * folded into its fp32 weight, which is split into fp16 hi/lo against V's
 * exact parts.
 *   q  [B, Hq, D] int16, q_scale [B, Hq] fp32
 *   k, v  [B, T, Hkv, D] int16 (the KV cache), k_scale, v_scale [B, T, Hkv]
 *   out   [B, Hq, D] fp32
 *   workspace  device, >= heal_attn_decode_workspace(B, T, Hq, Hkv, D)
 *   bytes, 256-byte aligned.  All tensors dense, 16-byte aligned.
 * Limits: D == 128, Hq % Hkv == 0, Hq / Hkv <= 8, 1 <= T <= 262144 and
 * T * Hkv * D * 2 < 2^32 (one batch's K or V block is addressed with 32-bit
 * byte offsets) when B*Hq > 0; the launches' thread counts
 * B * Hkv * ceil(T / 256) * 256 and B * Hq * 512 below 2^32; otherwise
 * HEAL_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------ */
heal_status heal_attn_decode_i16(const int16_t* q, const float* q_scale,
                                 const int16_t* k, const float* k_scale,
                                 const int16_t* v, const float* v_scale,
                                 float* out, int64_t B, int64_t T, int64_t Hq, int64_t Hkv,
                                 int64_t D, void* workspace, size_t workspace_bytes,
                                 void* stream);

size_t heal_attn_decode_workspace(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D);

/* ------------------------------------------------------------------------
 * heal_attn_prefill_i16 -- causal self-attention of a prompt over INT16
 * Q/K/V with the dual-FP16 expansion.   [INT16]
 *  For every batch b, query token t and head h (KV head h / (Hq / Hkv)):
 *    o[b,t,h] = sum_{s <= t} softmax_s(s_q s_k (q . k_s) / sqrt(D)) s_v v_s
 *  with q, k_s, v_s the INT16 codes and s_* their row scales; codes enter the
 *  MFMA products as their exact fp16 parts (64 (c >> 6) and c & 63) with fp32
 *  accumulation, the softmax weights split into fp16 hi + lo, as in
 *  heal_attn_decode_i16.  Error bar as there.
 *   q      device int16 [B, T, Hq, D], 16-byte aligned; q_scale fp32 [B, T, Hq]
 *   k, v   device int16 [B, T, Hkv, D] (the decode cache layout), 16-byte
 *          aligned; k_scale, v_scale fp32 [B, T, Hkv]
 *   out    device fp32 [B, T, Hq, D], 4-byte aligned
 * Limits: D = 128; Hq % Hkv == 0; T <= 262144; T Hkv D 2 < 2^32; the
 * launch's thread count B Hq ceil(T / 128) 512 below 2^32 (else
 * HEAL_ERR_UNSUPPORTED).  No workspace.
 * ------------------------------------------------------------------------ */
heal_status heal_attn_prefill_i16(const int16_t* q, const float* q_scale, const int16_t* k,
                                  const float* k_scale, const int16_t* v, const float* v_scale, float* out,
                                  int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, void* stream);

/* ------------------------------------------------------------------------
 * Roofline calibration (measurement only; not part of the method).  The
 * denominators of the library's roofline figures, measured on the device.
 *
 * heal_calib_mfma_f16 -- `workgroups` workgroups of 4 waves (one per compute
 *  unit as the prefill GEMM runs), each wave issuing `iters` rounds of 16
 *  independent v_mfma_f32_32x32x16_f16 on registers (no LDS, no memory):
 *  workgroups * 4 * iters * 16 * 32768 flops.  out: device fp32
 *  [workgroups * 256], 4-byte aligned (a checksum that keeps the work).
 * heal_calib_read -- a streaming read of `bytes` bytes at buf (16-byte
 *  aligned, bytes % 16 == 0) by `workgroups` workgroups of 256 threads.
 *  out: device fp32 [workgroups * 256], 4-byte aligned.
 * Limits: workgroups <= 2^20.
 * ------------------------------------------------------------------------ */
heal_status heal_calib_mfma_f16(int64_t iters, int64_t workgroups, float* out, void* stream);
heal_status heal_calib_read(const void* buf, int64_t bytes, int64_t workgroups, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HEAL_H */
