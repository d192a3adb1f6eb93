// C ABI of libheal: argument validation (host only, before any HIP call),
// workspace layout and kernel selection.  Entry points and their contracts
// are documented in include/heal.h.
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>

#include "heal_internal.h"

using namespace heal;

namespace heal {
// Path choice for heal_gemm_f32c.  The decode kernel streams an fp32 [N,K]
// weight directly; every other case packs the operands for the prefill kernel.
// The decode kernel addresses its split activation (256 bytes per k) and
// each 16-row slice of W with 32-bit byte offsets.
bool decode_path(int64_t M, int64_t K, uint32_t flags) {
    // a packed weight has no layout flag: its rows are [N, K]
    return M <= 64 && K < ((int64_t)1 << 23) && !(flags & (HEAL_A_PACKED | HEAL_BF16X3)) &&
           ((flags & HEAL_W_PACKED) || (flags & HEAL_W_KN) == 0);
}

// Call epochs for the decode GEMM's split-K flags: unique within the
// process; the start is taken from the clock so that a workspace that held
// another process's counters is not mistaken for this one's.
uint64_t next_epoch() {
    static std::atomic<uint64_t> next{
        ((uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() & 0xFFFFFFFFull) << 12 | 1u};
    for (;;) {
        const uint64_t e = next.fetch_add(1, std::memory_order_relaxed) & 0xFFFFFFFFFFFFull;
        if (e != 0) return e;
    }
}
}  // namespace heal

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;
// a launch's thread count must fit the dispatch packet's 32-bit grid size
bool fits_u32(__int128 threads) { return threads < ((__int128)1 << 32); }

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }
int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }
heal_status hip_status(hipError_t e) { return e == hipSuccess ? HEAL_OK : HEAL_ERR_HIP; }

bool use_decode(int64_t M, int64_t K, uint32_t flags) { return decode_path(M, K, flags); }
// bytes of one packed operand in the form the flags select
int64_t packed_bytes(int64_t R, int64_t K, uint32_t flags) {
    if (flags & HEAL_BF16X3) return pack_bytes_x3(R, K);
    return (flags & HEAL_W_F16) ? pack_bytes_hi(R, K) : pack_bytes(R, K);
}
// The Q/K/V projection quantizes in the prefill GEMM's epilogue for heads of
// 128 outputs, the 3- and 2-product forms, and shapes the prefill kernel runs
// without its k split; other cases store the fp32 product and quantize it in
// a second pass (identical codes either way).
bool qkv_fused(int64_t M, int64_t N, int64_t K, int64_t D, uint32_t flags) {
    return D == 128 && K > 0 && !use_decode(M, K, flags) && !(flags & (HEAL_ONE_PRODUCT | HEAL_BF16X3)) &&
           !prefill_ksplit(M, N, K);
}
constexpr int64_t kMaxDecodeLdw = (int64_t)1 << 26;
constexpr int64_t kMaxDecodeLda = (int64_t)1 << 24;   // A (<= 64 rows) addressed with 32-bit byte offsets

__global__ void zero_rows_kernel(float* C, int64_t ldc, int64_t M, int64_t N) {
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / N;
        C[m * ldc + (i - m * N)] = 0.0f;
    }
}

}  // namespace

extern "C" {

const char* heal_status_str(heal_status s) {
    switch (s) {
        case HEAL_OK: return "HEAL_OK";
        case HEAL_ERR_NULL: return "HEAL_ERR_NULL: a required pointer is NULL";
        case HEAL_ERR_SHAPE: return "HEAL_ERR_SHAPE: a dimension is negative or out of range";
        case HEAL_ERR_STRIDE: return "HEAL_ERR_STRIDE: a leading dimension is smaller than its row";
        case HEAL_ERR_ALIGN: return "HEAL_ERR_ALIGN: a pointer or leading dimension is misaligned";
        case HEAL_ERR_UNSUPPORTED: return "HEAL_ERR_UNSUPPORTED: unsupported flags or sizes";
        case HEAL_ERR_WORKSPACE: return "HEAL_ERR_WORKSPACE: workspace missing or too small";
        case HEAL_ERR_HIP: return "HEAL_ERR_HIP: a HIP kernel launch failed";
    }
    return "HEAL: unknown status";
}

int heal_version(void) { return (1 << 16) | (3 << 8); }

heal_status heal_split_f32(const float* X, int64_t n, uint16_t* hi, uint16_t* lo,
                           uint32_t* dev_status, void* stream) {
    if (n < 0) return HEAL_ERR_SHAPE;
    if (n == 0) return HEAL_OK;
    if (!X || !hi || !lo) return HEAL_ERR_NULL;
    if (misaligned(X, 16) || misaligned(hi, 8) || misaligned(lo, 8) || misaligned(dev_status, 4))
        return HEAL_ERR_ALIGN;
    return hip_status(launch_split(X, n, hi, lo, dev_status, static_cast<hipStream_t>(stream)));
}

size_t heal_pack_w_bytes(int64_t N, int64_t K, uint32_t flags) {
    if (N <= 0 || K <= 0 || N >= kMaxDim || K >= kMaxDim) return 0;
    return (size_t)packed_bytes(N, K, flags);
}

heal_status heal_pack_w(const void* W, int64_t ldw, int64_t N, int64_t K, uint32_t flags,
                        const int8_t* kshift, void* packed, size_t packed_bytes, uint32_t* dev_status,
                        void* stream) {
    if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim) return HEAL_ERR_SHAPE;
    if (flags & ~(uint32_t)(HEAL_W_KN | HEAL_W_F16 | HEAL_BF16X3)) return HEAL_ERR_UNSUPPORTED;
    const bool x3 = flags & HEAL_BF16X3;
    if (x3 && ((flags & HEAL_W_F16) || kshift)) return HEAL_ERR_UNSUPPORTED;   // fp32 input, no shifts
    if (N == 0 || K == 0) return HEAL_OK;
    if (!W || !packed) return HEAL_ERR_NULL;
    const bool kn = flags & HEAL_W_KN;
    const bool f16 = flags & HEAL_W_F16;
    if (ldw < (kn ? N : K)) return HEAL_ERR_STRIDE;
    if (misaligned(W, f16 ? 2 : 4) || misaligned(packed, 256) || misaligned(dev_status, 4)) return HEAL_ERR_ALIGN;
    if (packed_bytes < heal_pack_w_bytes(N, K, flags)) return HEAL_ERR_WORKSPACE;
    if (x3)
        return hip_status(launch_pack_bf16x3(static_cast<const float*>(W), ldw, N, K, kn ? 1 : 0, packed, dev_status,
                                             static_cast<hipStream_t>(stream)));
    return hip_status(launch_pack(W, f16, ldw, N, K, kn ? 1 : 0, kshift, packed, dev_status,
                                  static_cast<hipStream_t>(stream)));
}

size_t heal_gemm_f32c_workspace(int64_t M, int64_t N, int64_t K, uint32_t flags) {
    if (M <= 0 || N <= 0 || K <= 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return 0;
    if (use_decode(M, K, flags)) {
        return (size_t)decode_plan(M, N, K).bytes();
    }
    int64_t b = (flags & HEAL_A_PACKED) ? 0 : round256(packed_bytes(M, K, flags & HEAL_BF16X3));
    if (!(flags & HEAL_W_PACKED)) b += round256(packed_bytes(N, K, flags));
    return (size_t)b;
}

}  // extern "C"

namespace {
// heal_gemm_f32c; with qkv set (the fused Q/K/V projection, qkv_fused true)
// the prefill kernel quantizes its output instead of storing C.
heal_status gemm_impl(const float* A, int64_t lda, const void* W, int64_t ldw, float* C, int64_t ldc, int64_t M,
                      int64_t N, int64_t K, uint32_t flags, const int8_t* a_kshift, void* workspace,
                      size_t workspace_bytes, uint32_t* dev_status, void* stream, const QkvDst* qkv,
                      unsigned long long* counters = nullptr) {
    if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return HEAL_ERR_SHAPE;
    if (flags & ~(uint32_t)(HEAL_W_KN | HEAL_W_PACKED | HEAL_A_PACKED | HEAL_W_F16 | HEAL_ONE_PRODUCT | HEAL_BF16X3))
        return HEAL_ERR_UNSUPPORTED;
    if ((flags & HEAL_A_PACKED) && a_kshift) return HEAL_ERR_UNSUPPORTED;   // a packed A carries its shifts
    // the BF16 three-way mode takes fp32 operands and needs no range shifts
    if ((flags & HEAL_BF16X3) && ((flags & (HEAL_W_F16 | HEAL_ONE_PRODUCT)) || a_kshift))
        return HEAL_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return HEAL_OK;
    if (!C && !qkv) return HEAL_ERR_NULL;
    if (!qkv && ldc < N) return HEAL_ERR_STRIDE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) {
        const int64_t blocks = std::min<int64_t>((M * N + 255) / 256, 4096);
        hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, C, ldc, M, N);
        return hip_status(hipGetLastError());
    }
    if (!A || !W) return HEAL_ERR_NULL;
    // launch sizes in threads (32-bit): the prefill grid (256 x 256 tiles,
    // at most two k halves) and the decode grid (one 64-row group per 256
    // threads, about 512 workgroups in all when the rows are few)
    if (!fits_u32((__int128)((M + 255) / 256) * ((N + 255) / 256) * 2 * 256) ||
        !fits_u32((__int128)((N + 63) / 64) * 256 + 512 * 512))
        return HEAL_ERR_UNSUPPORTED;
    const bool packed = flags & HEAL_W_PACKED;
    const bool a_packed = flags & HEAL_A_PACKED;
    const bool kn = flags & HEAL_W_KN;
    const bool wf16 = flags & HEAL_W_F16;
    const bool one = flags & HEAL_ONE_PRODUCT;
    if (!a_packed && lda < K) return HEAL_ERR_STRIDE;
    if (!packed && ldw < (kn ? N : K)) return HEAL_ERR_STRIDE;
    if (misaligned(A, a_packed ? 256 : 4) || misaligned(W, packed ? 256 : (wf16 ? 2 : 4)) || misaligned(C, 4) ||
        misaligned(dev_status, 4))
        return HEAL_ERR_ALIGN;
    const size_t need = heal_gemm_f32c_workspace(M, N, K, flags);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return HEAL_ERR_WORKSPACE;
        if (misaligned(workspace, 256)) return HEAL_ERR_ALIGN;
    }

    if (use_decode(M, K, flags)) {
        if ((!packed && ldw >= kMaxDecodeLdw) || lda >= kMaxDecodeLda) return HEAL_ERR_UNSUPPORTED;
        const DecodePlan p = decode_plan(M, N, K);
        // the epoch of a captured call would be replayed with the graph, and
        // a replay would take the previous one's flags for its own (chunks
        // that meet in LDS use no flags)
        if (p.splits > 1 && !counters && !decode_chunks_as_waves(M, N, p, a_kshift != nullptr)) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing(s, &cs) != hipSuccess) return HEAL_ERR_HIP;
            if (cs != hipStreamCaptureStatusNone) return HEAL_ERR_UNSUPPORTED;
        }
        unsigned char* ws = static_cast<unsigned char*>(workspace);
        return hip_status(launch_gemm_decode(A, lda, a_kshift, W, wf16, packed, one, ldw, C, ldc, M, N, K, ws, p,
                                             next_epoch(), counters, dev_status, s));
    }
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    const void* apk = A;
    const void* bpk = W;
    if (flags & HEAL_BF16X3) {
        if (!a_packed) {
            if (launch_pack_bf16x3(A, lda, M, K, 0, ws, dev_status, s) != hipSuccess) return HEAL_ERR_HIP;
            apk = ws;
            ws += round256(pack_bytes_x3(M, K));
        }
        if (!packed) {
            if (launch_pack_bf16x3(static_cast<const float*>(W), ldw, N, K, kn ? 1 : 0, ws, dev_status, s) !=
                hipSuccess)
                return HEAL_ERR_HIP;
            bpk = ws;
        }
        return hip_status(launch_gemm_prefill(apk, bpk, 6, true, C, ldc, M, N, K, s, qkv));
    }
    // one product: an activation packed here keeps its hi parts alone (half the
    // GEMM's A staging); the workspace keeps the size of the hi/lo form
    const bool a_hi = one && !a_packed && !a_kshift && !misaligned(A, 16) && (lda & 3) == 0;
    if (!a_packed) {
        hipError_t e = a_hi ? launch_pack_hi_f32(A, lda, M, K, ws, dev_status, s)
                            : launch_pack(A, false, lda, M, K, 0, a_kshift, ws, dev_status, s);
        if (e != hipSuccess) return HEAL_ERR_HIP;
        apk = ws;
        ws += round256(pack_bytes(M, K));
    }
    if (!packed) {
        void* wpk = ws;
        hipError_t e;
        e = launch_pack(W, wf16, ldw, N, K, kn ? 1 : 0, nullptr, wpk, dev_status, s);
        if (e != hipSuccess) return HEAL_ERR_HIP;
        bpk = wpk;
    }
    return hip_status(launch_gemm_prefill(apk, bpk, one ? 1 : (wf16 ? 2 : 3), wf16, C, ldc, M, N, K, s, qkv, a_hi));
}
}  // namespace

heal_status heal::gemm_f32c_counters(const float* A, int64_t lda, const void* W, int64_t ldw, float* C,
                                     int64_t ldc, int64_t M, int64_t N, int64_t K, uint32_t flags,
                                     const int8_t* a_kshift, void* workspace, size_t workspace_bytes,
                                     unsigned long long* counters, uint32_t* dev_status, void* stream) {
    return gemm_impl(A, lda, W, ldw, C, ldc, M, N, K, flags, a_kshift, workspace, workspace_bytes, dev_status,
                     stream, nullptr, counters);
}

extern "C" {

heal_status heal_gemm_f32c(const float* A, int64_t lda, const void* W, int64_t ldw, float* C,
                           int64_t ldc, int64_t M, int64_t N, int64_t K, uint32_t flags, const int8_t* a_kshift,
                           void* workspace, size_t workspace_bytes, uint32_t* dev_status,
                           void* stream) {
    return gemm_impl(A, lda, W, ldw, C, ldc, M, N, K, flags, a_kshift, workspace, workspace_bytes, dev_status,
                     stream, nullptr);
}

heal_status heal_scale_k(const void* X, int64_t ldx, int64_t rows, int64_t K, uint32_t flags,
                         const int8_t* kshift, void* out, int64_t ldo, void* stream) {
    if (rows < 0 || K < 0 || rows >= kMaxDim || K >= kMaxDim) return HEAL_ERR_SHAPE;
    if (flags & ~(uint32_t)(HEAL_W_KN | HEAL_W_F16)) return HEAL_ERR_UNSUPPORTED;
    if (rows == 0 || K == 0) return HEAL_OK;
    if (!X || !kshift || !out) return HEAL_ERR_NULL;
    const bool kn = flags & HEAL_W_KN;
    const bool f16 = flags & HEAL_W_F16;
    const int64_t row_len = kn ? rows : K;
    if (ldx < row_len || ldo < row_len) return HEAL_ERR_STRIDE;
    if (misaligned(X, f16 ? 2 : 4) || misaligned(out, f16 ? 2 : 4)) return HEAL_ERR_ALIGN;
    return hip_status(launch_scale_k(X, f16, ldx, rows, K, kn ? 1 : 0, kshift, out, ldo,
                                     static_cast<hipStream_t>(stream)));
}

heal_status heal_kshift_from_absmax(const float* absmax, int64_t K, float limit, int8_t* kshift) {
    if (K < 0 || K >= kMaxDim) return HEAL_ERR_SHAPE;
    if (K == 0) return HEAL_OK;
    if (!absmax || !kshift) return HEAL_ERR_NULL;
    if (!(limit >= 1.0f && limit <= 65504.0f)) return HEAL_ERR_UNSUPPORTED;
    // smallest s >= 0 with absmax * 2^-s < limit: scaling by a power of two is
    // exact in double, so each comparison is exact.  Validate all first, so a
    // rejected call writes nothing.
    auto shift_of = [limit](double a) {
        int sh = 0;
        while (sh <= 127 && std::ldexp(a, -sh) >= (double)limit) ++sh;
        return sh;
    };
    for (int64_t k = 0; k < K; ++k) {
        const double a = absmax[k];
        if (!(a >= 0.0 && a <= 3.4028234663852886e38)) return HEAL_ERR_UNSUPPORTED;   // negative, NaN, inf
        if (shift_of(a) > 127) return HEAL_ERR_UNSUPPORTED;
    }
    for (int64_t k = 0; k < K; ++k) kshift[k] = (int8_t)shift_of(absmax[k]);
    return HEAL_OK;
}

heal_status heal_qkv_quant_i16(const float* X, int64_t rows, int64_t D, int64_t ldx, int16_t* codes,
                               int64_t ldq, float* scales, void* stream) {
    if (rows < 0 || D < 0) return HEAL_ERR_SHAPE;
    if (rows == 0) return HEAL_OK;
    if (D < 4 || D > 4096 || (D & 3)) return HEAL_ERR_SHAPE;
    if (!X || !codes || !scales) return HEAL_ERR_NULL;
    if (ldx < D || ldq < D) return HEAL_ERR_STRIDE;
    if (misaligned(X, 16) || (ldx & 3) || misaligned(codes, 8) || (ldq & 3) || misaligned(scales, 4))
        return HEAL_ERR_ALIGN;
    return hip_status(launch_quant(X, rows, D, ldx, codes, ldq, scales, static_cast<hipStream_t>(stream)));
}

size_t heal_qkv_proj_quant_workspace(int64_t M, int64_t K, int64_t Hq, int64_t Hkv, int64_t D,
                                     uint32_t flags) {
    if (M <= 0 || K < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || M >= kMaxDim || K >= kMaxDim) return 0;
    const int64_t N = (Hq + 2 * Hkv) * D;
    if (N >= kMaxDim) return 0;
    const size_t gemm = heal_gemm_f32c_workspace(M, N, K, flags);   // 0 when K == 0
    // unless the GEMM quantizes in its epilogue, the fp32 product is staged
    // here (K == 0 included: a zero product, quantized to zero codes)
    return qkv_fused(M, N, K, D, flags) ? gemm : (size_t)round256(M * N * 4) + gemm;
}

heal_status heal_qkv_proj_quant_i16(const float* A, int64_t lda, const void* W, int64_t ldw, int64_t M,
                                    int64_t K, int64_t Hq, int64_t Hkv, int64_t D, uint32_t flags,
                                    const int8_t* a_kshift, int16_t* q_codes, float* q_scales,
                                    const int64_t* slot_mapping, int64_t num_slots, int16_t* k_cache,
                                    float* k_scales, int16_t* v_cache, float* v_scales, void* workspace,
                                    size_t workspace_bytes, uint32_t* dev_status, void* stream) {
    if (M < 0 || K < 0 || Hq < 1 || Hkv < 1 || num_slots < 0 || M >= kMaxDim || K >= kMaxDim)
        return HEAL_ERR_SHAPE;
    if (D < 4 || D > 4096 || (D & 3) || (Hq + 2 * Hkv) * D >= kMaxDim) return HEAL_ERR_SHAPE;
    if (flags & HEAL_W_KN) return HEAL_ERR_UNSUPPORTED;
    if (M == 0) return HEAL_OK;
    if (!q_codes || !q_scales || !slot_mapping || !k_cache || !k_scales || !v_cache || !v_scales)
        return HEAL_ERR_NULL;
    if (misaligned(q_codes, 8) || misaligned(k_cache, 8) || misaligned(v_cache, 8) || misaligned(q_scales, 4) ||
        misaligned(k_scales, 4) || misaligned(v_scales, 4) || misaligned(slot_mapping, 8) ||
        misaligned(dev_status, 4))
        return HEAL_ERR_ALIGN;
    const int64_t N = (Hq + 2 * Hkv) * D;
    const size_t need = heal_qkv_proj_quant_workspace(M, K, Hq, Hkv, D, flags);
    if (need > 0 && (!workspace || workspace_bytes < need)) return HEAL_ERR_WORKSPACE;
    if (misaligned(workspace, 256)) return HEAL_ERR_ALIGN;
    if (qkv_fused(M, N, K, D, flags)) {   // the INT16 epilogue of the GEMM itself
        const QkvDst dst{q_codes, q_scales, k_cache, k_scales, v_cache, v_scales, slot_mapping, num_slots,
                         (int)Hq, (int)Hkv, (int)D, dev_status};
        return gemm_impl(A, lda, W, ldw, nullptr, N, M, N, K, flags, a_kshift, workspace, workspace_bytes, dev_status,
                         stream, &dst);
    }
    // the fp32 product lands in the workspace, the GEMM's own workspace after
    // it (need >= round256(M N 4) was checked above, so the rest is >= 0)
    float* C = static_cast<float*>(workspace);
    const size_t cbytes = (size_t)round256(M * N * 4);
    if (need < cbytes || workspace_bytes < cbytes) return HEAL_ERR_WORKSPACE;
    unsigned char* gws = static_cast<unsigned char*>(workspace) + cbytes;
    const heal_status st = heal_gemm_f32c(A, lda, W, ldw, C, N, M, N, K, flags, a_kshift, gws,
                                          workspace_bytes - cbytes, dev_status, stream);
    if (st != HEAL_OK) return st;
    return hip_status(launch_quant_qkv(C, M, Hq, Hkv, D, q_codes, q_scales, slot_mapping, num_slots, k_cache,
                                       k_scales, v_cache, v_scales, dev_status, static_cast<hipStream_t>(stream)));
}

heal_status heal_kv_dequant_i16(const int16_t* codes, int64_t rows, int64_t D, int64_t ldq,
                                const float* scales, int fmt, void* out, void* out_lo, int64_t ldo,
                                void* stream) {
    if (rows < 0 || D < 0) return HEAL_ERR_SHAPE;
    if (fmt != HEAL_DQ_F32 && fmt != HEAL_DQ_F16X2) return HEAL_ERR_UNSUPPORTED;
    if (rows == 0) return HEAL_OK;
    if (D < 4 || D > 4096 || (D & 3)) return HEAL_ERR_SHAPE;
    if (!codes || !out) return HEAL_ERR_NULL;
    if (fmt == HEAL_DQ_F32 && !scales) return HEAL_ERR_NULL;
    if (fmt == HEAL_DQ_F16X2 && !out_lo) return HEAL_ERR_NULL;
    if (ldq < D || ldo < D) return HEAL_ERR_STRIDE;
    if (misaligned(codes, 8) || (ldq & 3) || (ldo & 3) || misaligned(scales, 4)) return HEAL_ERR_ALIGN;
    if (fmt == HEAL_DQ_F32 ? misaligned(out, 16) : (misaligned(out, 8) || misaligned(out_lo, 8)))
        return HEAL_ERR_ALIGN;
    return hip_status(launch_dequant(codes, rows, D, ldq, scales, fmt, out, out_lo, ldo,
                                     static_cast<hipStream_t>(stream)));
}

size_t heal_attn_decode_workspace(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D) {
    if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return 0;
    if (B >= kMaxDim || T >= kMaxDim || Hq >= kMaxDim || Hkv >= kMaxDim) return 0;   // no valid call
    return (size_t)attn_workspace_bytes(B, T, Hq, Hkv, D);
}

heal_status heal_attn_decode_i16(const int16_t* q, const float* q_scale, const int16_t* k,
                                 const float* k_scale, const int16_t* v, const float* v_scale,
                                 float* out, int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || T < 0 || Hq < 0 || Hkv < 0 || D < 0 || B >= kMaxDim || T >= kMaxDim || Hq >= kMaxDim ||
        Hkv >= kMaxDim)
        return HEAL_ERR_SHAPE;
    if (B == 0 || Hq == 0) return HEAL_OK;
    if (Hkv == 0 || Hq % Hkv) return HEAL_ERR_SHAPE;
    if (T == 0) return HEAL_ERR_SHAPE;
    if (D != 128 || Hq / Hkv > 8 || T > 262144) return HEAL_ERR_UNSUPPORTED;
    if (T * Hkv * D * 2 >= ((int64_t)1 << 32)) return HEAL_ERR_UNSUPPORTED;   // 32-bit offsets per batch
    // launch sizes in threads (32-bit): the range kernel and the merge
    if (!fits_u32((__int128)B * Hkv * ((T + 255) / 256) * 256) || !fits_u32((__int128)B * Hq * 512))
        return HEAL_ERR_UNSUPPORTED;
    if (!q || !q_scale || !k || !k_scale || !v || !v_scale || !out) return HEAL_ERR_NULL;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) ||
        misaligned(q_scale, 4) || misaligned(k_scale, 4) || misaligned(v_scale, 4))
        return HEAL_ERR_ALIGN;
    const size_t need = heal_attn_decode_workspace(B, T, Hq, Hkv, D);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return HEAL_ERR_WORKSPACE;
        if (misaligned(workspace, 256)) return HEAL_ERR_ALIGN;
    }
    return hip_status(launch_attn_decode(q, q_scale, k, k_scale, v, v_scale, out, B, T, Hq, Hkv, D,
                                         workspace, static_cast<hipStream_t>(stream)));
}

heal_status heal_attn_prefill_i16(const int16_t* q, const float* q_scale, const int16_t* k,
                                  const float* k_scale, const int16_t* v, const float* v_scale, float* out,
                                  int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, void* stream) {
    if (B < 0 || T < 0 || Hq < 0 || Hkv < 0 || D < 0 || B >= kMaxDim || T >= kMaxDim || Hq >= kMaxDim ||
        Hkv >= kMaxDim)
        return HEAL_ERR_SHAPE;
    if (B == 0 || T == 0 || Hq == 0) return HEAL_OK;
    if (Hkv == 0 || Hq % Hkv) return HEAL_ERR_SHAPE;
    if (D != 128 || T > 262144 || !fits_u32((__int128)B * Hq * ((T + 127) / 128) * 512))
        return HEAL_ERR_UNSUPPORTED;   // launch size in threads (32-bit)
    if (T * Hkv * D * 2 >= ((int64_t)1 << 32)) return HEAL_ERR_UNSUPPORTED;   // 32-bit offsets per batch
    if (!q || !q_scale || !k || !k_scale || !v || !v_scale || !out) return HEAL_ERR_NULL;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 4) ||
        misaligned(q_scale, 4) || misaligned(k_scale, 4) || misaligned(v_scale, 4))
        return HEAL_ERR_ALIGN;
    return hip_status(launch_attn_prefill(q, q_scale, k, k_scale, v, v_scale, out, B, T, Hq, Hkv, D,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"
