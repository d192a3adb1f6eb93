// Internal declarations shared by the HIP translation units of libheal.
// Device helpers for the dual-FP16 representation and the kernel launchers
// that the C ABI layer (api.hip) calls after validating arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "heal.h"

namespace heal {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
// 16 (8) bytes read once from global memory, with the non-temporal hint.
// Measured per kernel: it speeds up the quantizer's and dequantizer's streams
// (5.45 -> 5.86 and 5.73 -> 5.81 TB/s) but slows the split, the decode GEMM's
// weight stream and decode attention, which keep ordinary loads.
__device__ __forceinline__ float4 load_nt_f4(const float* p) {
    return __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ u32x2v load_nt_8b(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(p));
}

// Buffer resource for raw buffer loads over [base, base + bytes): the address
// is base + voffset (per lane, 32-bit) + soffset (wave-uniform), so a loop of
// loads needs one VGPR per lane and keeps every other offset in scalars.
// Loads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// fp32 -> fp16 with round-to-nearest-even and fp16 subnormals kept (the
// hardware conversion under the default rounding and denormal modes), and the
// dual-FP16 residual lo = fp16((x - hi) * 2^10); x - hi is exact in fp32.
__device__ __forceinline__ void split_one(float x, _Float16& hi, _Float16& lo) {
    hi = (_Float16)x;
    float r = x - (float)hi;
    lo = (_Float16)(r * 1024.0f);
}

__device__ __forceinline__ uint16_t f16_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

// Row normalization (the packed GEMM operands and the decode activation):
// each row is multiplied by 2^e with e = 14 - floor(log2(max |x|)), so its
// largest magnitude lies in [2^14, 2^15), the top binade that cannot round
// past 65504; e = 0 for a zero row.  The product is multiplied back by
// 2^-(e_a + e_b) in fp32.  frexp's exponent p gives max = f 2^p, f in [0.5, 1).
__device__ __forceinline__ int row_norm_exp(float amax) {
    return amax > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(amax) : 0;
}
// Split of a normalized element with its residual at its own scale:
// hi = fp16(x), res = fp16(x - hi) (x - hi exact in fp32).  On a normalized
// row res equals the paper's lo / 2^10 for every element above 2^-17 of the
// row's largest, so the three products accumulate with no scaling.
__device__ __forceinline__ void split_res(float x, _Float16& hi, _Float16& res) {
    hi = (_Float16)x;
    res = (_Float16)(x - (float)hi);
}

// An operand magnitude at or above 65520 rounds to an infinite fp16 high part.
__device__ __forceinline__ bool f16_out_of_range(float x) { return __builtin_fabsf(x) >= 65520.0f; }
__device__ __forceinline__ bool f16_out_of_range4(const float4& v) {
    return fmaxf(fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)),
                 fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w))) >= 65520.0f;
}

// Lane reductions with no LDS-pipe instruction (all lanes active).  DPP
// row_ror:N hands lane i of each 16-lane row the value of lane (i - N) mod 16
// of the same row; v_permlane16_swap of x with itself exchanges rows 0 <-> 1
// and 2 <-> 3, v_permlane32_swap the two halves, so one of the two results
// holds the partner lane's value.  The swap results are copied into scalars
// before they are reinterpreted: this compiler's __builtin_bit_cast of a
// vector element reads element 0.
template <int N>
__device__ __forceinline__ float max_row_ror(float x) {
    return fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + N,
                                                                          0xF, 0xF, false)));
}
__device__ __forceinline__ float max_swap16(float x) {   // with lane ^ 16
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t a0 = a[0], a1 = a[1];
    return fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
}
__device__ __forceinline__ float max_swap32(float x) {   // with lane ^ 32
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t a0 = a[0], a1 = a[1];
    return fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
}
// over the 16 lanes of the wave that share lane % 4
__device__ __forceinline__ float max16_mod4(float x) {
    return max_swap32(max_swap16(max_row_ror<8>(max_row_ror<4>(x))));
}
// over the 32 lanes of each half wave
__device__ __forceinline__ float max_half(float x) {
    return max_swap16(max_row_ror<8>(max_row_ror<4>(max_row_ror<2>(max_row_ror<1>(x)))));
}

// ---- packed dual-FP16 operand layout used by the prefill GEMM --------------
// Row r of a packed operand is normalized (row_norm_exp) and holds, for each
// 32-wide block kb of the reduction dimension, 32 fp16 hi parts followed by
// 32 fp16 residuals (split_res; 128 bytes), rows pack_row_bytes apart.  Rows
// are padded to a multiple of kPackRows and k to a multiple of kPackK, with
// zeros, so the GEMM main loop needs no bounds checks.  After the rows come the row exponents, int32
// [pack_rows(R)] (0 for padding rows).  A 16-bit weight (its residuals are
// zero) packs as the hi parts alone, not normalized: row r holds its Kp fp16
// values (64 bytes per 32-wide block), same padding, exponents 0.  An fp32
// activation packed for the one-product mode keeps its normalized hi parts
// alone in the same form.
constexpr int kPackK = 32;
constexpr int kPackRows = 256;

// Each packed row is followed by 256 unused bytes: rows whose stride is a
// multiple of 16 KB (K = 4096) would otherwise start in the same memory
// channel, and a kernel reading 16 rows at one k would queue on it.
constexpr int kPackRowPad = 256;

__host__ __device__ inline int64_t pack_kp(int64_t K) { return (K + kPackK - 1) / kPackK * kPackK; }
__host__ __device__ inline int64_t pack_rows(int64_t R) { return (R + kPackRows - 1) / kPackRows * kPackRows; }
// byte stride of the rows of a packed operand: hi/res form, hi-only form
__host__ __device__ inline int64_t pack_row_bytes(int64_t K) { return pack_kp(K) * 4 + kPackRowPad; }
__host__ __device__ inline int64_t pack_row_bytes_hi(int64_t K) { return pack_kp(K) * 2 + kPackRowPad; }
// bytes of the rows of a packed operand (hi/res form), where its exponents start
__host__ __device__ inline int64_t pack_data_bytes(int64_t R, int64_t K) { return pack_rows(R) * pack_row_bytes(K); }
__host__ __device__ inline int64_t pack_data_bytes_hi(int64_t R, int64_t K) { return pack_rows(R) * pack_row_bytes_hi(K); }
// bytes of one packed operand of R rows and reduction length K: rows, then exponents
__host__ __device__ inline int64_t pack_bytes(int64_t R, int64_t K) { return pack_data_bytes(R, K) + pack_rows(R) * 4; }
// bytes of the hi-only packed form
__host__ __device__ inline int64_t pack_bytes_hi(int64_t R, int64_t K) { return pack_data_bytes_hi(R, K) + pack_rows(R) * 4; }

// bytes of the BF16 three-way packed form: per row and 32-wide k block, the
// 32 bf16 b0, then the 32 b1, then the 32 b2 (192 bytes), same padding; not
// normalized (bf16 has fp32's exponent range) and no exponents
__host__ __device__ inline int64_t pack_bytes_x3(int64_t R, int64_t K) { return pack_rows(R) * pack_kp(K) * 6; }

// Rows of a fused Q/K/V projection output [M, (Hq + 2 Hkv) D]: row r is
// (token m, head h).  Q heads go to q_codes [M, Hq, D] and q_scales [M, Hq];
// K and V heads go to cache slot slot_mapping[m] of k/v_cache
// [num_slots, Hkv, D] and k/v_scales [num_slots, Hkv].  A negative slot is
// skipped (a padding token); a slot >= num_slots is skipped and flagged.
struct QkvDst {
    int16_t* qc;
    float* qs;
    int16_t* kc;
    float* ks;
    int16_t* vc;
    float* vs;
    const int64_t* slots;
    int64_t num_slots;
    int hq, hkv, d;
    uint32_t* status;
    __device__ bool at(int64_t r, int16_t*& c, float*& s) const {
        const int H = hq + 2 * hkv;
        const int64_t m = r / H;
        const int h = (int)(r - m * H);
        if (h < hq) {
            c = qc + (m * hq + h) * d;
            s = qs + m * hq + h;
            return true;
        }
        const int64_t slot = slots[m];
        if (slot < 0) return false;
        if (slot >= num_slots) {
            if (status) atomicOr(status, (uint32_t)HEAL_FLAG_SLOT_RANGE);
            return false;
        }
        const bool is_k = h < hq + hkv;
        const int hk = is_k ? h - hq : h - hq - hkv;
        c = (is_k ? kc : vc) + (slot * hkv + hk) * d;
        s = (is_k ? ks : vs) + slot * hkv + hk;
        return true;
    }
};

// ---- launchers (return the launch status; never synchronize) -------------
hipError_t launch_split(const float* X, int64_t n, uint16_t* hi, uint16_t* lo, uint32_t* status,
                        hipStream_t s);
// Pack rows into the layout above.  src holds fp32 values (normalized rows,
// hi/res form), or binary16 values when f16 (hi-only form, exponents 0).
// kn == 0: src is [rows, K] with ld; kn == 1: src is [K, rows] with ld (the
// packed operand is its transpose).  kshift (nullable): element (r, k) is
// multiplied by 2^-kshift[k] first (before the row's maximum is taken).
hipError_t launch_pack(const void* src, bool f16, int64_t ld, int64_t rows, int64_t K, int kn,
                       const int8_t* kshift, void* packed, uint32_t* status, hipStream_t s);
// The normalized hi parts alone of fp32 rows [rows, K], in the hi-only packed
// layout with their exponents, for the one-product mode.
hipError_t launch_pack_hi_f32(const float* src, int64_t ld, int64_t rows, int64_t K, void* packed, uint32_t* status,
                              hipStream_t s);
// BF16 three-way packing of fp32 rows (kn as for launch_pack); status gets
// HEAL_FLAG_F16_RANGE where a value's bf16 high part is not finite.
hipError_t launch_pack_bf16x3(const float* src, int64_t ld, int64_t rows, int64_t K, int kn, void* packed,
                              uint32_t* status, hipStream_t s);
// out = src with element (r, k) multiplied by 2^-kshift[k], same element type
// and layout (kn as above), ldo for out.
hipError_t launch_scale_k(const void* src, bool f16, int64_t ld, int64_t rows, int64_t K, int kn,
                          const int8_t* kshift, void* out, int64_t ldo, hipStream_t s);

hipError_t launch_quant(const float* X, int64_t rows, int64_t D, int64_t ldx, int16_t* codes,
                        int64_t ldq, float* scales, hipStream_t s);
// Quantize the rows of a Q/K/V projection output C [M, (Hq + 2 Hkv) D]
// (contiguous): Q heads to q_codes/q_scales, K and V heads to their cache
// slots slot_mapping[m] (negative: skipped; >= num_slots: skipped and flagged).
hipError_t launch_quant_qkv(const float* C, int64_t M, int64_t Hq, int64_t Hkv, int64_t D, int16_t* q_codes,
                            float* q_scales, const int64_t* slot_mapping, int64_t num_slots, int16_t* k_cache,
                            float* k_scales, int16_t* v_cache, float* v_scales, uint32_t* status, hipStream_t s);
hipError_t launch_dequant(const int16_t* codes, int64_t rows, int64_t D, int64_t ldq,
                          const float* scales, int fmt, void* out, void* out_lo, int64_t ldo,
                          hipStream_t s);

// C[M,N] from packed A (rows M) and packed B (rows N) with nprod products
// per k step: 3 (both fp32), 2 (B a 16-bit weight: A_hi.B_lo skipped), 1
// (plain FP16: A_hi.B_hi alone), or 6: the BF16 three-way mode (both
// operands in that packed form; b_hi ignored).  b_hi: B is in the hi-only form;
// a_hi (one product only): A is too.
// qkv (nullable): instead of storing C, quantize each (token, head) row of
// D = 128 outputs to INT16 in the epilogue and write it as dst.at() directs
// (3- and 2-product forms, shapes without the k split: see prefill_ksplit).
// The packed operands carry their row exponents (except in the BF16 mode):
// C = acc 2^-(e_a[m] + e_b[n]).
hipError_t launch_gemm_prefill(const void* Apk, const void* Bpk, int nprod, bool b_hi, float* C, int64_t ldc,
                               int64_t M, int64_t N, int64_t K, hipStream_t s, const QkvDst* qkv = nullptr,
                               bool a_hi = false);
// Whether the prefill kernel splits the k range of this shape in two.
bool prefill_ksplit(int64_t M, int64_t N, int64_t K);

// Decode path (M <= 64): W [N,K] streamed (fp32 split in registers, or
// binary16) or packed once, the activation normalized per row and 128-wide k
// block (in the GEMM kernel up to 16 rows and where that work stays light,
// else by a first small kernel that writes the split blocks).  Workspace,
// each part 256-byte aligned: the split-K flags (c_bytes), the split
// activation block images (a_bytes, M > 16), the split-K partials (p_bytes).
struct DecodePlan {
    int splits;        // number of K chunks (fixed by N and K only)
    int64_t kchunk;    // reduction length of one chunk (multiple of 256)
    int64_t ncount;    // split-K flags (per 64-row block of W and chunk), 0 without split-K
    int64_t c_bytes;   // workspace bytes of the flags
    int64_t a_bytes;   // workspace bytes of the split activation planes
    int64_t p_bytes;   // workspace bytes of the split-K partials
    int64_t bytes() const;
};
DecodePlan decode_plan(int64_t M, int64_t N, int64_t K);
// Whether the plan's k chunks are the waves of one workgroup and meet in LDS
// (one row tile, 2 .. 8 chunks of at most 4 blocks, at least 256 slices of 16
// rows, no a_kshift): no split-K completion through memory, so no epoch.
bool decode_chunks_as_waves(int64_t M, int64_t N, const DecodePlan& p, bool kshift);
// W is fp32, or binary16 values when wf16 (the two-product form); one: plain
// FP16 (A_hi.W_hi alone).  kshift (nullable): A's element (m, k) is
// multiplied by 2^-kshift[k] before its split.
// epoch: a number no earlier call in the process used (the split-K counters
// tell this call's arrivals from stale contents by it).
// packed: W is a heal_pack_w buffer for (N, K) (hi-only when wf16); ldw is
// then ignored.  Split-K completion: with counters == nullptr, flags in the
// workspace compared against `epoch` (a value no earlier call on this
// workspace used, never 0); otherwise `counters`, one 8-byte counter per
// workgroup row group (ceil(N / 64) suffice), zero on entry and left zero
// (the form a replayed graph needs).
hipError_t launch_gemm_decode(const float* A, int64_t lda, const int8_t* kshift, const void* W, bool wf16,
                              bool packed, bool one, int64_t ldw, float* C, int64_t ldc, int64_t M, int64_t N,
                              int64_t K, void* workspace, const DecodePlan& plan, uint64_t epoch,
                              unsigned long long* counters, uint32_t* status, hipStream_t s);
// A fresh call epoch (48 bits, never 0; thread-safe).
uint64_t next_epoch();
// Whether heal_gemm_f32c runs this shape and these flags on the decode kernel.
bool decode_path(int64_t M, int64_t K, uint32_t flags);
// heal_gemm_f32c on the decode path with the split-K counters of
// launch_gemm_decode (zero on entry, left zero) instead of epoch flags.
heal_status gemm_f32c_counters(const float* A, int64_t lda, const void* W, int64_t ldw, float* C, int64_t ldc,
                               int64_t M, int64_t N, int64_t K, uint32_t flags, const int8_t* a_kshift,
                               void* workspace, size_t workspace_bytes, unsigned long long* counters,
                               uint32_t* dev_status, void* stream);

int64_t attn_workspace_bytes(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D);
// Causal self-attention of a prompt: q [B, T, Hq, D], k/v [B, T, Hkv, D] INT16
// codes with scales [B, T, H]; out fp32 [B, T, Hq, D].
hipError_t launch_attn_prefill(const int16_t* q, const float* qs, const int16_t* k, const float* ks,
                               const int16_t* v, const float* vs, float* out, int64_t B, int64_t T, int64_t Hq,
                               int64_t Hkv, int64_t D, hipStream_t s);
hipError_t launch_attn_decode(const int16_t* q, const float* qs, const int16_t* k, const float* ks,
                              const int16_t* v, const float* vs, float* out, int64_t B, int64_t T,
                              int64_t Hq, int64_t Hkv, int64_t D, void* workspace, hipStream_t s);

}  // namespace heal
