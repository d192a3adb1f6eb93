// Operand split into the dual-FP16 pair x ~= hi + lo / 2^10.
//
// HEAL paper, section 3, "Mitigating GEMM Truncation via FP16 Promotion and
// Algebraic Compensation": the FP32 input is decomposed into an FP16 value
// plus an FP16 residual shifted by 2^10, so that 16-bit matrix units can
// evaluate the product; FP16's narrow dynamic range is handled by targeted
// power-of-two rescaling.  Kernels:
//  * split_kernel: plain elementwise planes (hi[], lo[]), bit-exact.
//  * pack kernels: the operand rows of the prefill GEMM, each normalized by
//    the power of two that puts its largest magnitude in [2^14, 2^15), split
//    as hi = fp16(x'), res = fp16(x' - hi) and written straight into the
//    padded, hi/res-interleaved layout the GEMM streams (one 128-byte line per
//    row and 32-wide k block), with the row exponents after the rows, so the
//    GEMM needs no bounds checks and no scaling in its main loop; a binary16
//    source packs its hi parts alone (not normalized), and an optional
//    per-channel power of two scales the source first.
//  * pack_bf16x3_kernel: the BF16 three-way split of the precision mode, in
//    the same padded layout with three 64-byte planes per k block.
//  * scale_k_kernel: the per-channel power-of-two rescaling of an operand.
// All are HBM-bound streaming maps (4 bytes read and 4 written per element
// for the fp32 split).
#include <algorithm>

#include "heal_internal.h"

namespace heal {

__global__ __launch_bounds__(256) void split_kernel(const float4* __restrict__ X, int64_t n,
                                                    uint2* __restrict__ hi, uint2* __restrict__ lo,
                                                    uint32_t* __restrict__ status) {
    const int64_t n4 = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 x = X[i];
        _Float16 h0, h1, h2, h3, l0, l1, l2, l3;
        split_one(x.x, h0, l0);
        split_one(x.y, h1, l1);
        split_one(x.z, h2, l2);
        split_one(x.w, h3, l3);
        bad |= f16_out_of_range4(x);
        hi[i] = make_uint2(f16_bits(h0) | ((uint32_t)f16_bits(h1) << 16),
                           f16_bits(h2) | ((uint32_t)f16_bits(h3) << 16));
        lo[i] = make_uint2(f16_bits(l0) | ((uint32_t)f16_bits(l1) << 16),
                           f16_bits(l2) | ((uint32_t)f16_bits(l3) << 16));
    }
    // ragged tail (n % 4 elements), one thread each
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < (n & 3)) {
        const float* Xs = reinterpret_cast<const float*>(X);
        int64_t j = (n4 << 2) + t;
        _Float16 h, l;
        split_one(Xs[j], h, l);
        bad |= f16_out_of_range(Xs[j]);
        reinterpret_cast<uint16_t*>(hi)[j] = f16_bits(h);
        reinterpret_cast<uint16_t*>(lo)[j] = f16_bits(l);
    }
    if (bad && status) atomicOr(status, (uint32_t)HEAL_FLAG_F16_RANGE);
}

hipError_t launch_split(const float* X, int64_t n, uint16_t* hi, uint16_t* lo, uint32_t* status,
                        hipStream_t s) {
    if (n == 0) return hipSuccess;
    int64_t n4 = n >> 2;
    int64_t blocks = (std::max<int64_t>(n4, 4) + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;
    hipLaunchKernelGGL(split_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(X), n, reinterpret_cast<uint2*>(hi),
                       reinterpret_cast<uint2*>(lo), status);
    return hipGetLastError();
}

// Source element T: float, or uint16_t holding binary16 values (whose split
// is the value itself with a zero residual).  A 16-bit source is written in
// the hi-only form (its lo parts would all be zero).
__device__ __forceinline__ float src_value(float x) { return x; }
__device__ __forceinline__ float src_value(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// x * 2^-kshift[k] (exact for normal results); kshift may be NULL.
__device__ __forceinline__ float kscaled(float x, const int8_t* kshift, int64_t k) {
    return kshift ? __builtin_ldexpf(x, -(int)kshift[k]) : x;
}

// Packed layout writer, source rows contiguous in k ([rows, K], ld).
// One thread per (row, 4 consecutive k); the grid covers the padded extent
// so the zero padding is written too.  kshift (nullable): element (r, k) is
// multiplied by 2^-kshift[k] before its split.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void pack_rowmajor_kernel(const T* __restrict__ src, int64_t ld,
                                                            int64_t rows, int64_t K, int64_t Kp,
                                                            int64_t rows_p, const int8_t* __restrict__ kshift,
                                                            uint16_t* __restrict__ out, int* __restrict__ exps,
                                                            uint32_t* __restrict__ status) {
    const int64_t kq = Kp >> 2;  // 4-wide groups per padded row
    const int64_t total = rows_p * kq;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / kq;
        const int64_t k = (i - r * kq) << 2;
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (r < rows) {
            const T* p = src + r * ld + k;
            if (VEC && k + 4 <= K) {
                if constexpr (sizeof(T) == 4) {
                    float4 v = *reinterpret_cast<const float4*>(p);
                    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
                } else {
                    const uint2 v = *reinterpret_cast<const uint2*>(p);
                    x[0] = src_value((uint16_t)(v.x & 0xffff)); x[1] = src_value((uint16_t)(v.x >> 16));
                    x[2] = src_value((uint16_t)(v.y & 0xffff)); x[3] = src_value((uint16_t)(v.y >> 16));
                }
            } else {
                for (int j = 0; j < 4; ++j)
                    if (k + j < K) x[j] = src_value(p[j]);
            }
            if (kshift)
                for (int j = 0; j < 4; ++j)
                    if (k + j < K) x[j] = kscaled(x[j], kshift, k + j);
        }
        uint16_t h[4], l[4];
        if constexpr (sizeof(T) == 4) {   // the row's normalization (exponents from rowexp_*_kernel)
            const int e = exps[r];
            for (int j = 0; j < 4; ++j) x[j] = __builtin_ldexpf(x[j], e);
        } else if (k == 0) {
            exps[r] = 0;                  // a 16-bit source is not normalized
        }
        for (int j = 0; j < 4; ++j) {
            _Float16 hh, ll;
            split_res(x[j], hh, ll);
            bad |= f16_out_of_range(x[j]);
            h[j] = f16_bits(hh);
            l[j] = f16_bits(ll);
        }
        if constexpr (sizeof(T) == 2) {   // a 16-bit source: the hi-only form
            uint16_t* o = out + r * (pack_row_bytes_hi(K) / 2) + k;
            *reinterpret_cast<uint2*>(o) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
        } else {
            uint16_t* o = out + r * (pack_row_bytes(K) / 2) + (k / kPackK) * (2 * kPackK) + (k % kPackK);
            *reinterpret_cast<uint2*>(o) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
            *reinterpret_cast<uint2*>(o + kPackK) =
                make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
        }
    }
    if (bad && status) atomicOr(status, (uint32_t)HEAL_FLAG_F16_RANGE);
}

// Packed layout writer for a source stored [K, rows] (ld >= rows): the packed
// operand is the transpose.  Threads run along the source row (the packed
// row index) so reads are coalesced; each thread packs 4 consecutive k.
template <typename T>
__global__ __launch_bounds__(256) void pack_colmajor_kernel(const T* __restrict__ src, int64_t ld,
                                                            int64_t rows, int64_t K, int64_t Kp,
                                                            int64_t rows_p, const int8_t* __restrict__ kshift,
                                                            uint16_t* __restrict__ out, int* __restrict__ exps,
                                                            uint32_t* __restrict__ status) {
    const int64_t kq = Kp >> 2;
    const int64_t total = rows_p * kq;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t kg = i / rows_p;
        const int64_t r = i - kg * rows_p;
        const int64_t k = kg << 2;
        int e = 0;
        if constexpr (sizeof(T) == 4) e = exps[r];   // the row's normalization
        else if (k == 0) exps[r] = 0;                 // a 16-bit source is not normalized
        uint16_t h[4], l[4];
        for (int j = 0; j < 4; ++j) {
            float x = (r < rows && k + j < K) ? kscaled(src_value(src[(k + j) * ld + r]), kshift, k + j) : 0.f;
            if constexpr (sizeof(T) == 4) x = __builtin_ldexpf(x, e);
            _Float16 hh, ll;
            split_res(x, hh, ll);
            bad |= f16_out_of_range(x);
            h[j] = f16_bits(hh);
            l[j] = f16_bits(ll);
        }
        if constexpr (sizeof(T) == 2) {   // a 16-bit source: the hi-only form
            uint16_t* o = out + r * (pack_row_bytes_hi(K) / 2) + k;
            *reinterpret_cast<uint2*>(o) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
        } else {
            uint16_t* o = out + r * (pack_row_bytes(K) / 2) + (k / kPackK) * (2 * kPackK) + (k % kPackK);
            *reinterpret_cast<uint2*>(o) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
            *reinterpret_cast<uint2*>(o + kPackK) =
                make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
        }
    }
    if (bad && status) atomicOr(status, (uint32_t)HEAL_FLAG_F16_RANGE);
}

__device__ __forceinline__ float wave_max(float m) { return max_swap32(max_half(m)); }

// Largest magnitude of the workgroup's values (256 threads); red holds 4
// floats of LDS and is free again when this returns.
__device__ __forceinline__ float block_max(float m, float* red) {
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return m;
}

// The fp32 row-major pack: one workgroup per packed row (grid-stride over the
// padded rows).  The row is loaded once into registers, MAXI items of 8
// consecutive k per thread (Kp <= 2048 MAXI), its largest magnitude reduced
// across the workgroup, and the normalized values split and stored: 16 bytes
// into each of the hi and res halves of the row's 128-byte line for that k
// block (or one 16-byte store of hi parts in the hi-only form).  VEC: rows
// 16-byte aligned.  SHIFT: element (r, k) is multiplied by 2^-kshift[k]
// first.  Padding rows and k write zeros and exponent 0.
template <bool HI_ONLY, bool VEC, bool SHIFT, int MAXI>
__global__ __launch_bounds__(256) void pack_rows_norm_kernel(const float* __restrict__ src, int64_t ld,
                                                             int64_t rows, int64_t K, int64_t Kp, int64_t rows_p,
                                                             const int8_t* __restrict__ kshift,
                                                             uint16_t* __restrict__ out, int* __restrict__ exps,
                                                             uint32_t* __restrict__ status) {
    __shared__ float red[4];
    const int c8n = (int)(Kp >> 3);
    const int tid = threadIdx.x;
    bool bad = false;
    for (int64_t r = blockIdx.x; r < rows_p; r += gridDim.x) {
        float x[MAXI][8];
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < MAXI; ++j) {
            const int c8 = tid + 256 * j;
            const int64_t k = (int64_t)c8 << 3;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[j][i] = 0.0f;
            if (r < rows && c8 < c8n) {
                const float* p = src + r * ld + k;
                if (VEC && k + 8 <= K) {
                    const float4 a = *reinterpret_cast<const float4*>(p);
                    const float4 b = *reinterpret_cast<const float4*>(p + 4);
                    x[j][0] = a.x; x[j][1] = a.y; x[j][2] = a.z; x[j][3] = a.w;
                    x[j][4] = b.x; x[j][5] = b.y; x[j][6] = b.z; x[j][7] = b.w;
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (k + i < K) x[j][i] = p[i];
                }
                if constexpr (SHIFT) {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (k + i < K) x[j][i] = __builtin_ldexpf(x[j][i], -(int)kshift[k + i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(x[j][i]));
        }
        m = block_max(m, red);
        bad |= !(m <= 3.40282347e38f);   // an infinite (or NaN) element
        const int e = row_norm_exp(m);
        if (tid == 0) exps[r] = e;
#pragma unroll
        for (int j = 0; j < MAXI; ++j) {
            const int c8 = tid + 256 * j;
            if (c8 >= c8n) break;
            const int64_t k = (int64_t)c8 << 3;
            uint32_t h[4], l[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                _Float16 h0, l0, h1, l1;
                split_res(__builtin_ldexpf(x[j][i], e), h0, l0);
                split_res(__builtin_ldexpf(x[j][i + 1], e), h1, l1);
                h[i >> 1] = f16_bits(h0) | ((uint32_t)f16_bits(h1) << 16);
                l[i >> 1] = f16_bits(l0) | ((uint32_t)f16_bits(l1) << 16);
            }
            if constexpr (HI_ONLY) {   // the hi-only layout: Kp fp16 per row
                *reinterpret_cast<uint4*>(out + r * (pack_row_bytes_hi(K) / 2) + k) = make_uint4(h[0], h[1], h[2], h[3]);
            } else {
                uint16_t* o = out + r * (pack_row_bytes(K) / 2) + (k / kPackK) * (2 * kPackK) + (k % kPackK);
                *reinterpret_cast<uint4*>(o) = make_uint4(h[0], h[1], h[2], h[3]);
                *reinterpret_cast<uint4*>(o + kPackK) = make_uint4(l[0], l[1], l[2], l[3]);
            }
        }
    }
    if (bad && status && tid == 0) atomicOr(status, (uint32_t)HEAL_FLAG_F16_RANGE);
}

// Row exponents for the general pack path.  [rows, K] source (kn == 0): one
// workgroup per row, threads along k.  [K, rows] source (kn == 1): one thread
// per packed row, walking k down its column (neighbouring threads read
// neighbouring addresses).  Padding rows get 0.
__global__ __launch_bounds__(256) void rowexp_nk_kernel(const float* __restrict__ src, int64_t ld, int64_t rows,
                                                        int64_t K, int64_t rows_p, const int8_t* __restrict__ kshift,
                                                        int* __restrict__ exps) {
    __shared__ float red[4];
    for (int64_t r = blockIdx.x; r < rows_p; r += gridDim.x) {
        float m = 0.0f;
        if (r < rows)
            for (int64_t k = threadIdx.x; k < K; k += 256) m = fmaxf(m, __builtin_fabsf(kscaled(src[r * ld + k], kshift, k)));
        m = block_max(m, red);
        if (threadIdx.x == 0) exps[r] = row_norm_exp(m);
    }
}

__global__ __launch_bounds__(256) void rowexp_kn_kernel(const float* __restrict__ src, int64_t ld, int64_t rows,
                                                        int64_t K, int64_t rows_p, const int8_t* __restrict__ kshift,
                                                        int* __restrict__ exps) {
    for (int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x; r < rows_p; r += (int64_t)gridDim.x * 256) {
        float m = 0.0f;
        if (r < rows)
            for (int64_t k = 0; k < K; ++k) m = fmaxf(m, __builtin_fabsf(kscaled(src[k * ld + r], kshift, k)));
        exps[r] = row_norm_exp(m);
    }
}

namespace {
// the fused row pack, items of 8 k per thread: MAXI 2 (Kp <= 4096) or 8 (<= 16384)
template <bool HI_ONLY, bool VEC, bool SHIFT>
void launch_rows_norm(const float* p, int64_t ld, int64_t rows, int64_t K, int64_t Kp, int64_t rows_p,
                      const int8_t* kshift, uint16_t* out, int* exps, uint32_t* status, hipStream_t s) {
    const dim3 grid((unsigned)std::min<int64_t>(rows_p, 65536));
    if (Kp <= 4096)
        hipLaunchKernelGGL((pack_rows_norm_kernel<HI_ONLY, VEC, SHIFT, 2>), grid, dim3(256), 0, s, p, ld, rows, K, Kp,
                           rows_p, kshift, out, exps, status);
    else
        hipLaunchKernelGGL((pack_rows_norm_kernel<HI_ONLY, VEC, SHIFT, 8>), grid, dim3(256), 0, s, p, ld, rows, K, Kp,
                           rows_p, kshift, out, exps, status);
}
constexpr int64_t kRowsNormMaxKp = 16384;
}  // namespace

hipError_t launch_pack(const void* src, bool f16, int64_t ld, int64_t rows, int64_t K, int kn,
                       const int8_t* kshift, void* packed, uint32_t* status, hipStream_t s) {
    const int64_t Kp = pack_kp(K), rows_p = pack_rows(rows);
    const int64_t total = rows_p * (Kp >> 2);
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    uint16_t* out = static_cast<uint16_t*>(packed);
    int* exps = reinterpret_cast<int*>(static_cast<unsigned char*>(packed) +
                                       (f16 ? pack_data_bytes_hi(rows, K) : pack_data_bytes(rows, K)));
    const uintptr_t align = f16 ? 7 : 15;   // 4 elements per vector load
    const bool vec = (reinterpret_cast<uintptr_t>(src) & align) == 0 && (ld & 3) == 0;
    if (f16) {
        const uint16_t* p = static_cast<const uint16_t*>(src);
        if (kn)
            hipLaunchKernelGGL(pack_colmajor_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, p, ld,
                               rows, K, Kp, rows_p, kshift, out, exps, status);
        else if (vec)
            hipLaunchKernelGGL((pack_rowmajor_kernel<uint16_t, true>), dim3((unsigned)blocks), dim3(256), 0, s, p,
                               ld, rows, K, Kp, rows_p, kshift, out, exps, status);
        else
            hipLaunchKernelGGL((pack_rowmajor_kernel<uint16_t, false>), dim3((unsigned)blocks), dim3(256), 0, s,
                               p, ld, rows, K, Kp, rows_p, kshift, out, exps, status);
        return hipGetLastError();
    }
    const float* p = static_cast<const float*>(src);
    if (!kn && Kp <= kRowsNormMaxKp) {   // one pass: the row in registers
        if (vec && kshift) launch_rows_norm<false, true, true>(p, ld, rows, K, Kp, rows_p, kshift, out, exps, status, s);
        else if (vec) launch_rows_norm<false, true, false>(p, ld, rows, K, Kp, rows_p, kshift, out, exps, status, s);
        else if (kshift) launch_rows_norm<false, false, true>(p, ld, rows, K, Kp, rows_p, kshift, out, exps, status, s);
        else launch_rows_norm<false, false, false>(p, ld, rows, K, Kp, rows_p, kshift, out, exps, status, s);
        return hipGetLastError();
    }
    // general path: the row exponents first, then the split
    if (kn)
        hipLaunchKernelGGL(rowexp_kn_kernel, dim3((unsigned)std::min<int64_t>((rows_p + 255) / 256, 4096)), dim3(256),
                           0, s, p, ld, rows, K, rows_p, kshift, exps);
    else
        hipLaunchKernelGGL(rowexp_nk_kernel, dim3((unsigned)std::min<int64_t>(rows_p, 65536)), dim3(256), 0, s, p, ld,
                           rows, K, rows_p, kshift, exps);
    if (kn)
        hipLaunchKernelGGL(pack_colmajor_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, p, ld, rows, K, Kp,
                           rows_p, kshift, out, exps, status);
    else if (vec)
        hipLaunchKernelGGL((pack_rowmajor_kernel<float, true>), dim3((unsigned)blocks), dim3(256), 0, s, p, ld, rows,
                           K, Kp, rows_p, kshift, out, exps, status);
    else
        hipLaunchKernelGGL((pack_rowmajor_kernel<float, false>), dim3((unsigned)blocks), dim3(256), 0, s, p, ld,
                           rows, K, Kp, rows_p, kshift, out, exps, status);
    return hipGetLastError();
}

hipError_t launch_pack_hi_f32(const float* src, int64_t ld, int64_t rows, int64_t K, void* packed, uint32_t* status,
                              hipStream_t s) {
    const int64_t Kp = pack_kp(K), rows_p = pack_rows(rows);
    if (rows_p * Kp == 0) return hipSuccess;
    if ((reinterpret_cast<uintptr_t>(src) & 15) != 0 || (ld & 3) != 0 || Kp > kRowsNormMaxKp)
        return hipErrorInvalidValue;
    int* exps = reinterpret_cast<int*>(static_cast<unsigned char*>(packed) + pack_data_bytes_hi(rows, K));
    launch_rows_norm<true, true, false>(src, ld, rows, K, Kp, rows_p, nullptr, static_cast<uint16_t*>(packed), exps,
                                        status, s);
    return hipGetLastError();
}

// ---- BF16 three-way split (a precision mode with fp32's exponent range) ----
// x = b0 + b1 + b2 with b0 = bf16(x), b1 = bf16(x - b0), b2 = bf16(x - b0 - b1),
// round to nearest even (the hardware conversion); both residuals are exact
// in fp32, and the three 8-bit significands hold all 24 of x's bits while the
// last part is a normal bf16 (|x| above about 2^-110).  A part is non-finite only if |x| rounds past bf16's largest value.
__device__ __forceinline__ void split3_bf16(float x, uint16_t& b0, uint16_t& b1, uint16_t& b2) {
    const __bf16 h0 = (__bf16)x;
    const float r1 = x - (float)h0;
    const __bf16 h1 = (__bf16)r1;
    const __bf16 h2 = (__bf16)(r1 - (float)h1);
    b0 = __builtin_bit_cast(uint16_t, h0);
    b1 = __builtin_bit_cast(uint16_t, h1);
    b2 = __builtin_bit_cast(uint16_t, h2);
}

// One item = 8 consecutive k of one row: reads 8 fp32 values (zero past the
// operand), writes 16 bytes into each of the three planes of its 32-wide k
// block.  kn == 0: src [rows, K] (k fastest across items); kn == 1: src
// [K, rows] (r fastest, so neighbouring items read neighbouring addresses).
template <int KN>
__global__ __launch_bounds__(256) void pack_bf16x3_kernel(const float* __restrict__ src, int64_t ld, int64_t rows,
                                                          int64_t K, int64_t Kp, int64_t rows_p,
                                                          uint16_t* __restrict__ out,
                                                          uint32_t* __restrict__ status) {
    const int64_t k8n = Kp >> 3;
    const int64_t total = rows_p * k8n;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        int64_t r, c8;
        if (KN) {
            c8 = i / rows_p;
            r = i - c8 * rows_p;
        } else {
            r = i / k8n;
            c8 = i - r * k8n;
        }
        const int64_t k0 = c8 << 3;
        uint32_t w0[4], w1[4], w2[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            uint16_t a0, a1, a2, c0, c1, c2;
            const int64_t ka = k0 + j, kb = k0 + j + 1;
            const float xa = (r < rows && ka < K) ? (KN ? src[ka * ld + r] : src[r * ld + ka]) : 0.f;
            const float xb = (r < rows && kb < K) ? (KN ? src[kb * ld + r] : src[r * ld + kb]) : 0.f;
            split3_bf16(xa, a0, a1, a2);
            split3_bf16(xb, c0, c1, c2);
            bad |= (a0 & 0x7F80u) == 0x7F80u;
            bad |= (c0 & 0x7F80u) == 0x7F80u;
            w0[j >> 1] = a0 | ((uint32_t)c0 << 16);
            w1[j >> 1] = a1 | ((uint32_t)c1 << 16);
            w2[j >> 1] = a2 | ((uint32_t)c2 << 16);
        }
        uint16_t* o = out + r * (Kp * 3) + (k0 / kPackK) * (3 * kPackK) + (k0 % kPackK);
        *reinterpret_cast<uint4*>(o) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
        *reinterpret_cast<uint4*>(o + kPackK) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
        *reinterpret_cast<uint4*>(o + 2 * kPackK) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
    }
    if (bad && status) atomicOr(status, (uint32_t)HEAL_FLAG_F16_RANGE);
}

hipError_t launch_pack_bf16x3(const float* src, int64_t ld, int64_t rows, int64_t K, int kn, void* packed,
                              uint32_t* status, hipStream_t s) {
    const int64_t Kp = pack_kp(K), rows_p = pack_rows(rows);
    const int64_t total = rows_p * (Kp >> 3);
    if (total == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 256 * 64);
    uint16_t* out = static_cast<uint16_t*>(packed);
    if (kn)
        hipLaunchKernelGGL(pack_bf16x3_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, src, ld, rows, K, Kp,
                           rows_p, out, status);
    else
        hipLaunchKernelGGL(pack_bf16x3_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, src, ld, rows, K, Kp,
                           rows_p, out, status);
    return hipGetLastError();
}

// out = src with element (r, k) multiplied by 2^-kshift[k]: rows of K
// ([rows, K], kn == 0) or K rows of `rows` ([K, rows], kn == 1).  Exact for
// results in the format's normal range.
template <typename T>
__global__ __launch_bounds__(256) void scale_k_kernel(const T* __restrict__ src, int64_t ld, int64_t rows,
                                                      int64_t K, int kn, const int8_t* __restrict__ kshift,
                                                      T* __restrict__ out, int64_t ldo) {
    const int64_t total = rows * K;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        // kn == 0: i runs along k within a row; kn == 1: along the row within a k
        const int64_t outer = kn ? i / rows : i / K;
        const int64_t inner = kn ? i - outer * rows : i - outer * K;
        const int64_t k = kn ? outer : inner;
        const int e = -(int)kshift[k];
        if constexpr (sizeof(T) == 4) {
            out[outer * ldo + inner] = __builtin_ldexpf(src[outer * ld + inner], e);
        } else {
            const float v = (float)__builtin_bit_cast(_Float16, src[outer * ld + inner]);
            out[outer * ldo + inner] = __builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf(v, e));
        }
    }
}

hipError_t launch_scale_k(const void* src, bool f16, int64_t ld, int64_t rows, int64_t K, int kn,
                          const int8_t* kshift, void* out, int64_t ldo, hipStream_t s) {
    const int64_t total = rows * K;
    if (total == 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 256 * 64);
    if (f16)
        hipLaunchKernelGGL(scale_k_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint16_t*>(src), ld, rows, K, kn, kshift, static_cast<uint16_t*>(out),
                           ldo);
    else
        hipLaunchKernelGGL(scale_k_kernel<float>, dim3(blocks), dim3(256), 0, s, static_cast<const float*>(src),
                           ld, rows, K, kn, kshift, static_cast<float*>(out), ldo);
    return hipGetLastError();
}

}  // namespace heal
