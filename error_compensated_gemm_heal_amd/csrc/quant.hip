// INT16 quantization and dequantization of Q/K/V rows.
//
// HEAL paper, section 3, "Mitigating QKV Truncation Error via INT16
// Quantization": Q_INT16(X) = Round((2^15 - 1) X / max|X|), one max per
// row of D values (token x head); step Delta = M / (2^15 - 1).  The INT16
// code is later unpacked into the exact dual-FP16 pair hi + lo / 2^10.
//
// Both kernels are HBM-bound streaming maps (6 bytes per element plus 4 per
// row).  A row of D floats is owned by a group of LPR lanes of one wave
// (LPR = D/4 rounded up to a power of two, at most 64).  Each lane holds
// NCH float4 chunks in registers, so a row is read from HBM once; a wave
// issues the loads of several row groups before processing any of them, with
// the non-temporal hint (each input byte is read once), and the grid holds up
// to 80 blocks per compute unit before it strides.  The row
// maximum is a butterfly over the group, which is exact and order-free.  The
// per-element arithmetic follows the formula's own order with correctly
// rounded fp32 operations: t = fl(32767 x), u = fl(t / M), q = rne(u).  That
// makes the codes identical to a scalar CPU evaluation of the same formula.
#include "heal_internal.h"

namespace heal {

namespace {

// Each wave step covers U groups of RPW consecutive rows; all U x NCH
// loads of a step are issued before any of them is used, so a wave keeps
// U x 1 KB (or more) of reads in flight.
template <int LPR, int NCH>
struct RowTiling {
    static constexpr int RPW = 64 / LPR;                 // rows per wave per group
    static constexpr int U = NCH >= 4 ? 1 : 4 / NCH;     // row groups per step
    static constexpr int ROWS = U * RPW;                 // rows per wave per step
};

// Where a quantized row goes: at(r, codes, scale) sets the row's D codes and
// its scale, or returns false for a row that is not written.
struct PlainDst {   // codes [rows, ldq], scales [rows]
    int16_t* codes;
    int64_t ldq;
    float* scales;
    __device__ bool at(int64_t r, int16_t*& c, float*& s) const {
        c = codes + r * ldq;
        s = scales + r;
        return true;
    }
};

template <int LPR, int NCH, class Dst>
__global__ __launch_bounds__(256) void quant_kernel(const float* __restrict__ X, int64_t rows, int D,
                                                    int64_t ldx, Dst dst) {
    using RT = RowTiling<LPR, NCH>;
    const int lane = threadIdx.x & 63;
    const int sub = lane / LPR;     // which row of a group
    const int gl = lane % LPR;      // lane within the row group
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int d4 = D >> 2;

    for (int64_t r0 = wave * RT::ROWS; r0 < rows; r0 += nwaves * RT::ROWS) {
        float4 x[RT::U][NCH];
#pragma unroll
        for (int u = 0; u < RT::U; ++u) {
            const int64_t r = r0 + u * RT::RPW + sub;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int j = gl + c * LPR;
                x[u][c] = (r < rows && j < d4) ? load_nt_f4(X + r * ldx + 4 * j)
                                               : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < RT::U; ++u) {
            const int64_t r = r0 + u * RT::RPW + sub;
            float m = 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                m = fmaxf(m, fmaxf(fmaxf(__builtin_fabsf(x[u][c].x), __builtin_fabsf(x[u][c].y)),
                                   fmaxf(__builtin_fabsf(x[u][c].z), __builtin_fabsf(x[u][c].w))));
#pragma unroll
            for (int off = LPR / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
            if (r >= rows) continue;
            int16_t* crow;
            float* srow;
            if (!dst.at(r, crow, srow)) continue;
            if (gl == 0) *srow = (m == 0.0f) ? 0.0f : __fdiv_rn(m, 32767.0f);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int j = gl + c * LPR;
                if (j < d4) {
                    short4 q;
                    if (m == 0.0f) {
                        q = make_short4(0, 0, 0, 0);
                    } else {
                        q.x = (short)__builtin_rintf(__fdiv_rn(__fmul_rn(32767.0f, x[u][c].x), m));
                        q.y = (short)__builtin_rintf(__fdiv_rn(__fmul_rn(32767.0f, x[u][c].y), m));
                        q.z = (short)__builtin_rintf(__fdiv_rn(__fmul_rn(32767.0f, x[u][c].z), m));
                        q.w = (short)__builtin_rintf(__fdiv_rn(__fmul_rn(32767.0f, x[u][c].w), m));
                    }
                    *reinterpret_cast<short4*>(crow + 4 * j) = q;
                }
            }
        }
    }
}

template <int LPR, int NCH, int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const int16_t* __restrict__ codes, int64_t rows,
                                                      int D, int64_t ldq, const float* __restrict__ scales,
                                                      void* __restrict__ out, void* __restrict__ out_lo,
                                                      int64_t ldo) {
    using RT = RowTiling<LPR, NCH>;
    const int lane = threadIdx.x & 63;
    const int sub = lane / LPR;
    const int gl = lane % LPR;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int d4 = D >> 2;
    for (int64_t r0 = wave * RT::ROWS; r0 < rows; r0 += nwaves * RT::ROWS) {
        short4 qv[RT::U][NCH];
        float sv[RT::U];
#pragma unroll
        for (int u = 0; u < RT::U; ++u) {
            const int64_t r = r0 + u * RT::RPW + sub;
            sv[u] = (FMT == HEAL_DQ_F32 && r < rows) ? scales[r] : 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int j = gl + c * LPR;
                qv[u][c] = (r < rows && j < d4) ? __builtin_bit_cast(short4, load_nt_8b(codes + r * ldq + 4 * j))
                                                : make_short4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < RT::U; ++u) {
            const int64_t r = r0 + u * RT::RPW + sub;
            if (r >= rows) continue;
            const float s = sv[u];
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int j = gl + c * LPR;
                if (j >= d4) continue;
                const short4 q = qv[u][c];
                if constexpr (FMT == HEAL_DQ_F32) {
                    float4 o = make_float4(__fmul_rn((float)q.x, s), __fmul_rn((float)q.y, s),
                                           __fmul_rn((float)q.z, s), __fmul_rn((float)q.w, s));
                    *reinterpret_cast<float4*>(static_cast<float*>(out) + r * ldo + 4 * j) = o;
                } else {
                    const float qf[4] = {(float)q.x, (float)q.y, (float)q.z, (float)q.w};
                    uint16_t h[4], l[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        _Float16 hh, ll;
                        split_one(qf[e], hh, ll);  // exact for every int16 code
                        h[e] = f16_bits(hh);
                        l[e] = f16_bits(ll);
                    }
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + r * ldo + 4 * j) =
                        make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out_lo) + r * ldo + 4 * j) =
                        make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
                }
            }
        }
    }
}

// Lanes per row and float4 chunks per lane for a row of D (D % 4 == 0, <= 4096).
void row_shape(int64_t D, int& lpr, int& nch) {
    int64_t d4 = D / 4;
    lpr = 1;
    while (lpr < d4 && lpr < 64) lpr <<= 1;
    int64_t c = (d4 + lpr - 1) / lpr;
    nch = 1;
    while (nch < c) nch <<= 1;
}

unsigned grid_for(int64_t rows, int rows_per_wave_step) {
    const int64_t waves = (rows + rows_per_wave_step - 1) / rows_per_wave_step;
    int64_t blocks = (waves + 3) / 4;  // 4 waves per 256-thread block
    const int64_t cap = 256 * 80;      // enough resident waves to cover HBM latency
    return (unsigned)std::max<int64_t>(1, std::min(blocks, cap));
}

}  // namespace

#define HEAL_QUANT_CASE(L, C)                                                                        \
    if (lpr == L && nch == C) {                                                                      \
        hipLaunchKernelGGL((quant_kernel<L, C, Dst>), dim3(grid_for(rows, RowTiling<L, C>::ROWS)), dim3(256), 0, s, X, \
                           rows, (int)D, ldx, dst);                                                  \
        return hipGetLastError();                                                                    \
    }

template <class Dst>
hipError_t launch_quant_to(const float* X, int64_t rows, int64_t D, int64_t ldx, const Dst& dst, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    int lpr, nch;
    row_shape(D, lpr, nch);
    HEAL_QUANT_CASE(1, 1) HEAL_QUANT_CASE(2, 1) HEAL_QUANT_CASE(4, 1) HEAL_QUANT_CASE(8, 1)
    HEAL_QUANT_CASE(16, 1) HEAL_QUANT_CASE(32, 1) HEAL_QUANT_CASE(64, 1) HEAL_QUANT_CASE(64, 2)
    HEAL_QUANT_CASE(64, 4) HEAL_QUANT_CASE(64, 8) HEAL_QUANT_CASE(64, 16)
    return hipErrorInvalidValue;
}
#undef HEAL_QUANT_CASE

hipError_t launch_quant(const float* X, int64_t rows, int64_t D, int64_t ldx, int16_t* codes,
                        int64_t ldq, float* scales, hipStream_t s) {
    return launch_quant_to(X, rows, D, ldx, PlainDst{codes, ldq, scales}, s);
}

hipError_t launch_quant_qkv(const float* C, int64_t M, int64_t Hq, int64_t Hkv, int64_t D, int16_t* q_codes,
                            float* q_scales, const int64_t* slot_mapping, int64_t num_slots, int16_t* k_cache,
                            float* k_scales, int16_t* v_cache, float* v_scales, uint32_t* status, hipStream_t s) {
    const QkvDst dst{q_codes, q_scales, k_cache, k_scales, v_cache, v_scales, slot_mapping, num_slots,
                     (int)Hq, (int)Hkv, (int)D, status};
    return launch_quant_to(C, M * (Hq + 2 * Hkv), D, D, dst, s);
}

#define HEAL_DQ_CASE(L, C)                                                                            \
    if (lpr == L && nch == C) {                                                                       \
        if (fmt == HEAL_DQ_F32)                                                                       \
            hipLaunchKernelGGL((dequant_kernel<L, C, HEAL_DQ_F32>), dim3(grid_for(rows, RowTiling<L, C>::ROWS)), dim3(256), \
                               0, s, codes, rows, (int)D, ldq, scales, out, out_lo, ldo);             \
        else                                                                                          \
            hipLaunchKernelGGL((dequant_kernel<L, C, HEAL_DQ_F16X2>), dim3(grid_for(rows, RowTiling<L, C>::ROWS)), \
                               dim3(256), 0, s, codes, rows, (int)D, ldq, scales, out, out_lo, ldo);  \
        return hipGetLastError();                                                                     \
    }

hipError_t launch_dequant(const int16_t* codes, int64_t rows, int64_t D, int64_t ldq,
                          const float* scales, int fmt, void* out, void* out_lo, int64_t ldo,
                          hipStream_t s) {
    if (rows == 0) return hipSuccess;
    int lpr, nch;
    row_shape(D, lpr, nch);
    HEAL_DQ_CASE(1, 1) HEAL_DQ_CASE(2, 1) HEAL_DQ_CASE(4, 1) HEAL_DQ_CASE(8, 1) HEAL_DQ_CASE(16, 1)
    HEAL_DQ_CASE(32, 1) HEAL_DQ_CASE(64, 1) HEAL_DQ_CASE(64, 2) HEAL_DQ_CASE(64, 4)
    HEAL_DQ_CASE(64, 8) HEAL_DQ_CASE(64, 16)
    return hipErrorInvalidValue;
}
#undef HEAL_DQ_CASE

}  // namespace heal
