// Decode-shaped FP32-accurate GEMM (M <= 64) on gfx950 16-bit MFMA.
//
// Same arithmetic as the prefill kernel (HEAL paper, section 3, "Mitigating
// GEMM Truncation via FP16 Promotion and Algebraic Compensation"):
//     C = A_hi.B_hi + 2^-10 (A_hi.B_lo + A_lo.B_hi),  fp32 accumulation,
// but shaped for a skinny activation.  The weight dominates the traffic, so:
//  * W is read once from HBM as fp32 [N, K] (4 bytes per element, the same
//    bytes as its two fp16 parts) and split into hi/lo in registers;
//  * the activation block (<= 64 rows x 256 k) is split once per workgroup
//    into LDS, stored in MFMA fragment order so every lane's read is one
//    conflict-free 16-byte access;
//  * v_mfma_f32_16x16x32_f16 with the activation as the 16-row operand and W
//    as the 16-column operand, so output columns are consecutive lanes;
//  * inside each 32-wide k step, lane group g (lanes 16g..16g+15) carries
//    k = 4g..4g+3 and 16+4g..16+4g+3: any k order is valid as long as both
//    operands use it, and this one makes each W load a 64-byte run per row;
//  * W for the next 8 k steps is in flight while the current 8 are used;
//  * split-K: the k range is cut into chunks chosen from (N, K) only, and
//    chunk partials are summed in chunk order by a second kernel.  The
//    summation order of an output therefore does not depend on M: a
//    decode-sized product does not change with the batch it is computed in.
#include "heal_internal.h"

namespace heal {

namespace {

constexpr int KA = 256;             // k block of activations staged in LDS
constexpr int STEPS = KA / 32;      // k32 steps per block
constexpr int ROWS_PER_WAVE = 16;
constexpr int DEC_ROWS = 4 * ROWS_PER_WAVE;   // W rows (outputs) per workgroup

__device__ __forceinline__ void mfma16(const half8& a, const half8& b, floatx4& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Load this lane's 8 W values of one k32 step (k = k0 + 4g..+3 and k0 + 16 + 4g..+3).
template <bool VEC>
__device__ __forceinline__ void load_w(const float* __restrict__ wrow, bool row_ok, int64_t k0, int g,
                                       int64_t K, float4& lo4, float4& hi4) {
    const int64_t ka = k0 + 4 * g, kb = k0 + 16 + 4 * g;
    if (VEC && row_ok && k0 + 32 <= K) {
        lo4 = *reinterpret_cast<const float4*>(wrow + ka);
        hi4 = *reinterpret_cast<const float4*>(wrow + kb);
    } else {
        float t[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            t[j] = (row_ok && ka + j < K) ? wrow[ka + j] : 0.f;
            t[4 + j] = (row_ok && kb + j < K) ? wrow[kb + j] : 0.f;
        }
        lo4 = make_float4(t[0], t[1], t[2], t[3]);
        hi4 = make_float4(t[4], t[5], t[6], t[7]);
    }
}

__device__ __forceinline__ void split8(const float4& a, const float4& b, half8& h, half8& l) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        _Float16 hh, ll;
        split_one(v[j], hh, ll);
        h[j] = hh;
        l[j] = ll;
    }
}

template <int MT, bool VEC>
__global__ __launch_bounds__(256) void gemm_decode_kernel(const float* __restrict__ A, int64_t lda,
                                                          const float* __restrict__ W, int64_t ldw,
                                                          float* __restrict__ out, int64_t ldo,
                                                          int64_t split_stride, int M, int N, int K,
                                                          int kchunk, uint32_t* __restrict__ status) {
    constexpr int MP = MT * 16;                  // padded activation rows
    constexpr int PLANE = STEPS * 4 * MP * 16;   // bytes per hi or lo plane of one k block
    __shared__ __attribute__((aligned(16))) unsigned char sa[2 * PLANE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4;
    const int n = blockIdx.x * DEC_ROWS + wave * ROWS_PER_WAVE + (lane & 15);
    const bool row_ok = n < N;
    const float* wrow = W + (int64_t)(row_ok ? n : 0) * ldw;
    const int split = blockIdx.y;
    const int64_t k_begin = (int64_t)split * kchunk;
    const int64_t k_end = std::min<int64_t>(k_begin + kchunk, K);
    const int nsteps = (int)((k_end - k_begin + 31) / 32);
    const int nblocks = (nsteps + STEPS - 1) / STEPS;

    floatx4 acc_hh[MT], acc_c[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) { acc_hh[t][e] = 0.f; acc_c[t][e] = 0.f; }

    float4 wa[STEPS], wb[STEPS];
    bool bad = false;
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
        if (s < nsteps) load_w<VEC>(wrow, row_ok, k_begin + 32 * s, g, K, wa[s], wb[s]);

    for (int blk = 0; blk < nblocks; ++blk) {
        const int64_t kb0 = k_begin + (int64_t)blk * KA;
        // ---- stage the activation block: split into fragment-ordered LDS ----
        __syncthreads();
#pragma unroll
        for (int i = 0; i < MP * (KA / 4) / 256; ++i) {
            const int f = tid + 256 * i;
            const int m = f / (KA / 4);
            const int kk = (f % (KA / 4)) * 4;      // k offset inside the block
            const int64_t k = kb0 + kk;
            float x[4] = {0.f, 0.f, 0.f, 0.f};
            if (m < M) {
                const float* ap = A + (int64_t)m * lda + k;
                if (VEC && k + 4 <= k_end) {
                    const float4 v = *reinterpret_cast<const float4*>(ap);
                    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (k + j < k_end) x[j] = ap[j];
                }
            }
            uint16_t h[4], l[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                _Float16 hh, ll;
                split_one(x[j], hh, ll);
                bad |= f16_out_of_range(x[j]);
                h[j] = f16_bits(hh);
                l[j] = f16_bits(ll);
            }
            const int kb = kk >> 5, kw = kk & 31;
            const int half_sel = kw >> 4, grp = (kw & 15) >> 2;
            const int off = ((kb * 4 + grp) * MP + m) * 16 + half_sel * 8;
            *reinterpret_cast<uint2*>(sa + off) =
                make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
            *reinterpret_cast<uint2*>(sa + PLANE + off) =
                make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
        }
        __syncthreads();

        // ---- 8 k32 steps: consume W in registers, prefetch the next block ----
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int step = blk * STEPS + s;
            if (step < nsteps) {
                half8 wh, wl;
                split8(wa[s], wb[s], wh, wl);
                bad |= f16_out_of_range4(wa[s]) || f16_out_of_range4(wb[s]);
                const int nxt = step + STEPS;
                if (nxt < nsteps) load_w<VEC>(wrow, row_ok, k_begin + 32 * (int64_t)nxt, g, K, wa[s], wb[s]);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const int off = ((s * 4 + g) * MP + t * 16 + (lane & 15)) * 16;
                    const half8 ah = *reinterpret_cast<const half8*>(sa + off);
                    const half8 al = *reinterpret_cast<const half8*>(sa + PLANE + off);
                    mfma16(ah, wh, acc_hh[t]);
                    mfma16(ah, wl, acc_c[t]);
                    mfma16(al, wh, acc_c[t]);
                }
            }
        }
    }
    if (bad && status) atomicOr(status, (uint32_t)HEAL_FLAG_F16_RANGE);

    // ---- epilogue: lane holds column n, rows t*16 + 4g + e ------------------
    if (!row_ok) return;
    float* o = out + split * split_stride;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = t * 16 + 4 * g + e;
            if (m < M) o[(int64_t)m * ldo + n] = acc_hh[t][e] + acc_c[t][e] * 0.0009765625f;
        }
}

// C[m, n] = sum over chunks s (in order) of P[s, m, n].
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, int splits,
                                                            int64_t M, int64_t N, float* __restrict__ C,
                                                            int64_t ldc) {
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        float acc = P[i];
        for (int s = 1; s < splits; ++s) acc += P[s * total + i];
        const int64_t m = i / N, n = i - m * N;
        C[m * ldc + n] = acc;
    }
}

}  // namespace

DecodePlan decode_plan(int64_t M, int64_t N, int64_t K) {
    DecodePlan p{};
    const int64_t nblk = (N + DEC_ROWS - 1) / DEC_ROWS;
    const int64_t kblocks = std::max<int64_t>(1, (K + KA - 1) / KA);
    int64_t want = std::max<int64_t>(1, (512 + nblk - 1) / std::max<int64_t>(nblk, 1));
    want = std::min(want, kblocks);
    const int64_t per = (K + want - 1) / want;
    p.kchunk = std::max<int64_t>(KA, (per + KA - 1) / KA * KA);
    p.splits = (int)std::max<int64_t>(1, (K + p.kchunk - 1) / p.kchunk);
    p.a_bytes = 0;
    p.p_bytes = p.splits > 1 ? (p.splits * M * N * 4 + 255) / 256 * 256 : 0;
    return p;
}

hipError_t launch_gemm_decode(const float* A, int64_t lda, const float* W, int64_t ldw, float* C,
                              int64_t ldc, int64_t M, int64_t N, int64_t K, void* workspace,
                              const DecodePlan& plan, uint32_t* status, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    if (M > 64 || K == 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((N + DEC_ROWS - 1) / DEC_ROWS), (unsigned)plan.splits);
    float* out = plan.splits > 1 ? static_cast<float*>(workspace) : C;
    const int64_t ldo = plan.splits > 1 ? N : ldc;
    const int64_t stride = plan.splits > 1 ? M * N : 0;
    // 16-byte vector loads need 16-byte aligned rows of both operands
    const bool vec = ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(W)) & 15) == 0 &&
                     ((lda | ldw) & 3) == 0;
#define HEAL_DEC(MT_)                                                                                    \
    if (vec)                                                                                             \
        hipLaunchKernelGGL((gemm_decode_kernel<MT_, true>), grid, dim3(256), 0, s, A, lda, W, ldw, out, \
                           ldo, stride, (int)M, (int)N, (int)K, (int)plan.kchunk, status);               \
    else                                                                                                 \
        hipLaunchKernelGGL((gemm_decode_kernel<MT_, false>), grid, dim3(256), 0, s, A, lda, W, ldw, out, \
                           ldo, stride, (int)M, (int)N, (int)K, (int)plan.kchunk, status)
    if (M <= 16) {
        HEAL_DEC(1);
    } else if (M <= 32) {
        HEAL_DEC(2);
    } else {
        HEAL_DEC(4);
    }
#undef HEAL_DEC
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    const int64_t total = M * N;
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 256 * 16);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const float*>(workspace), plan.splits, M, N, C, ldc);
    return hipGetLastError();
}

}  // namespace heal
