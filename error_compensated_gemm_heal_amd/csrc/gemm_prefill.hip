// Prefill-shaped FP32-accurate GEMM on gfx950 16-bit MFMA.
//
// HEAL paper, section 3, "Mitigating GEMM Truncation via FP16 Promotion and
// Algebraic Compensation": each FP32 operand is written as an FP16 value
// plus an FP16 residual shifted by 2^10, and the product is expanded into
// 16-bit products with FP32 accumulation.  With both operands in FP32 the
// expansion keeps three products:
//     C = A_hi.B_hi + 2^-10 (A_hi.B_lo + A_lo.B_hi)
// (the lo.lo term is 2^-20 of the result and is dropped).
//
// Kernel structure (MFMA-bound; 3 x 2MNK flops on the 16-bit pipe):
//  * operands arrive packed by the split kernels: per row, each 32-wide k
//    block is one 128-byte line [32 hi | 32 lo] fp16, zero-padded to whole
//    tiles, so the main loop has no bounds checks;
//  * block tile 256 (M) x 128 (N) x 32 (K), 4 waves in a 2 x 2 grid of
//    128 x 64 wave tiles, each made of 4 x 2 tiles of v_mfma_f32_32x32x16_f16;
//  * two fp32 accumulator sets per wave tile (hi.hi and the correction sum),
//    256 registers, combined once in the epilogue: C = hh + c * 2^-10;
//  * k tiles staged global -> registers -> LDS with two LDS buffers (one
//    barrier per k tile); LDS rows padded to 80 bytes so the 16-byte fragment
//    reads of 16 consecutive rows hit distinct banks;
//  * block -> tile order keeps the blocks that share a B tile on one XCD
//    (blocks are dealt to the 8 XCDs round-robin), so B is read from HBM once
//    and re-served from that XCD's L2.
#include "heal_internal.h"

namespace heal {

namespace {

constexpr int BM = 256, BN = 128, BK = 32;
constexpr int WM = 128, WN = 64;            // wave tile
constexpr int TM = WM / 32, TN = WN / 32;   // 32x32 MFMA tiles per wave
constexpr int ROWB = 80;                    // LDS bytes per row per plane (64 data + 16 pad)
constexpr int A_PLANE = BM * ROWB;          // bytes
constexpr int B_PLANE = BN * ROWB;
constexpr int STAGE = 2 * A_PLANE + 2 * B_PLANE;   // 61440
constexpr int A_CHUNKS = BM * 8 / 256;     // 16-byte global chunks per thread per k tile (A)
constexpr int B_CHUNKS = BN * 8 / 256;     // (B)

__device__ __forceinline__ void mfma32(const half8& a, const half8& b, floatx16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_prefill_kernel(const uint4* __restrict__ Apk, const uint4* __restrict__ Bpk,
                         float* __restrict__ C, int64_t ldc, int M, int N, int Kp,
                         int tiles_m, int tiles_n) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    // ---- XCD-aware tile order -------------------------------------------
    const int nblk = tiles_m * tiles_n;
    int bid = blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int tm = bid % tiles_m;
    const int tn = bid / tiles_m;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    // Packed row stride in 16-byte chunks: Kp fp16 hi + Kp fp16 lo = Kp*4 bytes.
    const int64_t row_chunks = (int64_t)Kp / 4;
    const int nkt = Kp / BK;

    // ---- global -> register staging (one k tile) ---------------------------
    // chunk c = tid + 256 i of a tile: row c / 8 (= tid / 8 + 32 i), piece c % 8
    // (0..3 hi, 4..7 lo, 16 bytes each).  Chunk i sits 32 i rows below chunk 0,
    // so one base pointer per operand plus uniform offsets addresses them all.
    const int r0 = tid >> 3, p0 = tid & 7;
    const uint4* a_src = Apk + ((int64_t)tm * BM + r0) * row_chunks + p0;
    const uint4* b_src = Bpk + ((int64_t)tn * BN + r0) * row_chunks + p0;
    const int a_dst = (p0 >> 2) * A_PLANE + r0 * ROWB + (p0 & 3) * 16;
    const int b_dst = 2 * A_PLANE + (p0 >> 2) * B_PLANE + r0 * ROWB + (p0 & 3) * 16;
    const int64_t rows32 = 32 * row_chunks;
    u32x4 ra[A_CHUNKS], rb[B_CHUNKS];
#define HEAL_GLOAD(kt)                                                                         \
    do {                                                                                       \
        const u32x4* pa = reinterpret_cast<const u32x4*>(a_src + (kt) * 8);                    \
        const u32x4* pb = reinterpret_cast<const u32x4*>(b_src + (kt) * 8);                    \
        _Pragma("unroll") for (int i = 0; i < A_CHUNKS; ++i) ra[i] = pa[i * rows32];           \
        _Pragma("unroll") for (int i = 0; i < B_CHUNKS; ++i) rb[i] = pb[i * rows32];           \
    } while (0)
#define HEAL_SWRITE(buf)                                                                       \
    do {                                                                                       \
        unsigned char* base_ = smem + (buf) * STAGE;                                           \
        _Pragma("unroll") for (int i = 0; i < A_CHUNKS; ++i)                                   \
            *reinterpret_cast<u32x4*>(base_ + a_dst + i * 32 * ROWB) = ra[i];                  \
        _Pragma("unroll") for (int i = 0; i < B_CHUNKS; ++i)                                   \
            *reinterpret_cast<u32x4*>(base_ + b_dst + i * 32 * ROWB) = rb[i];                  \
    } while (0)

    floatx16 acc_hh[TM][TN], acc_c[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) { acc_hh[i][j][e] = 0.f; acc_c[i][j][e] = 0.f; }

    // fragment read offsets: lane reads row (l % 32) of a 32-row tile, k half (l / 32)
    const int frag_off = (lane & 31) * ROWB + (lane >> 5) * 16;
    const int a_frag = wm * WM * ROWB + frag_off;
    const int b_frag = 2 * A_PLANE + wn * WN * ROWB + frag_off;

    HEAL_GLOAD(0);
    HEAL_SWRITE(0);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nkt) HEAL_GLOAD(kt + 1);
        const unsigned char* base = smem + buf * STAGE;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {           // two k16 steps per k tile
            half8 ah[TM], al[TM], bh[TN], bl[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                ah[i] = *reinterpret_cast<const half8*>(base + a_frag + i * 32 * ROWB + ks * 32);
                al[i] = *reinterpret_cast<const half8*>(base + a_frag + A_PLANE + i * 32 * ROWB + ks * 32);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                bh[j] = *reinterpret_cast<const half8*>(base + b_frag + j * 32 * ROWB + ks * 32);
                bl[j] = *reinterpret_cast<const half8*>(base + b_frag + B_PLANE + j * 32 * ROWB + ks * 32);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    mfma32(ah[i], bh[j], acc_hh[i][j]);
                    mfma32(ah[i], bl[j], acc_c[i][j]);
                }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) mfma32(al[i], bh[j], acc_c[i][j]);
        }
        if (kt + 1 < nkt) HEAL_SWRITE(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: one fp32 combination, bounds-checked store ---------------
    const int row0 = tm * BM + wm * WM + (lane >> 5) * 4;
    const int col0 = tn * BN + wn * WN + (lane & 31);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = col0 + j * 32;
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = row0 + i * 32 + (e >> 2) * 8 + (e & 3);
                if (row < M) C[(int64_t)row * ldc + col] = acc_hh[i][j][e] + acc_c[i][j][e] * 0.0009765625f;
            }
        }
#undef HEAL_GLOAD
#undef HEAL_SWRITE
}

}  // namespace

hipError_t launch_gemm_prefill(const void* Apk, const void* Bpk, float* C, int64_t ldc, int64_t M,
                               int64_t N, int64_t K, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    const int64_t Kp = pack_kp(K);
    if (Kp == 0) return hipErrorInvalidValue;  // K == 0 is handled by the caller
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    static bool attr_set = false;  // idempotent; racing first calls set the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_prefill_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 2 * STAGE);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(gemm_prefill_kernel, dim3(tiles_m * tiles_n), dim3(256), 2 * STAGE, s,
                       static_cast<const uint4*>(Apk), static_cast<const uint4*>(Bpk), C, ldc, (int)M,
                       (int)N, (int)Kp, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace heal
