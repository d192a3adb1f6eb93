// Roofline calibration kernels (measurement only, not part of the method):
// the chip's sustained 16-bit MFMA rate and HBM read rate, measured in the
// launch shapes of the kernels they are the ceilings of.
//  * calib_mfma_kernel: a register-only loop of v_mfma_f32_32x32x16_f16 in the
//    prefill GEMM's shape: one workgroup of 4 waves per compute unit, each
//    wave 16 independent 32 x 32 accumulators (the GEMM's 4 x 4 wave tile),
//    issued back to back; the A operand's bits change every round, so the
//    matrix cores switch data as they do on real operands.  No LDS and no
//    memory traffic: what it reaches is the ceiling under the clock the MFMA
//    load sustains.
//  * calib_read_kernel: a streaming read of a buffer, 16 bytes per lane with
//    eight non-temporal loads in flight, reduced to one value per thread so
//    nothing is optimized away: the HBM read ceiling of a streaming kernel.
#include "heal_internal.h"

namespace heal {

namespace {

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void calib_mfma_kernel(int64_t iters, float* __restrict__ out) {
    const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 2654435761u;
    u32x4 ab, bb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // fp16 pairs in [1, 2): exponent 15, random fraction bits
        ab[j] = 0x3C003C00u | ((seed >> j) & 0x03FF03FFu);
        bb[j] = 0x3C003C00u | ((seed >> (j + 5)) & 0x03FF03FFu);
    }
    const half8 b = __builtin_bit_cast(half8, bb);
    floatx16 acc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
        const half8 a = __builtin_bit_cast(half8, ab);
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[t], 0, 0, 0);
        ab ^= (u32x4){0x00550055u, 0x00AA00AAu, 0x01330133u, 0x02CC02CCu};   // fraction bits only
    }
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[t][e];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void calib_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                         float* __restrict__ out) {
    constexpr int U = 8;   // 16-byte loads in flight per thread
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= (v[u][0] ^ v[u][1]) + (v[u][2] ^ v[u][3]);
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= (v[0] ^ v[1]) + (v[2] ^ v[3]);
    }
    out[blockIdx.x * 256 + threadIdx.x] = (float)acc;
}

}  // namespace

}  // namespace heal

extern "C" {

heal_status heal_calib_mfma_f16(int64_t iters, int64_t workgroups, float* out, void* stream) {
    if (iters < 0 || workgroups < 0 || workgroups > ((int64_t)1 << 20)) return HEAL_ERR_SHAPE;
    if (iters == 0 || workgroups == 0) return HEAL_OK;
    if (!out) return HEAL_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(out) & 3) != 0) return HEAL_ERR_ALIGN;
    hipLaunchKernelGGL(heal::calib_mfma_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                       static_cast<hipStream_t>(stream), iters, out);
    return hipGetLastError() == hipSuccess ? HEAL_OK : HEAL_ERR_HIP;
}

heal_status heal_calib_read(const void* buf, int64_t bytes, int64_t workgroups, float* out, void* stream) {
    if (bytes < 0 || workgroups < 0 || workgroups > ((int64_t)1 << 20)) return HEAL_ERR_SHAPE;
    if (bytes == 0 || workgroups == 0) return HEAL_OK;
    if (!buf || !out) return HEAL_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0 || (bytes & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(out) & 3) != 0)
        return HEAL_ERR_ALIGN;
    hipLaunchKernelGGL(heal::calib_read_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const heal::u32x4*>(buf), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? HEAL_OK : HEAL_ERR_HIP;
}

}  // extern "C"
