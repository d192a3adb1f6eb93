// heal_gemm_f32c_noalloc: the decode-path compensated GEMM for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its kernels are heal_gemm_f32c's; their
// scratch memory (split-K flags, split activation blocks, split-K partials)
// lives in a file-scope device array that the library owns, one copy per GPU,
// held until the process ends.  Nothing here allocates.
//
// The array's name is a host-side stand-in on the host: its device address
// is looked up once per device, with that device current, by
// hipGetSymbolAddress, and only that address is handed to kernels.
//
// Nothing in the array needs clearing between calls: the split-K flags are
// compared against a per-call epoch that no earlier call used (the array
// starts zeroed and epochs are never 0), and every partial or split block
// is written before it is read within a call.  Calls that overlap on one GPU
// (different streams, or threads) share the array and race.
#include <mutex>

#include "heal_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;   // 16 MiB per GPU
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The device address of the current device's copy of the array.
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [dev]() {
        void* p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = p;
    });
    if (g_err[dev] != hipSuccess) return g_err[dev];
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" heal_status heal_gemm_f32c_noalloc(const float* A, int64_t lda, const void* W, int64_t ldw, float* C,
                                              int64_t ldc, int64_t M, int64_t N, int64_t K, uint32_t flags,
                                              const int8_t* a_kshift, uint32_t* dev_status, void* stream) {
    if (M < 0 || N < 0 || K < 0 || M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31))
        return HEAL_ERR_SHAPE;
    if (!heal::decode_path(M, K, flags)) return HEAL_ERR_UNSUPPORTED;   // M <= 64, [N, K] or packed W, A unpacked
    if (heal_gemm_f32c_workspace(M, N, K, flags) > kScratchBytes) return HEAL_ERR_WORKSPACE;
    if (M == 0 || N == 0) return HEAL_OK;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return HEAL_ERR_HIP;
    return heal_gemm_f32c(A, lda, W, ldw, C, ldc, M, N, K, flags, a_kshift, ws, kScratchBytes, dev_status, stream);
}
