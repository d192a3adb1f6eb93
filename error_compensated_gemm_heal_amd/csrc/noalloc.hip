// heal_gemm_f32c_noalloc: the decode-path compensated GEMM for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its kernels are heal_gemm_f32c's; their
// scratch memory (split-K counters, split activation blocks, split-K
// partials) lives in a file-scope device array that the library owns, one
// copy per GPU, held until the process ends.  Nothing here allocates.
//
// The array's name is a host-side stand-in on the host: its device address
// is looked up once per device, with that device current, by
// hipGetSymbolAddress, and only that address is handed to kernels.
//
// The split-K completion uses the counter form: the array's first 64 KiB
// hold one counter per workgroup row group, zero when the process starts
// and put back to zero by the workgroup that counts last, so every call
// finds them zero, including the replays of a captured graph (a per-call
// epoch would be frozen into the graph).  Everything else in the array is
// written before it is read within a call.  Calls that overlap on one GPU
// (different streams, or threads) share the array and race.
#include <mutex>

#include "heal_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;   // 16 MiB per GPU
constexpr size_t kCounterBytes = (size_t)64 << 10;   // its first 64 KiB: split-K counters
constexpr int64_t kMaxRowGroups = kCounterBytes / 8;  // one per 64 rows of W at most
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
    if ((N + 63) / 64 > kMaxRowGroups) return HEAL_ERR_UNSUPPORTED;     // a counter per 64 rows of W
    if (heal_gemm_f32c_workspace(M, N, K, flags) > kScratchBytes - kCounterBytes) return HEAL_ERR_WORKSPACE;
    if (M == 0 || N == 0) return HEAL_OK;
    void* base = nullptr;
    if (scratch_address(&base) != hipSuccess) return HEAL_ERR_HIP;
    unsigned char* p = static_cast<unsigned char*>(base);
    return heal::gemm_f32c_counters(A, lda, W, ldw, C, ldc, M, N, K, flags, a_kshift, p + kCounterBytes,
                                    kScratchBytes - kCounterBytes, reinterpret_cast<unsigned long long*>(p),
                                    dev_status, stream);
}
