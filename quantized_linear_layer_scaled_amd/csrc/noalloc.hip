// gemm_fp8_scaled_noalloc: the FP8 GEMM entry point for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  It takes no workspace: the Split-K
// partial sums go to a static device array, `scratch`, of kScratchBytes per
// GPU, which the code object holds on every device the library runs on until
// the process ends.  Nothing here calls hipMalloc, hipFree or any allocating
// routine.
//
// The host may not use the array's name as a device address (in host code it
// names a host-side stand-in): its address on each device is looked up once,
// with that device current, by hipGetSymbolAddress -- at qll_init for the
// device current then, else at the first call on a device -- and kept per
// device; the kernels receive that pointer as their workspace.
//
// The Split-K partials need no clearing: the first stage writes every element
// of every piece before the second stage reads it.  All calls on one GPU share
// its array, so calls that overlap on one GPU (two streams, two threads) race
// and must be serialized by the caller.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/qll.h"
#include "qll_internal.h"

namespace qll {

int gemm_plan(int op, int64_t M, int64_t N, int64_t K, qll_cfg* cfg, uint64_t* ws_need);
int gemm_run(int op, const void* A, const void* B, const float* sa, const float* sb,
             void* out, int out_dtype, int64_t M, int64_t N, int64_t K, void* ws,
             size_t ws_bytes, void* stream, const qll_cfg* cfg);
int gemm_validate(int op, const void* A, const void* B, const float* sa, const float* sb,
                  const void* out, int out_dtype, int64_t M, int64_t N, int64_t K);

namespace {

constexpr size_t kScratchBytes = (size_t)QLL_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_setup;

// The array's address on the current device (looked up once per device).
hipError_t scratch_on_current(void** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_setup);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return e != hipSuccess ? e : hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace

hipError_t noalloc_setup()
{
    void* p = nullptr;
    return scratch_on_current(&p);
}

}  // namespace qll

extern "C" int gemm_fp8_scaled_noalloc(const void* A, const void* B, const float* sa,
                                       const float* sb, void* out, int out_dtype, int64_t M,
                                       int64_t N, int64_t K, void* stream)
{
    using namespace qll;
    int rc = gemm_validate(OP_FP8, A, B, sa, sb, out, out_dtype, M, N, K);
    if (rc != QLL_OK || M == 0)
        return rc;
    qll_cfg cfg;
    uint64_t need = 0;
    gemm_plan(OP_FP8, M, N, K, &cfg, &need);
    if (need > kScratchBytes)
        return QLL_ERR_WORKSPACE;  // more Split-K partials than the array holds
    void* ws = nullptr;
    if (need > 0 && scratch_on_current(&ws) != hipSuccess) {
        (void)hipGetLastError();
        return QLL_ERR_HIP;
    }
    return gemm_run(OP_FP8, A, B, sa, sb, out, out_dtype, M, N, K, ws,
                    need > 0 ? kScratchBytes : 0, stream, &cfg);
}
