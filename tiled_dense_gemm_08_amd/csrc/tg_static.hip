// tg_static.hip — tg_gemm_ws_static: tg_gemm_ws with a workspace the library
// holds in a file-scope device array instead of one the caller passes, for
// callers that cannot allocate device memory at all (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).  Each GPU
// the library runs on holds its own copy of the array until the process ends.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tg.h"

namespace {

// The workspace of every tg_gemm_ws_static call on a device.  Its name is a
// host-side stand-in in host code: kernels get the device address from
// hipGetSymbolAddress below, never the name itself.
static __device__ __align__(256) char scratch[TG_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device (guarded by g_mu)

// The address of `scratch` on the current device, looked up once per device
// with that device current; nullptr if the runtime cannot resolve it.
void *scratch_address(int dev)
{
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" tg_status tg_gemm_ws_static(int config_id, int splits, tg_op op_a, tg_op op_b,
                                       const void *A, const void *B, const float *bias, void *C,
                                       int64_t M, int64_t N, int64_t K, int64_t lda,
                                       int64_t ldb, int64_t ldc, tg_dtype c_dtype,
                                       hipStream_t stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return TG_ERROR_UNSUPPORTED;
    }
    void *ws = scratch_address(dev);
    if (ws == nullptr)
        return TG_ERROR_LAUNCH;
    return tg_gemm_ws(config_id, splits, op_a, op_b, A, B, bias, C, M, N, K, lda, ldb, ldc,
                      c_dtype, ws, TG_STATIC_SCRATCH_BYTES, stream);
}
