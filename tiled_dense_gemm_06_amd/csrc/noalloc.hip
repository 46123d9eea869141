// tlg_gemm_relu_noalloc: C = ReLU(A . B) without a handle and without any
// allocation, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The split kernels' workspace (their counters and fp32 partials) is the
// file-scope device array `scratch` below, of a fixed size. Each GPU the
// library runs on holds its own copy of it from the code object's load
// until the process ends. In host code the array's name only stands in for
// the symbol: its device address is taken once per device with
// hipGetSymbolAddress and kept per device, and only that address is handed
// to kernels.
//
// Every call on a GPU shares that GPU's array. Calls on one GPU that may run
// at the same time (on different streams, or from different threads without
// ordering) race on it; callers must order them. The counter area is cleared
// by a kernel on the call's stream before every split kernel that uses it;
// the partials are always written before they are read within a call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kernels.h"
#include "tlg.h"

namespace {

// 64 KiB of counters followed by 8 MiB of fp32 partials.
constexpr int64_t kScratchBytes = tlg::kCounterBytes + (8ll << 20);
static_assert(kScratchBytes == TLG_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    bool ready = false;
    bool supported = false;
    int cus = 0;
    float *ptr = nullptr;  // device address of `scratch` on this device
};
DeviceScratch g_dev[kMaxDevices];
std::mutex g_mutex;

// Set-up of the current device `dev` on its first call: the architecture
// check, the compute-unit count for the planner, and the device address of
// `scratch` (each device has its own). Allocates nothing.
tlg_status device_setup(int dev, DeviceScratch **out) {
    if (dev < 0 || dev >= kMaxDevices) return TLG_ERROR_NOT_SUPPORTED;
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceScratch &d = g_dev[dev];
    if (!d.ready) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TLG_ERROR_HIP;
        d.supported = tlg_arch_supported(prop.gcnArchName) != 0;
        if (d.supported) {
            void *p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
                (void)hipGetLastError();
                return TLG_ERROR_HIP;
            }
            d.ptr = (float *)p;
            d.cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
        }
        d.ready = true;
    }
    if (!d.supported) return TLG_ERROR_NOT_SUPPORTED;
    *out = &d;
    return TLG_SUCCESS;
}

__global__ void k_clear_words(int *p, int64_t words) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) p[i] = 0;
}

}  // namespace

namespace tlg {

hipError_t launch_clear_words(int *p, int64_t words, hipStream_t stream) {
    if (words <= 0) return hipSuccess;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(k_clear_words, dim3((unsigned)blocks), dim3(256), 0, stream, p, words);
    return hipGetLastError();
}

}  // namespace tlg

extern "C" tlg_status tlg_gemm_relu_noalloc(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                                            const void *B, int64_t ldb, void *C, int64_t ldc, hipStream_t stream) {
    try {
        tlg_status st = tlg_check_args(M, N, K, A, lda, B, ldb, C, ldc);
        if (st != TLG_SUCCESS) return st;
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess) return TLG_ERROR_HIP;
        DeviceScratch *d = nullptr;
        st = device_setup(dev, &d);
        if (st != TLG_SUCCESS) return st;
        return tlg::run_with_workspace(d->ptr, kScratchBytes, d->cus, true, TLG_VARIANT_AUTO, -1, 0,
                                       tlg::make_problem_c(M, N, K, A, lda, B, ldb, C, ldc), stream);
    } catch (...) {
        return TLG_ERROR_HIP;
    }
}

extern "C" int64_t tlg_noalloc_scratch_bytes(void) { return kScratchBytes; }
