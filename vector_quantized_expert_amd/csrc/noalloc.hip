// noalloc.hip -- the library's static device scratch, for the entry point that
// allocates nothing (rvq_moe_layer_forward_noalloc).
//
// Callers that cannot allocate device memory while they run (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc) get a
// layer call whose scratch -- the gate/up partial sums and the inter-workgroup
// completion counters of the table-path kernel -- lives in one file-scope
// device array instead of a handle's workspace.  Each GPU the library runs on
// holds its own copy of the array until the process ends; its device address
// is looked up once per device (at rvq_moe_open) and only that address is
// handed to kernels and fills.  Every call on a GPU shares that GPU's array:
// calls that overlap in time on one GPU race.
#include <mutex>

#include "internal.hpp"

namespace rvq {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
char *g_ptr[kMaxDevices];  // device address of `scratch` on each device (null until set up)
}  // namespace

hipError_t static_scratch_setup(int device) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[device]) return hipSuccess;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;  // the caller makes `device` current
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[device] = static_cast<char *>(p);
    return hipSuccess;
}

char *static_scratch(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    return g_ptr[device];
}

// Zero n ints at p (a plain kernel, so that a captured call records no memset node).
__global__ __launch_bounds__(256) void k_zero_ints(int *__restrict__ p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

hipError_t launch_zero_ints(int *p, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int blocks = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
    hipLaunchKernelGGL(k_zero_ints, dim3(blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace rvq
