// bra_noalloc.hip -- the device scratch array behind bra_forward_noalloc, the
// forward for callers that cannot allocate (code under HIP graph capture,
// serving loops, harnesses that forbid hipMalloc): the workspace that
// bra_create allocates for a handle is carved out of this fixed array
// instead.  Each device the library runs on holds its own copy of the array
// until the process ends; calls that overlap on one device share it and
// race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bra_launch.h"

namespace bra {
namespace {

constexpr size_t kScratchBytes = size_t{16} << 20;  // 16 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // the array's device address, per device

__global__ void zero_fill_kernel(float* __restrict__ p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

}  // namespace

size_t scratch_bytes() { return kScratchBytes; }

// The device address of `scratch` on `device`, which must be the current
// device: looked up once per device with hipGetSymbolAddress (the array's
// name is only a host-side stand-in), then cached.
hipError_t scratch_pointer(int device, void** ptr) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}

// Clears n floats with a kernel (not a memset node: the call may be captured
// in a graph).
hipError_t launch_zero_fill(float* p, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace bra
