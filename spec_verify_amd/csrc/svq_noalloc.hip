// svq_w4a16_gemm for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation):
// the cross-workgroup reductions use a file-scope device array of
// SVQ_NOALLOC_SCRATCH_BYTES instead of a caller-provided workspace.
//
// Each device the library runs on holds its own copy of the array until the
// process ends. In host code the array's name only stands for it: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and that address is what the kernels receive. The array starts
// zero-filled (the loader clears it, and the first call on a device clears the
// counter region once more with a fill kernel on the caller's stream); every
// kernel leaves its counters at zero, and the partials are overwritten before
// they are read. Calls on one device share the array: calls that overlap in
// time on one device race.
#include "../../include/svq.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "svq_launch.h"

namespace svq {
namespace {

constexpr size_t kScratchBytes = SVQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes >= kCounterBytes && kScratchBytes % 256 == 0, "scratch holds the counters");
constexpr int kMaxScratchDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4 *__restrict__ p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        p[i] = make_uint4(0, 0, 0, 0);
}

std::mutex g_mu;
struct DeviceScratch {
    void *ptr;     // device address of `scratch` on this device (null: not looked up yet)
    bool cleared;  // the counter region has been cleared once
};
DeviceScratch g_scratch[kMaxScratchDevices];

// This device's address of the scratch array: looked up once, with the device
// current (a query; nothing is launched or allocated).
int scratch_address(void **out, int *dev_out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return SVQ_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev].ptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SVQ_ERR_HIP;
        g_scratch[dev].ptr = p;
    }
    *out = g_scratch[dev].ptr;
    *dev_out = dev;
    return SVQ_OK;
}

// First call on a device: one fill kernel on the caller's stream clears the
// counter region (the loader's zero fill already did; this does not rely on it).
int clear_once(int dev, void *p, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev].cleared) return SVQ_OK;
    hipLaunchKernelGGL(scratch_clear_kernel, dim3(64), dim3(256), 0, stream, (uint4 *)p, kCounterBytes / 16);
    if (hipGetLastError() != hipSuccess) return SVQ_ERR_HIP;
    g_scratch[dev].cleared = true;
    return SVQ_OK;
}

}  // namespace
}  // namespace svq

using namespace svq;

extern "C" int svq_w4a16_gemm_noalloc(const void *x, const int32_t *qweight_tiled, const void *scales,
                                      void *out, int64_t M, int64_t N, int64_t K, int32_t group_size,
                                      void *stream) {
    const size_t need = svq_w4a16_workspace_bytes(SVQ_KERNEL_AUTO, M, N, K, group_size);
    if (need == (size_t)-1)  // invalid shape: the allocating entry point names the error
        return svq_w4a16_gemm(x, qweight_tiled, scales, out, M, N, K, group_size, nullptr, 0, stream);
    if (need > kScratchBytes) return SVQ_ERR_WORKSPACE;
    void *ws = nullptr;
    int dev = -1;
    if (need) {
        const int st = scratch_address(&ws, &dev);
        if (st != SVQ_OK) return st;
    }
    // validate every argument before anything is enqueued: the call is planned
    // as for real and its launch recorded, not made
    {
        LaunchShape shape{};
        capture_slot() = &shape;
        const int st = svq_w4a16_gemm(x, qweight_tiled, scales, out, M, N, K, group_size, ws,
                                      need ? kScratchBytes : 0, stream);
        capture_slot() = nullptr;
        if (st != SVQ_OK) return st;
    }
    if (need) {
        const int st = clear_once(dev, ws, (hipStream_t)stream);
        if (st != SVQ_OK) return st;
    }
    return svq_w4a16_gemm(x, qweight_tiled, scales, out, M, N, K, group_size, ws, need ? kScratchBytes : 0,
                          stream);
}
