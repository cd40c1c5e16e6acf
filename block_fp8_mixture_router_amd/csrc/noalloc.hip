// moe_forward_noalloc: moe_forward with the library's own workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// allocation-free serving loops).
//
// The workspace is `scratch`, a file-scope device array of
// MOE_NOALLOC_WORKSPACE_BYTES that every GPU the library runs on holds from
// the library's load until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in): the first
// call on each device, with that device current, looks up the device address
// of that device's copy once (hipGetSymbolAddress) and every later call uses
// that address.
//
// The array starts zero-filled (as moe_forward requires of a new workspace).
// moe_forward keeps a workspace valid between calls of one config; when a
// call on a device comes with a different config than the previous call on
// that device, the array is first cleared again by a fill kernel on the
// call's stream (no memset node: the call may be captured into a graph).
// All calls on one GPU share its array: calls that overlap in time on one
// GPU race, whatever their streams.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "moe.h"

namespace moe {
moe_status forward_checks(const moe_config *cfg, const moe_weights *w, const void *x, int32_t T,
                          const void *y, const void *workspace, size_t workspace_bytes,
                          bool own_workspace);
}

constexpr size_t SCRATCH_BYTES = MOE_NOALLOC_WORKSPACE_BYTES;
static_assert(SCRATCH_BYTES % 256 == 0, "whole 256-byte lines");

static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;

struct DeviceScratch {
    std::once_flag once;
    hipError_t rc = hipErrorNotInitialized;
    void *ptr = nullptr;  // device address of this device's copy of scratch
    std::mutex m;
    bool have_cfg = false;
    moe_config last{};  // config of the previous call on this device
};
DeviceScratch g_scratch[MAX_DEVICES];

// zero-fills n16 16-byte words
__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4 *p, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

moe_status moe_forward_noalloc(const moe_config *cfg, const moe_weights *w, const void *x,
                               int32_t T, void *y, void *stream) {
    // every host-side check before the device is touched: a call the array
    // cannot serve is refused and enqueues nothing
    if (cfg && T > 0 && moe_workspace_bytes(cfg, T) > SCRATCH_BYTES) return MOE_E_WORKSPACE;
    const moe_status s = moe::forward_checks(cfg, w, x, T, y, nullptr, 0, true);
    if (s != MOE_OK || T == 0) return s;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MOE_E_UNSUPPORTED;
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&d] {
        void *p = nullptr;
        d.rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (d.rc == hipSuccess) d.ptr = p;
    });
    if (d.rc != hipSuccess || !d.ptr) return MOE_E_LAUNCH;
    hipStream_t st = static_cast<hipStream_t>(stream);
    {
        std::lock_guard<std::mutex> lock(d.m);
        if (!d.have_cfg || std::memcmp(&d.last, cfg, sizeof(moe_config)) != 0) {
            hipLaunchKernelGGL(scratch_clear_kernel, dim3(1024), dim3(256), 0, st,
                               static_cast<uint4 *>(d.ptr), SCRATCH_BYTES / 16);
            if (hipGetLastError() != hipSuccess) return MOE_E_LAUNCH;
            d.last = *cfg;
            d.have_cfg = true;
        }
    }
    return moe_forward(cfg, w, x, T, y, d.ptr, SCRATCH_BYTES, stream);
}
