// mx_static.hip -- mx_gemm_static: mx_gemm with its workspace in a fixed, library-owned
// device buffer instead of one the caller allocates, for callers that cannot allocate device
// memory around the call (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// The buffer is a file-scope __device__ array: every GPU the library runs on holds its own
// copy for the life of the process.  Its device address is looked up once per device with
// hipGetSymbolAddress (the array's name in host code is only a host-side handle) and kept;
// kernels receive that address exactly as they receive a caller's workspace in mx_gemm.
// Nothing here allocates or frees memory.
#include <mutex>

#include "mx.h"
#include "mx_internal.h"

namespace {

constexpr size_t kScratchBytes = MX_GEMM_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// Device address of this device's copy of `scratch` (looked up on first use, with the device
// current); null on failure.
void* scratch_on(int dev)
{
    std::call_once(g_once[dev], [dev] {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        g_status[dev] = e;
        g_scratch[dev] = e == hipSuccess ? p : nullptr;
    });
    return g_status[dev] == hipSuccess ? g_scratch[dev] : nullptr;
}

}  // namespace

extern "C" mx_status mx_gemm_static(const void* x, int64_t m, int64_t n, int64_t k, int64_t ld_x,
                                    const uint8_t* w_codes, const uint8_t* w_scales, int block,
                                    mx_scale_fmt fmt, float tensor_scale, mx_layout layout,
                                    mx_act_mode mode, void* y, mx_dtype y_type, int64_t ld_y,
                                    void* stream)
{
    const size_t need = mx_gemm_workspace_size(m, n, k, block, mode);
    if (need == 0)  // W4A16, invalid arguments or an empty shape: mx_gemm decides
        return mx_gemm(x, m, n, k, ld_x, w_codes, w_scales, block, fmt, tensor_scale, layout, mode, y,
                       y_type, ld_y, nullptr, 0, stream);
    if (need > kScratchBytes) return MX_ERR_TOO_LARGE;
    // the device the work runs on: the stream's (the current device for the null stream)
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return MX_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MX_ERR_UNSUPPORTED;
    void* ws = scratch_on(dev);
    if (!ws) return MX_ERR_HIP;
    return mx_gemm(x, m, n, k, ld_x, w_codes, w_scales, block, fmt, tensor_scale, layout, mode, y, y_type,
                   ld_y, ws, kScratchBytes, stream);
}
