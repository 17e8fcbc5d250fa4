// mx_internal.h -- argument bundles and kernel launchers shared by the C ABI (mx_api.cpp)
// and the kernel files.  Private to libmx.  Arguments reaching these launchers have been
// validated by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mxk {

enum { FMT_E4M3 = 0, FMT_UE5M3 = 1, FMT_E8M0 = 2 };  // same values as mx_scale_fmt

// Unsigned division by a launch-constant d as a multiply and shift (Granlund & Montgomery's
// round-up method): q = (mulhi(u, mul) + u) >> shift, exact for every u < 2^31.
struct FastDiv {
    uint32_t mul, shift;
    static FastDiv make(uint32_t d)
    {
        uint32_t s = 0;
        while ((uint64_t(1) << s) < d) ++s;
        FastDiv f;
        f.mul = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
        f.shift = s;
        return f;
    }
    __host__ __device__ __forceinline__ uint32_t div(uint32_t u) const
    {
        return ((uint32_t)(((uint64_t)u * mul) >> 32) + u) >> shift;
    }
};

struct QuantArgs {
    const void* x;
    bool bf16;        // input element type
    int64_t rows, k, ldx;
    int block;
    int fmt;          // FMT_E4M3 / FMT_UE5M3 / FMT_E8M0
    double g;         // per-tensor scale (an fp32 value)
    uint8_t* codes;
    uint8_t* scales;
    bool fast;        // k % 32 == 0 and 16-byte aligned rows
};

struct DequantArgs {
    const uint8_t* codes;
    const uint8_t* scales;
    int64_t rows, k;
    int block;
    int fmt;
    double g;
    void* y;
    bool bf16;        // output element type
    int64_t ldy;
    bool fast;
};

struct GemmArgs {
    const uint16_t* x;        // bf16 activations, m x k
    int64_t m, n, k, ldx;
    const uint8_t* wc;        // n x k/2
    const uint8_t* ws;        // n x k/block
    int block;
    int fmt;
    float g;
    void* y;
    bool y_bf16;
    int64_t ldy;
    // W4A4: quantized activations (m x k/2 codes, m x k/32 scales) in the workspace
    uint8_t* xq_codes;
    uint8_t* xq_scales;
};

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st);
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t st);
hipError_t launch_gemm_a16(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_a4(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_a4_mfma(const GemmArgs& a, hipStream_t st);
hipError_t launch_fill_zero(void* y, int64_t m, int64_t n, int64_t ldy, bool bf16, hipStream_t st);

}  // namespace mxk
