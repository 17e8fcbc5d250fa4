// mx_internal.h -- argument bundles and kernel launchers shared by the C ABI (mx_api.cpp)
// and the kernel files.  Private to libmx.  Arguments reaching these launchers have been
// validated by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace mxk {

// The dynamic-LDS limit of one kernel, raised above the 64 KB default.  The limit is an
// attribute the runtime keeps per device, so it is set once on each device that launches the
// kernel (the device of the launch stream; the calling thread's current device for the null
// stream) and remembered in a bit per device; devices 32 and up set it on every launch.
class LdsLimit {
public:
    hipError_t ensure(const void* kernel, int bytes, hipStream_t st)
    {
        int dev = 0;
        hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint32_t bit = dev >= 0 && dev < 32 ? 1u << dev : 0u;
        if (bit && (done_.load(std::memory_order_acquire) & bit)) return hipSuccess;
        int cur = dev;
        if (st && (e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e == hipSuccess && bit) done_.fetch_or(bit, std::memory_order_release);
        return e;
    }

private:
    std::atomic<uint32_t> done_{0};
};

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
    uint32_t ts_ks;   // 0: row-major scales; else tiled scales with this many 256-k stages
    uint32_t ps_cb;   // 0: not preshuffled; else preshuffled scales with this many 2048-k chunks
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
    uint32_t ts_ks;   // 0: row-major scales; else tiled scales with this many 256-k stages
    uint32_t ps_cb;   // 0: not preshuffled; else preshuffled scales with this many 2048-k chunks
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
    bool ws_tiled;            // weight scales in the tiled layout (else row-major)
    bool ws_pre;              // weight scales in the preshuffled layout (m == 1 GEMV only)
    // W4A4: quantized activations in the workspace (m x k/2 codes; scales tiled for the
    // matrix-core kernel, row-major for the direct one)
    uint8_t* xq_codes;
    uint8_t* xq_scales;
};

// Tiled scale layout (block 32): rows in tiles of 256, k in stages of 256 (8 blocks); the
// 2048 bytes of a (row tile, stage) pair are contiguous, tile-major then stage, and inside
// them the byte of row r (0..255 in the tile), block b (0..7 in the stage) sits at
// 1024 (r / 128) + 32 (r % 32) + 8 ((r / 32) % 4) + b.
constexpr int64_t kTileRows = 256, kTileK = 256, kTileBytes = 2048;

// Preshuffled scale layout (block 32): rows in groups of 8, k in chunks of 2048 (64 blocks);
// the 512 bytes of a (row group, chunk) pair are contiguous, group-major then chunk, and inside
// them the byte of row r (0..7 in the group), block b (0..63 in the chunk) sits at 8 b + r, so
// that one 8-byte word holds one block's scales of all 8 rows.
constexpr int64_t kPreRows = 8, kPreBlocks = 64, kPreBytes = 512;
inline int64_t pre_chunks(int64_t k) { return (k / 32 + kPreBlocks - 1) / kPreBlocks; }
inline int64_t pre_scale_bytes(int64_t rows, int64_t k)
{
    return (rows + kPreRows - 1) / kPreRows * pre_chunks(k) * kPreBytes;
}
inline int64_t tiled_stages(int64_t k) { return (k + kTileK - 1) / kTileK; }
inline int64_t tiled_scale_bytes(int64_t rows, int64_t k)
{
    return (rows + kTileRows - 1) / kTileRows * tiled_stages(k) * kTileBytes;
}
// whether the W4A4 product runs on the matrix-core kernel (else the direct one)
bool a4_uses_mfma(const GemmArgs& a);
// whether the large-m W4A16 product runs on the pipelined kernel (else the simple one)
bool a16_uses_tiled(const GemmArgs& a);
hipError_t launch_gemm_a16_tiled(const GemmArgs& a, hipStream_t st);
// the same pipelined kernel with FP8 (E4M3) weight codes, n x k bytes (same conditions)
hipError_t launch_gemm_w8_tiled(const GemmArgs& a, hipStream_t st);
// the large-m W4A16 / W8A16 GEMM with 128 x 64 wave tiles (E4M3 / UE5M3 weight scales and FP8
// weights)
bool a16w_uses(const GemmArgs& a, bool w8);
hipError_t launch_gemm_a16w(const GemmArgs& a, bool w8, hipStream_t st);
// the large-m W4A16 GEMM with two 4-wave workgroups per CU (FP4 codes, E8M0 scales, more
// 128 x 256 tiles than CUs, and the pipelined kernel's other conditions)
bool a16p_uses(const GemmArgs& a);
hipError_t launch_gemm_a16p(const GemmArgs& a, hipStream_t st);
// whether the m <= 2 sweeping GEMV takes FP8 codes of this shape, and its launcher
bool w8_uses_sweep(const GemmArgs& a);
hipError_t launch_gemv_sweep_w8(const GemmArgs& a, hipStream_t st);
// the 2 <= m <= 16 GEMV with the activations in registers and 16-row weight units streamed in
// address order (k = 4096, blocks of 32 and more, row-major scales)
bool gemv16_applies(const GemmArgs& a);
hipError_t launch_gemv16(const GemmArgs& a, hipStream_t st);

struct ErrArgs {
    const void* x;
    bool bf16;        // input element type
    int64_t rows, k, ldx;
    int block;
    int fmt;
    double g;
    void* xhat;       // optional x^ output (element type of x), row stride ldxh
    int64_t ldxh;
    bool fast;        // k % 32 == 0, 16-byte aligned rows, rows * k / 32 < 2^31
    double* partials; // workspace: ERR_NP doubles per workgroup
    double* out;      // 7 doubles
};

constexpr int kErrMaxGroups = 1024;  // workgroups of the error reduction (fixed grid cap)
int quant_error_groups(int64_t rows, int64_t k, int block);

struct StatsArgs {
    const void* x;
    bool bf16;        // element type
    int64_t rows, k, ldx;
    bool vec;         // k % 8 == 0 and 16-byte aligned rows: 16-byte loads
    double* partials; // workspace: 2 doubles per workgroup
    double* out;      // mean, standard deviation, max |x|
};

constexpr int kStatsMaxGroups = 1024;  // workgroups of each statistics pass (fixed grid cap)
int stats_groups(int64_t rows, int64_t k);

// W8A16 GEMM with FP8 (E4M3) weights
struct W8Args {
    const uint16_t* x;        // bf16 activations, m x k
    int64_t m, n, k, ldx;
    const uint8_t* wc;        // n x k E4M3 bytes
    const uint8_t* ws;        // n x k/block scale bytes
    int block;
    int fmt;
    double g;
    void* y;
    bool y_bf16;
    int64_t ldy;
    bool fast;                // k % 32 == 0, 16-byte aligned rows, 32-bit offsets: matrix-core kernel
};

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t st);     // codes: rows x k bytes
hipError_t launch_dequantize_fp8(const DequantArgs& a, hipStream_t st);
hipError_t launch_gemm_w8(const W8Args& a, hipStream_t st);

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st);
hipError_t launch_tensor_stats(const StatsArgs& a, hipStream_t st);
hipError_t launch_quant_error(const ErrArgs& a, hipStream_t st);
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t st);
hipError_t launch_gemm_a16(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_a4(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_a4_mfma(const GemmArgs& a, hipStream_t st);
hipError_t launch_fill_zero(void* y, int64_t m, int64_t n, int64_t ldy, bool bf16, hipStream_t st);

}  // namespace mxk
