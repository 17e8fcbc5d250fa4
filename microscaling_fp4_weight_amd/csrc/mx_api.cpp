// mx_api.cpp -- the C ABI of libmx (declared in include/mx.h): argument validation,
// dispatch to the gfx950 kernels, and error mapping.  Host code only; no allocation, no
// synchronization, no global mutable state.
#include "mx.h"

#include <cmath>
#include <cstdint>

#include "mx_internal.h"

namespace {

bool valid_block(int b)
{
    return b == 4 || b == 8 || b == 16 || b == 32 || b == 64 || b == 128 || b == 256;
}

bool valid_g(float g) { return std::isfinite(g) && std::isnormal(g) && g > 0.0f; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mx_status from_hip(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

constexpr size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

// Large tensors are processed in row chunks so that every launch indexes fewer than 2^29
// work units (the kernels use 32-bit unit indices and grid sizes); k itself is bounded.
constexpr int64_t kMaxUnitsPerLaunch = int64_t(1) << 29;
constexpr int64_t kMaxK = int64_t(1) << 25;      // keeps per-workgroup buffer ranges below 2^31 bytes
constexpr int64_t kMaxGemmK = int64_t(1) << 22;  // 256-row operand tiles of k/2 bytes stay below 2^31

int64_t chunk_rows(int64_t k)
{
    const int64_t per_row = k / 2 > 1 ? k / 2 : 1;  // finest unit of any kernel: an element pair
    const int64_t r = kMaxUnitsPerLaunch / per_row;
    return r > 0 ? r : 1;
}

// Common checks of a quantized tensor description.
mx_status check_quantized(int64_t rows, int64_t k, int block, mx_scale_fmt fmt, float g,
                          mx_layout layout)
{
    if (rows < 0 || k < 0 || (k & 1) || !valid_block(block) || k % block != 0)
        return MX_ERR_INVALID_ARG;
    if (fmt != MX_SCALE_E4M3 && fmt != MX_SCALE_UE5M3 && fmt != MX_SCALE_E8M0)
        return MX_ERR_INVALID_ARG;
    if (layout != MX_LAYOUT_ROWMAJOR && layout != MX_LAYOUT_TILED && layout != MX_LAYOUT_PRESHUFFLED)
        return MX_ERR_INVALID_ARG;
    if (!valid_g(g)) return MX_ERR_INVALID_ARG;
    // the tiled scale layout is defined for 32-element blocks, and rows are processed in
    // whole 256-row tiles per launch, which bounds k as for the matmul
    if (layout == MX_LAYOUT_TILED && (block != 32 || k > kMaxGemmK)) return MX_ERR_UNSUPPORTED;
    if (layout == MX_LAYOUT_PRESHUFFLED && block != 32) return MX_ERR_UNSUPPORTED;
    return MX_OK;
}

// Rows per launch for a quantized tensor: whole 256-row tiles for tiled scales.
int64_t launch_rows(int64_t k, mx_layout layout)
{
    int64_t step = chunk_rows(k);
    if (layout == MX_LAYOUT_TILED) step = step < mxk::kTileRows ? mxk::kTileRows : step / mxk::kTileRows * mxk::kTileRows;
    if (layout == MX_LAYOUT_PRESHUFFLED) step = step < mxk::kPreRows ? mxk::kPreRows : step / mxk::kPreRows * mxk::kPreRows;
    return step;
}

// Offset of row r0's scales (r0 a multiple of 256 for tiled scales).
int64_t scale_offset(int64_t r0, int64_t k, int block, mx_layout layout)
{
    if (layout == MX_LAYOUT_TILED) return r0 / mxk::kTileRows * mxk::tiled_stages(k) * mxk::kTileBytes;
    if (layout == MX_LAYOUT_PRESHUFFLED) return r0 / mxk::kPreRows * mxk::pre_chunks(k) * mxk::kPreBytes;
    return r0 * (k / block);
}

}  // namespace

extern "C" {

size_t mx_scale_bytes(int64_t rows, int64_t k, int block, mx_layout layout)
{
    if (rows < 0 || k < 0 || (k & 1) || !valid_block(block) || k % block != 0) return 0;
    if (layout == MX_LAYOUT_ROWMAJOR) return (size_t)rows * (size_t)(k / block);
    if (layout == MX_LAYOUT_TILED && block == 32 && k <= kMaxGemmK) return (size_t)mxk::tiled_scale_bytes(rows, k);
    if (layout == MX_LAYOUT_PRESHUFFLED && block == 32) return (size_t)mxk::pre_scale_bytes(rows, k);
    return 0;
}

const char* mx_status_string(mx_status s)
{
    switch (s) {
        case MX_OK: return "success";
        case MX_ERR_INVALID_ARG: return "invalid argument";
        case MX_ERR_UNSUPPORTED: return "unsupported combination";
        case MX_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
        case MX_ERR_HIP: return "HIP runtime error";
        case MX_ERR_TOO_LARGE: return "needs more than the library's static scratch buffer";
    }
    return "unknown status";
}

mx_status mx_quantize(const void* x, mx_dtype x_type, int64_t rows, int64_t k, int64_t ld_x,
                      int block, mx_scale_fmt fmt, float tensor_scale, mx_layout layout,
                      uint8_t* codes, uint8_t* scales, void* stream)
{
    mx_status st = check_quantized(rows, k, block, fmt, tensor_scale, layout);
    if (st != MX_OK) return st;
    if (x_type != MX_F32 && x_type != MX_BF16) return MX_ERR_INVALID_ARG;
    if (ld_x < k) return MX_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return MX_OK;
    if (!x || !codes || !scales) return MX_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MX_ERR_ALIGNMENT;
    const int esize = x_type == MX_BF16 ? 2 : 4;
    if (k > kMaxK) return MX_ERR_UNSUPPORTED;
    mxk::QuantArgs a{};
    a.x = x;
    a.bf16 = x_type == MX_BF16;
    a.rows = rows;
    a.k = k;
    a.ldx = ld_x;
    a.block = block;
    a.fmt = (int)fmt;
    a.g = (double)tensor_scale;
    a.codes = codes;
    a.scales = scales;
    a.fast = (k % 32 == 0) && ((ld_x * esize) % 16 == 0);
    a.ts_ks = layout == MX_LAYOUT_TILED ? (uint32_t)mxk::tiled_stages(k) : 0u;
    a.ps_cb = layout == MX_LAYOUT_PRESHUFFLED ? (uint32_t)mxk::pre_chunks(k) : 0u;
    const int64_t step = launch_rows(k, layout);
    for (int64_t r0 = 0; r0 < rows; r0 += step) {
        mxk::QuantArgs c = a;
        c.x = static_cast<const uint8_t*>(x) + r0 * ld_x * esize;
        c.codes = codes + r0 * (k / 2);
        c.scales = scales + scale_offset(r0, k, block, layout);
        c.rows = rows - r0 < step ? rows - r0 : step;
        if (mxk::launch_quantize(c, static_cast<hipStream_t>(stream)) != hipSuccess) return MX_ERR_HIP;
    }
    return MX_OK;
}

mx_status mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                        int block, mx_scale_fmt fmt, float tensor_scale, mx_layout layout,
                        void* y, mx_dtype y_type, int64_t ld_y, void* stream)
{
    mx_status st = check_quantized(rows, k, block, fmt, tensor_scale, layout);
    if (st != MX_OK) return st;
    if (y_type != MX_F32 && y_type != MX_BF16) return MX_ERR_INVALID_ARG;
    if (ld_y < k) return MX_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return MX_OK;
    if (!y || !codes || !scales) return MX_ERR_INVALID_ARG;
    if (!aligned16(y) || !aligned16(codes) || !aligned16(scales)) return MX_ERR_ALIGNMENT;
    const int esize = y_type == MX_BF16 ? 2 : 4;
    if (k > kMaxK) return MX_ERR_UNSUPPORTED;
    mxk::DequantArgs a{};
    a.codes = codes;
    a.scales = scales;
    a.rows = rows;
    a.k = k;
    a.block = block;
    a.fmt = (int)fmt;
    a.g = (double)tensor_scale;
    a.y = y;
    a.bf16 = y_type == MX_BF16;
    a.ldy = ld_y;
    a.fast = (k % 32 == 0) && ((ld_y * esize) % 16 == 0);
    a.ts_ks = layout == MX_LAYOUT_TILED ? (uint32_t)mxk::tiled_stages(k) : 0u;
    a.ps_cb = layout == MX_LAYOUT_PRESHUFFLED ? (uint32_t)mxk::pre_chunks(k) : 0u;
    const int64_t step = launch_rows(k, layout);
    for (int64_t r0 = 0; r0 < rows; r0 += step) {
        mxk::DequantArgs c = a;
        c.codes = codes + r0 * (k / 2);
        c.scales = scales + scale_offset(r0, k, block, layout);
        c.y = static_cast<uint8_t*>(y) + r0 * ld_y * esize;
        c.rows = rows - r0 < step ? rows - r0 : step;
        if (mxk::launch_dequantize(c, static_cast<hipStream_t>(stream)) != hipSuccess) return MX_ERR_HIP;
    }
    return MX_OK;
}

size_t mx_quant_error_workspace_size(int64_t rows, int64_t k, int block)
{
    if (rows < 0 || k < 0 || (k & 1) || !valid_block(block) || k % block != 0) return 0;
    if (rows == 0 || k == 0) return 0;
    return round256((size_t)mxk::quant_error_groups(rows, k, block) * 6 * sizeof(double));
}

mx_status mx_quant_error(const void* x, mx_dtype x_type, int64_t rows, int64_t k, int64_t ld_x,
                         int block, mx_scale_fmt fmt, float tensor_scale, void* x_hat,
                         int64_t ld_x_hat, double* out, void* workspace, size_t workspace_bytes,
                         void* stream)
{
    mx_status st = check_quantized(rows, k, block, fmt, tensor_scale, MX_LAYOUT_ROWMAJOR);
    if (st != MX_OK) return st;
    if (x_type != MX_F32 && x_type != MX_BF16) return MX_ERR_INVALID_ARG;
    if (ld_x < k || (x_hat && ld_x_hat < k)) return MX_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return MX_OK;
    if (!x || !out) return MX_ERR_INVALID_ARG;
    const size_t need = mx_quant_error_workspace_size(rows, k, block);
    if (!workspace || workspace_bytes < need) return MX_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(out) || !aligned16(workspace) || (x_hat && !aligned16(x_hat)))
        return MX_ERR_ALIGNMENT;
    if (k > kMaxK) return MX_ERR_UNSUPPORTED;
    const int64_t esize = x_type == MX_BF16 ? 2 : 4;
    mxk::ErrArgs a;
    a.x = x;
    a.bf16 = x_type == MX_BF16;
    a.rows = rows;
    a.k = k;
    a.ldx = ld_x;
    a.block = block;
    a.fmt = (int)fmt;
    a.g = (double)tensor_scale;
    a.xhat = x_hat;
    a.ldxh = x_hat ? ld_x_hat : 0;
    a.fast = (k % 32 == 0) && ((ld_x * esize) % 16 == 0) && (!x_hat || (ld_x_hat * esize) % 16 == 0) &&
             rows * (k / 32) < (int64_t(1) << 31);
    a.partials = static_cast<double*>(workspace);
    a.out = out;
    return from_hip(mxk::launch_quant_error(a, static_cast<hipStream_t>(stream)));
}

size_t mx_tensor_stats_workspace_size(int64_t rows, int64_t k)
{
    if (rows <= 0 || k <= 0) return 0;
    return round256((size_t)mxk::stats_groups(rows, k) * 2 * sizeof(double));
}

mx_status mx_tensor_stats(const void* x, mx_dtype x_type, int64_t rows, int64_t k, int64_t ld_x, double* out,
                          void* workspace, size_t workspace_bytes, void* stream)
{
    if (rows < 0 || k < 0 || ld_x < k) return MX_ERR_INVALID_ARG;
    if (x_type != MX_F32 && x_type != MX_BF16) return MX_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return MX_OK;
    if (!x || !out) return MX_ERR_INVALID_ARG;
    const size_t need = mx_tensor_stats_workspace_size(rows, k);
    if (!workspace || workspace_bytes < need) return MX_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(out) || !aligned16(workspace)) return MX_ERR_ALIGNMENT;
    const int64_t esize = x_type == MX_BF16 ? 2 : 4;
    const bool vec = (k % 8 == 0) && ((ld_x * esize) % 16 == 0);
    if (rows * (vec ? k / 8 : k) >= (int64_t(1) << 31)) return MX_ERR_UNSUPPORTED;
    mxk::StatsArgs a;
    a.x = x;
    a.bf16 = x_type == MX_BF16;
    a.rows = rows;
    a.k = k;
    a.ldx = ld_x;
    a.vec = vec;
    a.partials = static_cast<double*>(workspace);
    a.out = out;
    return from_hip(mxk::launch_tensor_stats(a, static_cast<hipStream_t>(stream)));
}

int mx_adaptive_block_size(double sigma)
{
    if (sigma < 0.01) return 128;
    if (sigma < 0.1) return 64;
    return 32;  // also NaN
}

int mx_layer_block_size(mx_layer_kind kind)
{
    switch (kind) {
        case MX_LAYER_QKV: return 64;
        case MX_LAYER_FFN_GATE_UP: return 32;
        case MX_LAYER_OUTPUT: return 128;
        default: return 0;
    }
}

// ---------------------------------------------------------------------------------------
// FP8 weight fallback
// ---------------------------------------------------------------------------------------
mx_status mx_quantize_fp8(const void* x, mx_dtype x_type, int64_t rows, int64_t k, int64_t ld_x, int block,
                          mx_scale_fmt fmt, float tensor_scale, uint8_t* codes, uint8_t* scales, void* stream)
{
    mx_status st = check_quantized(rows, k, block, fmt, tensor_scale, MX_LAYOUT_ROWMAJOR);
    if (st != MX_OK) return st;
    if (x_type != MX_F32 && x_type != MX_BF16) return MX_ERR_INVALID_ARG;
    if (ld_x < k) return MX_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return MX_OK;
    if (!x || !codes || !scales) return MX_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MX_ERR_ALIGNMENT;
    if (k > kMaxK) return MX_ERR_UNSUPPORTED;
    const int64_t esize = x_type == MX_BF16 ? 2 : 4;
    mxk::QuantArgs a{};
    a.x = x;
    a.bf16 = x_type == MX_BF16;
    a.rows = rows;
    a.k = k;
    a.ldx = ld_x;
    a.block = block;
    a.fmt = (int)fmt;
    a.g = (double)tensor_scale;
    a.codes = codes;
    a.scales = scales;
    a.fast = (k % 8 == 0) && ((ld_x * esize) % 16 == 0) && rows * (k / 8) < (int64_t(1) << 31);
    a.ts_ks = 0;
    a.ps_cb = 0;
    return from_hip(mxk::launch_quantize_fp8(a, static_cast<hipStream_t>(stream)));
}

mx_status mx_dequantize_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k, int block,
                            mx_scale_fmt fmt, float tensor_scale, void* y, mx_dtype y_type, int64_t ld_y,
                            void* stream)
{
    mx_status st = check_quantized(rows, k, block, fmt, tensor_scale, MX_LAYOUT_ROWMAJOR);
    if (st != MX_OK) return st;
    if (y_type != MX_F32 && y_type != MX_BF16) return MX_ERR_INVALID_ARG;
    if (ld_y < k) return MX_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return MX_OK;
    if (!codes || !scales || !y) return MX_ERR_INVALID_ARG;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(y)) return MX_ERR_ALIGNMENT;
    if (k > kMaxK) return MX_ERR_UNSUPPORTED;
    const int64_t esize = y_type == MX_BF16 ? 2 : 4;
    mxk::DequantArgs a{};
    a.codes = codes;
    a.scales = scales;
    a.rows = rows;
    a.k = k;
    a.block = block;
    a.fmt = (int)fmt;
    a.g = (double)tensor_scale;
    a.y = y;
    a.bf16 = y_type == MX_BF16;
    a.ldy = ld_y;
    a.fast = (k % 8 == 0) && ((ld_y * esize) % 16 == 0) && rows * (k / 8) < (int64_t(1) << 31);
    a.ts_ks = 0;
    a.ps_cb = 0;
    return from_hip(mxk::launch_dequantize_fp8(a, static_cast<hipStream_t>(stream)));
}

mx_status mx_gemm_fp8(const void* x, int64_t m, int64_t n, int64_t k, int64_t ld_x, const uint8_t* w_codes,
                      const uint8_t* w_scales, int block, mx_scale_fmt fmt, float tensor_scale, void* y,
                      mx_dtype y_type, int64_t ld_y, void* stream)
{
    if (m < 0 || n < 0) return MX_ERR_INVALID_ARG;
    mx_status st = check_quantized(n, k, block, fmt, tensor_scale, MX_LAYOUT_ROWMAJOR);
    if (st != MX_OK) return st;
    if (y_type != MX_F32 && y_type != MX_BF16) return MX_ERR_INVALID_ARG;
    if (ld_x < k || ld_y < n) return MX_ERR_INVALID_ARG;
    if (m == 0 || n == 0) return MX_OK;
    if (!y) return MX_ERR_INVALID_ARG;
    if (!aligned16(y)) return MX_ERR_ALIGNMENT;
    if (k == 0)
        return from_hip(mxk::launch_fill_zero(y, m, n, ld_y, y_type == MX_BF16, static_cast<hipStream_t>(stream)));
    if (!x || !w_codes || !w_scales) return MX_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_codes) || !aligned16(w_scales)) return MX_ERR_ALIGNMENT;
    if (k > kMaxGemmK) return MX_ERR_UNSUPPORTED;
    mxk::W8Args a{};
    a.x = static_cast<const uint16_t*>(x);
    a.m = m;
    a.n = n;
    a.k = k;
    a.ldx = ld_x;
    a.wc = w_codes;
    a.ws = w_scales;
    a.block = block;
    a.fmt = (int)fmt;
    a.g = (double)tensor_scale;
    a.y = y;
    a.y_bf16 = y_type == MX_BF16;
    a.ldy = ld_y;
    const int64_t xspan = (63 * ld_x + k) * 2, yspan = (63 * ld_y + 16) * 4;
    a.fast = (k % 32 == 0) && ((ld_x * 2) % 16 == 0) && xspan < (int64_t(1) << 31) &&
             yspan < (int64_t(1) << 31) && 16 * k < (int64_t(1) << 31);
    return from_hip(mxk::launch_gemm_w8(a, static_cast<hipStream_t>(stream)));
}

int mx_use_fp8(double sigma)
{
    return sigma < 1e-4 ? 1 : 0;
}

size_t mx_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int block, mx_act_mode mode)
{
    if (m < 0 || n < 0 || k < 0 || (k & 1) || !valid_block(block) || k % block != 0) return 0;
    if (mode != MX_A4) return 0;
    if (block != 32) return 0;
    // activation scales in the tiled layout (never smaller than row-major ones)
    return round256((size_t)m * (size_t)(k / 2)) + round256((size_t)mxk::tiled_scale_bytes(m, k));
}

mx_status mx_gemm(const void* x, int64_t m, int64_t n, int64_t k, int64_t ld_x,
                  const uint8_t* w_codes, const uint8_t* w_scales, int block, mx_scale_fmt fmt,
                  float tensor_scale, mx_layout layout, mx_act_mode mode, void* y,
                  mx_dtype y_type, int64_t ld_y, void* workspace, size_t workspace_bytes,
                  void* stream)
{
    if (m < 0 || n < 0) return MX_ERR_INVALID_ARG;
    mx_status st = check_quantized(n, k, block, fmt, tensor_scale, layout);
    if (st != MX_OK) return st;
    if (mode != MX_A16 && mode != MX_A4) return MX_ERR_INVALID_ARG;
    if (y_type != MX_F32 && y_type != MX_BF16) return MX_ERR_INVALID_ARG;
    if (ld_x < k || ld_y < n) return MX_ERR_INVALID_ARG;
    if (mode == MX_A4 && (fmt != MX_SCALE_E8M0 || block != 32)) return MX_ERR_UNSUPPORTED;
    if (m == 0 || n == 0) return MX_OK;
    if (!y) return MX_ERR_INVALID_ARG;
    if (!aligned16(y)) return MX_ERR_ALIGNMENT;
    if (k == 0)  // an empty sum: Y = 0
        return from_hip(mxk::launch_fill_zero(y, m, n, ld_y, y_type == MX_BF16, static_cast<hipStream_t>(stream)));
    if (!x || !w_codes || !w_scales) return MX_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(y))
        return MX_ERR_ALIGNMENT;
    const size_t need = mx_gemm_workspace_size(m, n, k, block, mode);
    if (workspace_bytes < need || (need && !workspace)) return MX_ERR_INVALID_ARG;
    if (need && !aligned16(workspace)) return MX_ERR_ALIGNMENT;
    if (k > kMaxGemmK) return MX_ERR_UNSUPPORTED;

    mxk::GemmArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.m = m;
    a.n = n;
    a.k = k;
    a.ldx = ld_x;
    a.wc = w_codes;
    a.ws = w_scales;
    a.block = block;
    a.fmt = (int)fmt;
    a.g = tensor_scale;
    a.y = y;
    a.y_bf16 = y_type == MX_BF16;
    a.ldy = ld_y;
    a.ws_tiled = layout == MX_LAYOUT_TILED;
    a.ws_pre = layout == MX_LAYOUT_PRESHUFFLED;
    a.xq_codes = nullptr;
    a.xq_scales = nullptr;
    // weight scales in the tiled layout are read by the W4A4 matrix-core kernel only
    const bool mfma_a4 = mode == MX_A4 && mxk::a4_uses_mfma(a);
    if (a.ws_tiled && !mfma_a4) return MX_ERR_UNSUPPORTED;
    // preshuffled weight scales are read by the m = 1 GEMV only
    if (a.ws_pre && (mode != MX_A16 || m != 1 || (ld_x * 2) % 16 != 0)) return MX_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    // rows of Y per launch: keeps per-launch unit counts (outputs, pre-pass pairs) < 2^29;
    // W4A4 launches take whole 256-row tiles (the activation scales are tiled)
    const int64_t per_row = n > k / 2 ? n : k / 2;
    int64_t step = kMaxUnitsPerLaunch / (per_row > 0 ? per_row : 1);
    step = step < 1 ? 1 : (step > 256 ? step & ~int64_t(255) : step);
    if (mode == MX_A4 && step < 256) step = 256;
    for (int64_t r0 = 0; r0 < m; r0 += step) {
        mxk::GemmArgs c = a;
        c.m = m - r0 < step ? m - r0 : step;
        c.x = a.x + r0 * ld_x;
        c.y = static_cast<uint8_t*>(y) + r0 * ld_y * (y_type == MX_BF16 ? 2 : 4);
        if (mode == MX_A16) {
            if (mxk::launch_gemm_a16(c, s) != hipSuccess) return MX_ERR_HIP;
            continue;
        }
        // W4A4: MX-quantize the activations (block 32, E8M0, g = 1) into the workspace with
        // the quantize kernel itself, then run the FP4 matrix-core product.
        c.xq_codes = ws + r0 * (k / 2);
        const mx_layout xl = mfma_a4 ? MX_LAYOUT_TILED : MX_LAYOUT_ROWMAJOR;
        c.xq_scales = ws + round256((size_t)m * (size_t)(k / 2)) + scale_offset(r0, k, 32, xl);
        mxk::QuantArgs q{};
        q.x = c.x;
        q.bf16 = true;
        q.rows = c.m;
        q.k = k;
        q.ldx = ld_x;
        q.block = 32;
        q.fmt = mxk::FMT_E8M0;
        q.g = 1.0;
        q.codes = c.xq_codes;
        q.scales = c.xq_scales;
        q.fast = (ld_x * 2) % 16 == 0;  // k % 32 == 0 holds (block 32)
        q.ts_ks = mfma_a4 ? (uint32_t)mxk::tiled_stages(k) : 0u;
        q.ps_cb = 0;
        if (mxk::launch_quantize(q, s) != hipSuccess) return MX_ERR_HIP;
        if (mxk::launch_gemm_a4(c, s) != hipSuccess) return MX_ERR_HIP;
    }
    return MX_OK;
}

}  // extern "C"
