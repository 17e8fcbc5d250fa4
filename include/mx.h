/*
 * mx.h -- C ABI of libmx: MX FP4 block quantization and the FP4-weight matmul on AMD
 * MI355X (gfx950).
 *
 * Method (pages cited by key):
 *  [MXS]  hotelren.com/news/2192771, the article opening with "量化技术演进与微缩量化原理"
 *         (microscaling: FP4 elements sharing one FP8 block scale).
 *  [FP4L] gtnt.cn/news/16247, "为什么我们需要4-bit浮点量化" (4-bit float quantization).
 *
 *  Quantize ([MXS] section 3.1 item 2, quantize_block; item 3, two-level scaling): for every
 *  block of `block` consecutive elements along a row, a = max |x|; the block scale s is the
 *  value of the scale format nearest to a / (6 g) (ties to the even code; E8M0 ties to the
 *  larger power of two; out-of-range values saturate); every element becomes the E2M1 code
 *  nearest to |x| / (s g), clipped at 6 ([FP4L] section 2.1, round(clip(.))), ties to the
 *  even code, with the sign bit of x; a zero scale codes the whole block as zero.
 *  Dequantize ([MXS] sections 1 and 3.1 item 3): x^ = e(code) * s * g.
 *  Matmul ([FP4L] section 3.1, dequantize then matmul): Y = X . dequant(Wq)^T.
 *
 * Formats
 *  E2M1 element code (4 bits): [sign][exp 2][man 1], bias 1, values
 *    {0, 0.5, 1, 1.5, 2, 3, 4, 6} and their negatives; no Inf/NaN.
 *  MX_SCALE_E4M3:  OCP E4M3FN byte (bias 7, subnormals, 0x7F NaN, max 448); a block scale
 *                  of 0 (byte 0x00) flushes the block.
 *  MX_SCALE_UE5M3: unsigned 5-bit exponent (bias 15, subnormals), 3-bit mantissa,
 *                  0xFF NaN, max 114688.
 *  MX_SCALE_E8M0:  2^(byte - 127), bytes 0..254; never zero.
 *  The NaN bytes of the scale formats (E4M3 0x7F and 0xFF, UE5M3 0xFF, E8M0 0xFF) are never
 *  written by mx_quantize; mx_dequantize and mx_gemm read them as unspecified values.
 *  tensor_scale g: fp32, finite, normal, > 0 (1.0 = single-level scaling).
 *
 * Layout MX_LAYOUT_ROWMAJOR:
 *  codes : rows x (k/2) bytes, row-major, no padding; byte j of row r holds element 2j in
 *          its low nibble and element 2j+1 in its high nibble ([FP4L] section 4.3: two FP4
 *          values per byte).
 *  scales: rows x (k/block) bytes, row-major, no padding; byte b of row r is the scale of
 *          elements [b*block, (b+1)*block) of row r.
 * Layout MX_LAYOUT_TILED (block 32 only; k <= 4,194,304): the same codes; the scales are
 *  stored in the order the W4A4 matrix-core GEMM streams them, so that each of its k steps
 *  reads one contiguous 2 KB piece instead of 8 bytes from each of 256 rows.  Rows are
 *  grouped in tiles of 256 (T = r / 256, t = r % 256) and blocks in stages of 8 (256
 *  elements; S = b / 8, u = b % 8); with KS = ceil(k / 256) stages, the scale of (r, b) is
 *  byte  2048 (T KS + S) + 1024 (t / 128) + 32 (t % 32) + 8 ((t / 32) % 4) + u.
 *  The buffer holds ceil(rows / 256) KS 2048 bytes (mx_scale_bytes).  Bytes of blocks
 *  past the end of k in a row's last stage are written as 0 by mx_quantize; bytes of rows
 *  past the end are never written nor used.
 * Layout MX_LAYOUT_PRESHUFFLED (block 32; [MXS] section 3.2 item 2 and section 5.3 item 3:
 *  scale factors grouped in aligned words, tensors rearranged for the kernel that reads
 *  them): the same codes; the scales in the order the m = 1 GEMV reads them, so that one
 *  8-byte word holds one 32-element block's scales of 8 consecutive rows.  Rows are grouped
 *  by 8 (R = r / 8, t = r % 8) and blocks in chunks of 64 (2048 elements; C = b / 64,
 *  u = b % 64); with KC = ceil(k / 2048) chunks, the scale of (r, b) is byte
 *  512 (R KC + C) + 8 u + t.  Bytes of the last chunk past the row's last block are written
 *  as 0; bytes of rows past the last row (rows % 8 != 0) are not written.  Size
 *  ceil(rows / 8) * KC * 512 bytes (mx_scale_bytes).  Read by mx_dequantize and by mx_gemm
 *  in W4A16 mode with m == 1.
 * Dense tensors (x, y) are row-major with a leading dimension (row stride) in ELEMENTS.
 *
 * Conventions common to every entry point
 *  - Every pointer is a DEVICE pointer owned by the caller.  The library never allocates,
 *    frees, or synchronizes; apart from mx_gemm_static's static scratch buffer (see there)
 *    it keeps no global mutable state and is thread-safe.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 *    Outputs are valid once the stream has reached the call.
 *  - Arguments are validated on the host before anything is launched.  On an error status
 *    nothing has been written.  No exception crosses this boundary and nothing is printed.
 *  - Pointers to non-empty tensors must be 16-byte aligned (MX_ERR_ALIGNMENT otherwise).
 *  - A call on an empty tensor (rows, k, m or n equal to 0) returns MX_OK and launches
 *    nothing; its pointers may then be NULL.  Exception: mx_gemm with k == 0 and m, n > 0
 *    writes Y = 0 (an empty sum).
 *  - Inputs must be finite; the result for non-finite inputs is unspecified.
 *  - MX_ERR_HIP is returned when a launch fails (hipGetLastError after the launch).
 *  - Rows longer than 2^25 elements (k > 33,554,432; for mx_gemm k > 4,194,304) return
 *    MX_ERR_UNSUPPORTED.
 */
#ifndef MX_H
#define MX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MX_OK = 0,
    MX_ERR_INVALID_ARG = -1, /* null pointer, negative size, k % block, bad enum, bad g, ... */
    MX_ERR_UNSUPPORTED = -2, /* a valid combination this library does not implement        */
    MX_ERR_ALIGNMENT = -3,   /* a pointer is not 16-byte aligned                           */
    MX_ERR_HIP = -4,         /* the HIP runtime reported an error at launch                */
    MX_ERR_TOO_LARGE = -5    /* mx_gemm_static: the call needs more than its static scratch */
} mx_status;

typedef enum { MX_SCALE_E4M3 = 0, MX_SCALE_UE5M3 = 1, MX_SCALE_E8M0 = 2 } mx_scale_fmt;
typedef enum { MX_F32 = 0, MX_BF16 = 1 } mx_dtype;
typedef enum { MX_LAYOUT_ROWMAJOR = 0, MX_LAYOUT_TILED = 1, MX_LAYOUT_PRESHUFFLED = 2 } mx_layout;
typedef enum { MX_A16 = 0, MX_A4 = 1 } mx_act_mode;

/*
 * mx_quantize -- MX block quantization of a rows x k tensor.
 *  x          : input, rows x k, element type x_type (MX_F32 or MX_BF16), row stride ld_x >= k.
 *  block      : block size along k, one of 4, 8, 16, 32, 64, 128, 256; k % block == 0.
 *  fmt        : block-scale format.
 *  tensor_scale: per-tensor fp32 scale g ([MXS] section 3.1 item 3; 1.0 for none).
 *  layout     : MX_LAYOUT_ROWMAJOR, MX_LAYOUT_TILED or MX_LAYOUT_PRESHUFFLED (scale order,
 *               above).
 *  codes      : output, rows x k/2 bytes (layout above).
 *  scales     : output, mx_scale_bytes(rows, k, block, layout) bytes.
 * Errors: MX_ERR_INVALID_ARG for a null pointer, rows/k/ld_x negative or ld_x < k, k odd,
 * a block size outside the list, k % block != 0, an unknown fmt/x_type/layout, or g not a
 * finite normal positive number; MX_ERR_UNSUPPORTED for MX_LAYOUT_TILED with block != 32
 * or k > 4,194,304, or MX_LAYOUT_PRESHUFFLED with block != 32; MX_ERR_ALIGNMENT for a
 * misaligned pointer.
 * Codes and scale bytes are bit-exact with the definition above.
 */
mx_status mx_quantize(const void* x, mx_dtype x_type, int64_t rows, int64_t k, int64_t ld_x,
                      int block, mx_scale_fmt fmt, float tensor_scale, mx_layout layout,
                      uint8_t* codes, uint8_t* scales, void* stream);

/*
 * mx_dequantize -- y = e(code) * s * g for a rows x k quantized tensor.
 *  codes, scales, rows, k, block, fmt, tensor_scale, layout: as written by mx_quantize.
 *  y          : output, rows x k, element type y_type, row stride ld_y >= k.
 * Output value: one fp32 rounding (nearest even) of the exact product e*s*g; for MX_BF16
 * output, the nearest-even bf16 of that fp32 value.  With g = 1 both are exact unless the
 * product overflows (then +-Inf).  Errors as for mx_quantize.
 */
mx_status mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                        int block, mx_scale_fmt fmt, float tensor_scale, mx_layout layout,
                        void* y, mx_dtype y_type, int64_t ld_y, void* stream);

/*
 * mx_scale_bytes -- size in bytes of the scale buffer of a rows x k tensor quantized with
 * this block size and layout (rows * k / block for MX_LAYOUT_ROWMAJOR; the tiled size
 * above for MX_LAYOUT_TILED).  Returns 0 for arguments mx_quantize would reject.
 */
size_t mx_scale_bytes(int64_t rows, int64_t k, int block, mx_layout layout);

/*
 * mx_quant_error -- the error of MX quantization, decomposed ([MXS] section 2.2 items 1-3),
 * computed on the device in one pass over x: every block is quantized exactly as by
 * mx_quantize (row-major, same block, fmt, tensor_scale), dequantized (x^ = e(code) * s * g,
 * exact in fp64), and each squared error (x^ - x)^2 is added to one of three sums:
 *   zero-scale term: every element of a block whose scale is 0 (flushed);
 *   max term:        in the other blocks, one element holding the block's largest |x|
 *                    (elements tied at the maximum share its code and its error);
 *   element term:    every other element.
 *  x_hat      : optional device output (NULL: not written), rows x k, element type x_type,
 *               row stride ld_x_hat >= k: the dequantized tensor, rounded exactly as
 *               mx_dequantize rounds it (the forward pass of fake quantization).
 *  out        : device, 7 doubles: MSE_elem, MSE_max, MSE_zero (each sum divided by
 *               rows * k), MSE_total (its own sum of all squared errors, / (rows * k)),
 *               number of blocks, number of flushed blocks, number of non-flushed blocks
 *               whose maximum is not coded +-6.
 *  workspace  : device buffer of at least mx_quant_error_workspace_size(rows, k, block) bytes
 *               (per-workgroup partial sums).
 * Sums are accumulated in fp64 in an order fixed by the shape and the alignment of x and
 * x_hat, so repeated calls return the same bits.  Errors as for mx_quantize (x_hat must be
 * 16-byte aligned too), plus MX_ERR_INVALID_ARG for a null out, a missing or short
 * workspace, or ld_x_hat < k with x_hat given.  For an empty tensor nothing is launched and
 * out is not written.
 */
size_t mx_quant_error_workspace_size(int64_t rows, int64_t k, int block);
mx_status mx_quant_error(const void* x, mx_dtype x_type, int64_t rows, int64_t k, int64_t ld_x,
                         int block, mx_scale_fmt fmt, float tensor_scale, void* x_hat,
                         int64_t ld_x_hat, double* out, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * FP8 weight fallback ([MXS] section 5.3 item 1: weights whose standard deviation is below
 * 1e-4 come out of FP4 quantization as zeros, and FP8 is the remedy named there; section 6
 * item 1: key layers kept in FP8).  The MX block structure with an 8-bit element: per block
 * of `block` consecutive elements along a row, the scale s is the scale-format value nearest
 * to a / (448 g) (448, the largest E4M3 magnitude, in place of 6), and every element becomes
 * the E4M3 byte (OCP E4M3FN: sign, 4 exponent bits with bias 7 and subnormals, 3 mantissa
 * bits, largest magnitude 448) nearest to |x| / (s g), clipped at 448, ties to the even
 * code, with the sign bit of x; a zero scale codes the block as +-0.  Note that the scale
 * falls below a / 448: E4M3 scales (smallest 2^-9) flush blocks with a <= 448 * 2^-10 * g and
 * UE5M3 scales (smallest 2^-17) those with a <= 448 * 2^-18 * g; E8M0 scales, or a per-tensor
 * g, keep small weights.
 *  codes : rows x k bytes, row-major (one byte per element).
 *  scales: rows x k/block bytes, row-major (MX_LAYOUT_ROWMAJOR order).
 *
 * mx_quantize_fp8 / mx_dequantize_fp8: as mx_quantize / mx_dequantize (same arguments,
 * errors and value rules: dequantized value one fp32 rounding of e * s * g, bf16 the
 * nearest-even bf16 of that; byte 0x7F/0xFF, never written by the quantizer, reads as NaN),
 * row-major scales only.
 *
 * mx_gemm_fp8 -- Y = X . dequant(Wq)^T with bf16 X (m x k, row stride ld_x) and FP8 weights
 * (n x k codes, n x k/block scales as written by mx_quantize_fp8), fp32 accumulation, Y of
 * y_type (m x n, row stride ld_y).  Weights enter the bf16 matrix cores as e * s, exact for
 * |e * s| >= 2^-133; g multiplies the fp32 sums.  Errors as mx_gemm (W4A16); needs no
 * workspace.
 *
 * mx_use_fp8 -- the fallback rule (host): 1 when sigma < 1e-4, else 0.
 */
mx_status mx_quantize_fp8(const void* x, mx_dtype x_type, int64_t rows, int64_t k, int64_t ld_x, int block,
                          mx_scale_fmt fmt, float tensor_scale, uint8_t* codes, uint8_t* scales, void* stream);
mx_status mx_dequantize_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k, int block,
                            mx_scale_fmt fmt, float tensor_scale, void* y, mx_dtype y_type, int64_t ld_y,
                            void* stream);
mx_status mx_gemm_fp8(const void* x, int64_t m, int64_t n, int64_t k, int64_t ld_x, const uint8_t* w_codes,
                      const uint8_t* w_scales, int block, mx_scale_fmt fmt, float tensor_scale, void* y,
                      mx_dtype y_type, int64_t ld_y, void* stream);
int mx_use_fp8(double sigma);

/*
 * Block-size policy ([MXS] section 6 item 2: the block size follows the tensor's standard
 * deviation; section 5.1 item 1: a block size per layer kind).
 *
 * mx_tensor_stats -- mean, sample standard deviation and max |x| of a whole rows x k tensor
 * (element type x_type, row stride ld_x >= k), on the device, in two fp64 passes:
 * mean = sum(x) / n, std = sqrt(sum((x - mean)^2) / (n - 1)) (NaN when n == 1).
 *  out        : device, 3 doubles: mean, std, max |x|.
 *  workspace  : device buffer of at least mx_tensor_stats_workspace_size(rows, k) bytes.
 * The sums run in an order fixed by the shape and alignment, so repeated calls return the
 * same bits.  Errors: MX_ERR_INVALID_ARG for negative sizes, ld_x < k, an unknown x_type, a
 * null x/out or a missing or short workspace; MX_ERR_ALIGNMENT unless x, out and workspace
 * are 16-byte aligned; MX_ERR_UNSUPPORTED beyond 2^31 - 1 load units (8 elements each for
 * k % 8 == 0 and 16-byte row strides, else single elements).  An empty tensor launches
 * nothing and leaves out unwritten.
 */
size_t mx_tensor_stats_workspace_size(int64_t rows, int64_t k);
mx_status mx_tensor_stats(const void* x, mx_dtype x_type, int64_t rows, int64_t k, int64_t ld_x, double* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * mx_adaptive_block_size -- block size for a tensor of standard deviation sigma (host):
 * 128 when sigma < 0.01, 64 when sigma < 0.1, otherwise 32 (NaN included).
 */
int mx_adaptive_block_size(double sigma);

/*
 * mx_layer_block_size -- block size by layer kind (host): Q/K/V projections 64, FFN gate and
 * up projections 32, output projection 128; 0 for an unknown kind.
 */
typedef enum { MX_LAYER_QKV = 0, MX_LAYER_FFN_GATE_UP = 1, MX_LAYER_OUTPUT = 2 } mx_layer_kind;
int mx_layer_block_size(mx_layer_kind kind);

/*
 * mx_gemm_workspace_size -- bytes of device workspace mx_gemm needs for this shape and mode
 * (0 when none).  MX_A4 needs room for the quantized activations: m*k/2 code bytes and
 * mx_scale_bytes(m, k, 32, MX_LAYOUT_TILED) scale bytes, each rounded up to 256 bytes.
 * Returns 0 for arguments mx_gemm would reject.
 */
size_t mx_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int block, mx_act_mode mode);

/*
 * mx_gemm -- Y = X . dequant(Wq)^T with fp32 accumulation.
 *  x          : activations, bf16, m x k, row stride ld_x >= k.
 *  w_codes    : weight codes, n x k/2 bytes; w_scales: mx_scale_bytes(n, k, block, layout)
 *               bytes (mx_quantize output for an n x k weight).
 *  block, fmt, tensor_scale, layout: those of the weight.  MX_LAYOUT_TILED weights are
 *               accepted in MX_A4 mode with k % 128 == 0 (MX_ERR_UNSUPPORTED otherwise)
 *               and make the W4A4 product faster; MX_LAYOUT_PRESHUFFLED weights in
 *               MX_A16 mode with m == 1 and ld_x a multiple of 8 (MX_ERR_UNSUPPORTED
 *               otherwise), with results bit-identical to the row-major order.
 *  mode       : MX_A16 -- X is used as given (bf16 x dequantized weight);
 *               MX_A4  -- X is first MX-quantized along k with block 32, E8M0 scales and
 *               g = 1 (bit-identical to mx_quantize with those arguments) into `workspace`,
 *               and the product runs on the block-scaled FP4 matrix cores.  Requires
 *               fmt == MX_SCALE_E8M0 and block == 32 (MX_ERR_UNSUPPORTED otherwise).
 *  y          : output, m x n, element type y_type, row stride ld_y >= n.
 *  workspace  : device buffer of at least mx_gemm_workspace_size(...) bytes (may be NULL
 *               when that is 0); owned by the caller, contents on return unspecified.
 * The weight's per-tensor scale is applied to the fp32 accumulator.  Accuracy: for each
 * output, |Y - Y_exact| <= 2e-5 * sum_k |Xhat_k * What_k| before the output rounding
 * (bf16 output adds at most half a bf16 ulp).
 * Errors: as for mx_quantize, plus MX_ERR_INVALID_ARG when ld_y < n or the workspace is
 * smaller than required, and MX_ERR_UNSUPPORTED as above.
 */
mx_status mx_gemm(const void* x, int64_t m, int64_t n, int64_t k, int64_t ld_x,
                  const uint8_t* w_codes, const uint8_t* w_scales, int block, mx_scale_fmt fmt,
                  float tensor_scale, mx_layout layout, mx_act_mode mode, void* y,
                  mx_dtype y_type, int64_t ld_y, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * mx_gemm_static -- mx_gemm without a workspace argument, for callers that cannot allocate
 * device memory around the call: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  The W4A4 activation codes and scales go to a scratch
 * buffer the library owns: a static device array of MX_GEMM_STATIC_SCRATCH_BYTES (32 MiB)
 * that every GPU the library runs on holds until the process ends.  Nothing is allocated or
 * freed by this call.
 *  Arguments, results and errors as mx_gemm (the same kernels run), plus MX_ERR_TOO_LARGE when
 *  mx_gemm_workspace_size(m, n, k, block, mode) exceeds MX_GEMM_STATIC_SCRATCH_BYTES (W4A4 with
 *  m * k above about 6.3e7), checked on the host before anything is launched.  W4A16 calls use
 *  no scratch.
 *  All calls on one GPU share that GPU's buffer: two W4A4 calls that may run at the same time
 *  on one GPU (different streams without ordering between them) race on it and give wrong
 *  results.  Calls ordered on one stream are safe; each call writes all the scratch it reads.
 *  The buffer's device address is looked up on the first call on each device.
 */
#define MX_GEMM_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
mx_status mx_gemm_static(const void* x, int64_t m, int64_t n, int64_t k, int64_t ld_x,
                         const uint8_t* w_codes, const uint8_t* w_scales, int block, mx_scale_fmt fmt,
                         float tensor_scale, mx_layout layout, mx_act_mode mode, void* y,
                         mx_dtype y_type, int64_t ld_y, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* mx_status_string(mx_status s);

#ifdef __cplusplus
}
#endif

#endif /* MX_H */
