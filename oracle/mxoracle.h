/*
 * mxoracle.h -- CPU oracle for MX FP4 block quantization and the FP4-weight matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  This code exists to check the HIP library.  Only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * build, load or call it.  It shares no source, header, table or constant with
 * the HIP library, and the library never calls it.
 *
 * Everything here is plain single-threaded C with IEEE double arithmetic (no
 * fast-math, denormals kept).  See mxoracle.c for the page citations.
 */
#ifndef MXORACLE_H
#define MXORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Scale formats and element dtypes (the oracle's own numbering). */
enum { OX_E4M3 = 0, OX_UE5M3 = 1, OX_E8M0 = 2 };
enum { OX_F32 = 0, OX_BF16 = 1 };
enum { OX_A16 = 0, OX_A4 = 1 };

/* Decoded value of a 4-bit E2M1 code (0..15), sign included. */
double ox_e2m1_value(unsigned code);

/* Decoded value of a scale byte in format fmt; NaN for the format's NaN byte. */
double ox_scale_value(unsigned byte, int fmt);

/* Scale byte for a block with absolute maximum a under per-tensor scale g:
 * the representable value nearest to the exact real a/(6g). */
unsigned ox_scale_byte(double a, double g, int fmt);

/* 4-bit code of element x in a block whose decoded scale is s (per-tensor g). */
unsigned ox_elem_code(double x, double s, double g);

/* Quantize a rows x k tensor (row stride ldx elements) in blocks of `block`
 * consecutive elements along k.  codes: rows x k/2 bytes (even element in the
 * low nibble); scales: rows x k/block bytes.  Returns 0, or -1 on bad args. */
int ox_quantize(const void* x, int xtype, int64_t rows, int64_t k, int64_t ldx,
                int block, int fmt, float g, uint8_t* codes, uint8_t* scales);

/* Dequantize to fp32 (ytype OX_F32) or bf16 (OX_BF16, raw uint16 bits). */
int ox_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                  int block, int fmt, float g, void* y, int ytype, int64_t ldy);

/* Batch forms: out[i] = ox_scale_byte(a[i], g, fmt) / ox_elem_code(x[i], s, g). */
void ox_scale_bytes(const double* a, int64_t n, double g, int fmt, uint8_t* out);
void ox_elem_codes(const double* x, int64_t n, double s, double g, uint8_t* out);

/* fp32 -> bf16 bits, round to nearest even. */
uint16_t ox_f32_to_bf16(float f);

/* Y[i][j] = sum_k Xhat[mi][k] * What[nj][k] in fp64 (sequential k), and
 * A[i][j] = sum_k |Xhat*What|, for mi = mrows[i], nj = ncols[j].
 * x: bf16 bits, m x k with row stride ldx.  mode OX_A16: Xhat = X;
 * OX_A4: Xhat = dequant(quantize(X, block 32, E8M0, g = 1)).
 * y, aabs: nm x nn, row-major. */
int ox_gemm(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
            const uint8_t* wcodes, const uint8_t* wscales, int64_t n,
            int block, int fmt, float g, int mode,
            const int64_t* mrows, int64_t nm, const int64_t* ncols, int64_t nn,
            double* y, double* aabs);

/* Error split of quantize->dequantize against the exact input.
 * out[0] MSE_elem, out[1] MSE_max, out[2] MSE_zero, out[3] MSE_total,
 * out[4] number of blocks, out[5] blocks with scale 0,
 * out[6] non-flushed blocks whose maximum element is not coded as +-6. */
int ox_mse_split(const void* x, int xtype, int64_t rows, int64_t k, int64_t ldx,
                 int block, int fmt, float g, double out[7]);

/* FP8 weight fallback: E4M3 element bytes (OCP E4M3FN, largest magnitude 448)
 * in blocks of `block` along k under the same scale formats; the block scale is
 * the value nearest to a / (448 g).  codes: rows x k bytes (one per element). */
double ox_e4m3_value(unsigned code);
unsigned ox_scale_byte_fp8(double a, double g, int fmt);
unsigned ox_elem_code_fp8(double x, double s, double g);
int ox_quantize_fp8(const void* x, int xtype, int64_t rows, int64_t k, int64_t ldx,
                    int block, int fmt, float g, uint8_t* codes, uint8_t* scales);
int ox_dequantize_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                      int block, int fmt, float g, void* y, int ytype, int64_t ldy);
int ox_gemm_fp8(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                const uint8_t* wcodes, const uint8_t* wscales, int64_t n,
                int block, int fmt, float g,
                const int64_t* mrows, int64_t nm, const int64_t* ncols, int64_t nn,
                double* y, double* aabs);
void ox_scale_bytes_fp8(const double* a, int64_t n, double g, int fmt, uint8_t* out);
void ox_elem_codes_fp8(const double* x, int64_t n, double s, double g, uint8_t* out);

#ifdef __cplusplus
}
#endif
#endif
