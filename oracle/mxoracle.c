/*
 * mxoracle.c -- plain, slow, single-threaded CPU oracle for MX FP4 block
 * quantization, dequantization, the FP4-weight matmul and the error split.
 *
 * TEST INFRASTRUCTURE ONLY: built and called by the test suite, the smoke
 * check and the benchmark's CPU-baseline leg; never by the HIP library, with
 * which it shares no code.  Compile with -O2 and no fast-math (IEEE double,
 * denormals kept).
 *
 * Pages followed (cited below by the key in brackets):
 *  [MXS]  hotelren.com/news/2192771, the article opening with
 *         "量化技术演进与微缩量化原理" (microscaling with FP4 elements and
 *         FP8 E4M3 / UE5M3 block scales).
 *  [FP4L] gtnt.cn/news/16247, "为什么我们需要4-bit浮点量化" (4-bit float
 *         quantization for LLaMA/BERT).
 * The E2M1 value grid {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}, round to
 * nearest even, the E8M0 scale format and the per-tensor fp32 scale are fixed
 * by the benchmark spec rather than by the pages; where the pages are silent
 * or garbled, the reading taken is stated at the function.
 *
 * Method, as the pages give it ([MXS] section 3.1, item 2, quantize_block):
 *   absmax of the block -> scale = FP8(absmax / 6) -> block / scale -> FP4,
 * with the per-tensor factor of [MXS] section 3.1 item 3 (value = FP4 element
 * x FP8 block scale x per-tensor scale) and the clip-then-round of [FP4L]
 * section 2.1.  Both roundings are "nearest representable value": this file
 * decides them exactly by comparing the numerator with the denominator times
 * each midpoint between neighbouring representable values, all in double,
 * where every such product is exact (asserted at run time with fma).
 */
#include "mxoracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* E2M1 element: [sign 1][exponent 2][mantissa 1] ([FP4L] section 1; [MXS]
 * section 1 names it E2M1 with magnitudes 0.5..6).  Exponent bias 1; an
 * exponent field of 0 is subnormal, value = mantissa/2.  No infinities or
 * NaNs (the "+-inf" of [MXS] section 1 does not fit a 4-bit grid that reaches
 * 6; the task's grid has none). */
double ox_e2m1_value(unsigned code)
{
    unsigned sign = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
    return sign ? -mag : mag;
}

/* Scale byte -> value.
 *  E4M3 ([MXS] section 3.1 item 1, "standard E4M3"; taken as OCP E4M3FN):
 *    [sign 1][exp 4][man 3], bias 7, exp 0 subnormal, 0x7F/0xFF NaN.
 *  UE5M3 ([MXS] section 3.1 item 1: the sign bit is used as a fifth exponent
 *    bit, 3 mantissa bits): unsigned [exp 5][man 3]; the bias is not given on
 *    the page, taken as 15 (IEEE-style), exp 0 subnormal, 0xFF NaN.
 *  E8M0: unsigned power of two 2^(byte-127), 0xFF NaN, no zero. */
double ox_scale_value(unsigned byte, int fmt)
{
    byte &= 0xFFu;
    if (fmt == OX_E4M3) {
        unsigned sign = byte >> 7, e = (byte >> 3) & 15u, m = byte & 7u;
        double v;
        if (e == 15u && m == 7u) return NAN;
        v = (e == 0) ? ldexp((double)m / 8.0, 1 - 7) : ldexp(1.0 + m / 8.0, (int)e - 7);
        return sign ? -v : v;
    }
    if (fmt == OX_UE5M3) {
        unsigned e = byte >> 3, m = byte & 7u;
        if (byte == 0xFFu) return NAN;
        return (e == 0) ? ldexp((double)m / 8.0, 1 - 15) : ldexp(1.0 + m / 8.0, (int)e - 15);
    }
    if (fmt == OX_E8M0) {
        if (byte == 0xFFu) return NAN;
        return ldexp(1.0, (int)byte - 127);
    }
    return NAN;
}

/* Ascending table of the non-negative finite values of a format, with the
 * code of each. */
typedef struct {
    int n;
    double v[256];
    unsigned code[256];
} vtable;

static vtable g_e2m1, g_scale[3];
static int g_ready = 0;

static void build_tables(void)
{
    int f;
    unsigned c;
    if (g_ready) return;
    g_e2m1.n = 0;
    for (c = 0; c < 8; ++c) {
        g_e2m1.v[g_e2m1.n] = ox_e2m1_value(c);
        g_e2m1.code[g_e2m1.n++] = c;
    }
    for (f = 0; f < 3; ++f) {
        unsigned last = (f == OX_E4M3) ? 0x7Eu : 0xFEu; /* largest finite, sign clear */
        g_scale[f].n = 0;
        for (c = 0; c <= last; ++c) {
            g_scale[f].v[g_scale[f].n] = ox_scale_value(c, f);
            g_scale[f].code[g_scale[f].n++] = c;
        }
    }
    /* the tables must be strictly ascending for the search below */
    for (f = 0; f < 4; ++f) {
        const vtable* t = (f < 3) ? &g_scale[f] : &g_e2m1;
        int i;
        for (i = 1; i < t->n; ++i)
            if (!(t->v[i] > t->v[i - 1])) abort();
    }
    g_ready = 1;
}

/* Product that must be exact in double (operands with few significant bits). */
static double exact_mul(double a, double b)
{
    double p = a * b;
    if (fma(a, b, -p) != 0.0) abort();
    return p;
}

/* Index i of the table value nearest to the exact real num/den (num >= 0,
 * den > 0).  Values below the smallest entry go to it; values above the
 * largest saturate to it (the clip of [FP4L] section 2.1 for elements; the
 * saturating reading for scales).  A tie goes to the larger value when tie_up
 * is set (E8M0), else to the even code (round to nearest even). */
static int nearest(const vtable* t, double num, double den, int tie_up)
{
    int lo = 0, hi = t->n - 1;
    double thr;
    if (num <= exact_mul(den, t->v[0])) return 0;
    if (num >= exact_mul(den, t->v[hi])) return hi;
    while (hi - lo > 1) { /* keep den*v[lo] <= num < den*v[hi] */
        int mid = (lo + hi) / 2;
        if (exact_mul(den, t->v[mid]) <= num) lo = mid; else hi = mid;
    }
    thr = exact_mul(den, 0.5 * (t->v[lo] + t->v[hi])); /* den x midpoint */
    if (num < thr) return lo;
    if (num > thr) return hi;
    if (tie_up) return hi;
    return (t->code[lo] & 1u) ? hi : lo;
}

/* [MXS] section 3.1 item 2: scale = FP8(absmax / 6.0), and item 3: the
 * per-tensor scale multiplies the block scale, so the block scale is the FP8
 * value nearest to absmax / (6 g).  6 is the largest E2M1 magnitude. */
unsigned ox_scale_byte(double a, double g, int fmt)
{
    build_tables();
    if (fmt < 0 || fmt > 2) abort();
    return g_scale[fmt].code[nearest(&g_scale[fmt], fabs(a), exact_mul(6.0, g), fmt == OX_E8M0)];
}

/* [MXS] section 3.1 item 2: element / scale -> FP4, and [FP4L] section 2.1:
 * round(clip(x / scale)).  With the per-tensor scale the divisor is s*g.  A
 * zero scale flushes the block to zero ([MXS] section 2.2, third error
 * source).  The sign bit of x is kept, also on zero codes. */
unsigned ox_elem_code(double x, double s, double g)
{
    unsigned sign = signbit(x) ? 8u : 0u;
    build_tables();
    if (s == 0.0) return sign;
    return sign | g_e2m1.code[nearest(&g_e2m1, fabs(x), exact_mul(s, g), 0)];
}

/* ------------------------------------------------------------------------ */
/* Element access                                                            */
/* ------------------------------------------------------------------------ */

static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double load_elem(const void* x, int xtype, int64_t idx)
{
    if (xtype == OX_BF16) return bf16_value(((const uint16_t*)x)[idx]);
    return (double)((const float*)x)[idx];
}

uint16_t ox_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u); /* NaN stays NaN */
    u += 0x7FFFu + ((u >> 16) & 1u); /* nearest, ties to even */
    return (uint16_t)(u >> 16);
}

static int valid_block(int block)
{
    return block == 4 || block == 8 || block == 16 || block == 32 || block == 64 ||
           block == 128 || block == 256;
}

/* ------------------------------------------------------------------------ */
/* Quantize / dequantize                                                     */
/* ------------------------------------------------------------------------ */

int ox_quantize(const void* x, int xtype, int64_t rows, int64_t k, int64_t ldx,
                int block, int fmt, float g, uint8_t* codes, uint8_t* scales)
{
    int64_t r, b, i;
    int64_t nb = (block > 0) ? k / block : 0;
    if (!x || !codes || !scales || rows < 0 || k < 0 || ldx < k || !valid_block(block) ||
        k % block != 0 || fmt < 0 || fmt > 2 || !(g > 0.0f) || isinf(g))
        return -1;
    build_tables();
    memset(codes, 0, (size_t)(rows * (k / 2)));
    for (r = 0; r < rows; ++r) {
        for (b = 0; b < nb; ++b) {
            int64_t base = r * ldx + b * block;
            double a = 0.0, s;
            unsigned sb;
            for (i = 0; i < block; ++i) { /* block absmax */
                double v = fabs(load_elem(x, xtype, base + i));
                if (v > a) a = v;
            }
            sb = ox_scale_byte(a, (double)g, fmt);
            s = ox_scale_value(sb, fmt);
            scales[r * nb + b] = (uint8_t)sb;
            for (i = 0; i < block; ++i) {
                int64_t col = b * block + i;
                unsigned c = ox_elem_code(load_elem(x, xtype, base + i), s, (double)g);
                /* two codes per byte, even element in the low nibble ([FP4L] section 4.3) */
                codes[r * (k / 2) + col / 2] |= (uint8_t)(c << (4 * (col & 1)));
            }
        }
    }
    return 0;
}

/* Dequantized value as an exact double: e(c) * s * g ([MXS] section 3.1 item
 * 3).  e has <= 2 significant bits, s <= 4, g <= 24, so the product is exact. */
static double dq_exact(const uint8_t* codes, const uint8_t* scales, int64_t r, int64_t col,
                       int64_t k, int block, int fmt, double g)
{
    unsigned byte = codes[r * (k / 2) + col / 2];
    unsigned c = (col & 1) ? (byte >> 4) : (byte & 15u);
    double s = ox_scale_value(scales[r * (k / block) + col / block], fmt);
    return ox_e2m1_value(c) * s * g;
}

/* Output: one fp32 rounding of e*s*g; bf16 output is the nearest-even bf16 of
 * that fp32 value.  (With g = 1 both are exact.) */
int ox_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                  int block, int fmt, float g, void* y, int ytype, int64_t ldy)
{
    int64_t r, c;
    if (!codes || !scales || !y || rows < 0 || k < 0 || ldy < k || !valid_block(block) ||
        k % block != 0 || fmt < 0 || fmt > 2 || !(g > 0.0f) || isinf(g))
        return -1;
    for (r = 0; r < rows; ++r)
        for (c = 0; c < k; ++c) {
            float f = (float)dq_exact(codes, scales, r, c, k, block, fmt, (double)g);
            if (ytype == OX_BF16) ((uint16_t*)y)[r * ldy + c] = ox_f32_to_bf16(f);
            else ((float*)y)[r * ldy + c] = f;
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Matmul: dequantize, then multiply ([FP4L] section 3.1, dequantize_matmul) */
/* ------------------------------------------------------------------------ */

int ox_gemm(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
            const uint8_t* wcodes, const uint8_t* wscales, int64_t n,
            int block, int fmt, float g, int mode,
            const int64_t* mrows, int64_t nm, const int64_t* ncols, int64_t nn,
            double* y, double* aabs)
{
    int64_t i, j, kk;
    double *xh, *wh;
    uint8_t *xc = NULL, *xs = NULL;
    if (!x || !wcodes || !wscales || !mrows || !ncols || !y || !aabs || m < 0 || n < 0 ||
        k <= 0 || ldx < k || !valid_block(block) || k % block != 0 || fmt < 0 || fmt > 2 ||
        !(g > 0.0f) || isinf(g) || (mode != OX_A16 && mode != OX_A4))
        return -1;
    if (mode == OX_A4 && k % 32 != 0) return -1;
    for (i = 0; i < nm; ++i)
        if (mrows[i] < 0 || mrows[i] >= m) return -1;
    for (j = 0; j < nn; ++j)
        if (ncols[j] < 0 || ncols[j] >= n) return -1;
    /* the selected rows of X as values (A4: after their MX quantization), then one
     * dequantized weight row per selected column */
    xh = (double*)malloc(sizeof(double) * (size_t)(nm * k + k));
    if (!xh) return -1;
    wh = xh + nm * k;
    if (mode == OX_A4) {
        xc = (uint8_t*)malloc((size_t)k / 2);
        xs = (uint8_t*)malloc((size_t)k / 32);
    }
    for (i = 0; i < nm; ++i) {
        const uint16_t* xr = x + mrows[i] * ldx;
        if (mode == OX_A16) {
            for (kk = 0; kk < k; ++kk) xh[i * k + kk] = bf16_value(xr[kk]);
        } else { /* activations MX-quantized: block 32, E8M0, g = 1 */
            ox_quantize(xr, OX_BF16, 1, k, k, 32, OX_E8M0, 1.0f, xc, xs);
            for (kk = 0; kk < k; ++kk) xh[i * k + kk] = dq_exact(xc, xs, 0, kk, k, 32, OX_E8M0, 1.0);
        }
    }
    for (j = 0; j < nn; ++j) {
        for (kk = 0; kk < k; ++kk) wh[kk] = dq_exact(wcodes, wscales, ncols[j], kk, k, block, fmt, (double)g);
        for (i = 0; i < nm; ++i) {
            double acc = 0.0, accabs = 0.0;
            for (kk = 0; kk < k; ++kk) {
                double p = xh[i * k + kk] * wh[kk];
                acc += p;
                accabs += fabs(p);
            }
            y[i * nn + j] = acc;
            aabs[i * nn + j] = accabs;
        }
    }
    free(xh);
    free(xc);
    free(xs);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Error split ([MXS] section 2.2)                                           */
/* ------------------------------------------------------------------------ */

/* Per element error err = xhat - x in the input's units, xhat = e*s*g exact.
 *  MSE_zero: elements of blocks whose scale is 0 (the whole block is zero).
 *  MSE_max:  the block's maximum element (lowest index among equal |x|) in
 *            blocks with a non-zero scale -- its error comes only from the
 *            FP8 rounding of the scale when it is coded as +-6.
 *  MSE_elem: every other element of blocks with a non-zero scale.
 * Each is a sum over the tensor divided by the element count, so the three
 * add up to the total mean squared error. */
int ox_mse_split(const void* x, int xtype, int64_t rows, int64_t k, int64_t ldx,
                 int block, int fmt, float g, double out[7])
{
    int64_t r, b, i, n = rows * k, nb = (block > 0) ? k / block : 0;
    double se = 0.0, sm = 0.0, sz = 0.0, st = 0.0, nzero = 0.0, nnot6 = 0.0;
    if (!x || !out || rows < 0 || k < 0 || ldx < k || !valid_block(block) || k % block != 0 ||
        fmt < 0 || fmt > 2 || !(g > 0.0f) || isinf(g))
        return -1;
    build_tables();
    for (r = 0; r < rows; ++r)
        for (b = 0; b < nb; ++b) {
            int64_t base = r * ldx + b * block, imax = 0;
            double a = -1.0, s;
            for (i = 0; i < block; ++i) {
                double v = fabs(load_elem(x, xtype, base + i));
                if (v > a) { a = v; imax = i; }
            }
            s = ox_scale_value(ox_scale_byte(a, (double)g, fmt), fmt);
            if (s == 0.0) nzero += 1.0;
            for (i = 0; i < block; ++i) {
                double xv = load_elem(x, xtype, base + i);
                unsigned c = ox_elem_code(xv, s, (double)g);
                double err = ox_e2m1_value(c) * s * (double)g - xv, e2 = err * err;
                st += e2;
                if (s == 0.0) sz += e2;
                else if (i == imax) {
                    sm += e2;
                    if ((c & 7u) != 7u) nnot6 += 1.0;
                } else se += e2;
            }
        }
    out[0] = n ? se / (double)n : 0.0;
    out[1] = n ? sm / (double)n : 0.0;
    out[2] = n ? sz / (double)n : 0.0;
    out[3] = n ? st / (double)n : 0.0;
    out[4] = (double)(rows * nb);
    out[5] = nzero;
    out[6] = nnot6;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Batch forms of the two roundings (loops over the scalar functions, for    */
/* exhaustive checks).                                                       */
/* ------------------------------------------------------------------------ */

void ox_scale_bytes(const double* a, int64_t n, double g, int fmt, uint8_t* out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)ox_scale_byte(a[i], g, fmt);
}

void ox_elem_codes(const double* x, int64_t n, double s, double g, uint8_t* out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)ox_elem_code(x[i], s, g);
}

/* ------------------------------------------------------------------------ */
/* FP8 weight fallback ([MXS] section 5.3 item 1: a layer whose weights have  */
/* sigma < 1e-4 loses everything to FP4; the remedy named there is FP8; and   */
/* section 6 item 1: key layers kept in FP8).  Elements are E4M3 (the OCP     */
/* E4M3FN byte, largest magnitude 448) in the same blocks and under the same  */
/* three scale formats; 448 takes the place of 6 in the scale rule.           */
/* ------------------------------------------------------------------------ */

/* Decoded E4M3 element byte, sign included (NaN for 0x7F / 0xFF). */
double ox_e4m3_value(unsigned code)
{
    return ox_scale_value(code, OX_E4M3);
}

/* Block scale: the scale-format value nearest to the exact real a / (448 g). */
unsigned ox_scale_byte_fp8(double a, double g, int fmt)
{
    build_tables();
    if (fmt < 0 || fmt > 2) abort();
    return g_scale[fmt].code[nearest(&g_scale[fmt], fabs(a), exact_mul(448.0, g), fmt == OX_E8M0)];
}

/* Element byte: the E4M3 value nearest to |x| / (s g), clipped at 448, ties
 * to the even code, with the sign bit of x; a zero scale flushes to +-0. */
unsigned ox_elem_code_fp8(double x, double s, double g)
{
    unsigned sign = signbit(x) ? 0x80u : 0u;
    build_tables();
    if (s == 0.0) return sign;
    return sign | g_scale[OX_E4M3].code[nearest(&g_scale[OX_E4M3], fabs(x), exact_mul(s, g), 0)];
}

int ox_quantize_fp8(const void* x, int xtype, int64_t rows, int64_t k, int64_t ldx,
                    int block, int fmt, float g, uint8_t* codes, uint8_t* scales)
{
    int64_t r, b, i;
    const int64_t nb = (block > 0) ? k / block : 0;
    if (!x || !codes || !scales || rows < 0 || k < 0 || ldx < k || !valid_block(block) ||
        k % block != 0 || fmt < 0 || fmt > 2 || !(g > 0.0f) || isinf(g))
        return -1;
    for (r = 0; r < rows; ++r)
        for (b = 0; b < nb; ++b) {
            const int64_t base = r * ldx + b * block;
            double a = 0.0, s;
            unsigned sb;
            for (i = 0; i < block; ++i) {
                double v = fabs(load_elem(x, xtype, base + i));
                if (v > a) a = v;
            }
            sb = ox_scale_byte_fp8(a, (double)g, fmt);
            s = ox_scale_value(sb, fmt);
            scales[r * nb + b] = (uint8_t)sb;
            for (i = 0; i < block; ++i)
                codes[r * k + b * block + i] = (uint8_t)ox_elem_code_fp8(load_elem(x, xtype, base + i), s, (double)g);
        }
    return 0;
}

/* e(c) * s * g, exact in double (e has 4 significant bits, s 4, g 24). */
static double dq_exact_fp8(const uint8_t* codes, const uint8_t* scales, int64_t r, int64_t col,
                           int64_t k, int block, int fmt, double g)
{
    double e = ox_e4m3_value(codes[r * k + col]);
    double s = ox_scale_value(scales[r * (k / block) + col / block], fmt);
    return e * s * g;
}

int ox_dequantize_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                      int block, int fmt, float g, void* y, int ytype, int64_t ldy)
{
    int64_t r, c;
    if (!codes || !scales || !y || rows < 0 || k < 0 || ldy < k || !valid_block(block) ||
        k % block != 0 || fmt < 0 || fmt > 2 || !(g > 0.0f) || isinf(g))
        return -1;
    for (r = 0; r < rows; ++r)
        for (c = 0; c < k; ++c) {
            float f = (float)dq_exact_fp8(codes, scales, r, c, k, block, fmt, (double)g);
            if (ytype == OX_BF16) ((uint16_t*)y)[r * ldy + c] = ox_f32_to_bf16(f);
            else ((float*)y)[r * ldy + c] = f;
        }
    return 0;
}

/* Y = X . dequant(W8)^T with bf16 X, fp64 sums in k order, as ox_gemm (A16). */
int ox_gemm_fp8(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                const uint8_t* wcodes, const uint8_t* wscales, int64_t n,
                int block, int fmt, float g,
                const int64_t* mrows, int64_t nm, const int64_t* ncols, int64_t nn,
                double* y, double* aabs)
{
    int64_t i, j, kk;
    double* wh;
    if (!x || !wcodes || !wscales || !mrows || !ncols || !y || !aabs || m < 0 || n < 0 ||
        k <= 0 || ldx < k || !valid_block(block) || k % block != 0 || fmt < 0 || fmt > 2 ||
        !(g > 0.0f) || isinf(g))
        return -1;
    for (i = 0; i < nm; ++i)
        if (mrows[i] < 0 || mrows[i] >= m) return -1;
    for (j = 0; j < nn; ++j)
        if (ncols[j] < 0 || ncols[j] >= n) return -1;
    wh = (double*)malloc(sizeof(double) * (size_t)k);  /* one dequantized weight row */
    if (!wh) return -1;
    for (j = 0; j < nn; ++j) {
        for (kk = 0; kk < k; ++kk) wh[kk] = dq_exact_fp8(wcodes, wscales, ncols[j], kk, k, block, fmt, (double)g);
        for (i = 0; i < nm; ++i) {
            const uint16_t* xr = x + mrows[i] * ldx;
            double acc = 0.0, accabs = 0.0;
            for (kk = 0; kk < k; ++kk) {
                double p = bf16_value(xr[kk]) * wh[kk];
                acc += p;
                accabs += fabs(p);
            }
            y[i * nn + j] = acc;
            aabs[i * nn + j] = accabs;
        }
    }
    free(wh);
    return 0;
}

/* Batch forms for exhaustive checks. */
void ox_scale_bytes_fp8(const double* a, int64_t n, double g, int fmt, uint8_t* out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)ox_scale_byte_fp8(a[i], g, fmt);
}

void ox_elem_codes_fp8(const double* x, int64_t n, double s, double g, uint8_t* out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)ox_elem_code_fp8(x[i], s, g);
}
