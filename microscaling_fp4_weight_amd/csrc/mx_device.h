// mx_device.h -- gfx950 device helpers for MX FP4 block quantization (scale encoding,
// element encoding, dequantization).  Private to libmx.
//
// Method: hotelren.com/news/2192771, article "量化技术演进与微缩量化原理", section 3.1
// item 2 (block scale = FP8(absmax / 6); element = FP4(x / scale)) and item 3 (per-tensor
// scale g multiplies the block scale); gtnt.cn/news/16247 "为什么我们需要4-bit浮点量化",
// section 2.1 (clip, then round).  Rounding is to nearest, ties to the even code (E8M0:
// ties to the larger power of two); scales saturate.
//
// Hardware facts used here (gfx950, checked on the device against an exact CPU reference):
//  * v_cvt_scalef32_pk_fp4_{f32,bf16}(x, scale) returns the E2M1 code nearest to
//    x / 2^floor(log2 scale) (only the scale's exponent is used; denormal scales work),
//    ties to even, saturating at +-6, keeping the sign of zero;
//  * v_cvt_scalef32_pk_{f32,bf16}_fp4(code, scale) returns e(code) * 2^floor(log2 scale)
//    with IEEE overflow to Inf;
//  * fp32 division is correctly rounded and fp32 denormals are kept (kernel float mode 3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_internal.h"

namespace mxk {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

template <int FMT>
struct ScaleFmt;
template <>
struct ScaleFmt<FMT_E4M3> {
    static constexpr int bias = 7;
    static constexpr uint32_t maxcode = 0x7E;  // 448; 0x7F is NaN
};
template <>
struct ScaleFmt<FMT_UE5M3> {
    static constexpr int bias = 15;
    static constexpr uint32_t maxcode = 0xFE;  // 114688; 0xFF is NaN
};

__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// x >> s rounded to nearest, ties to even (1 <= s <= 31, x < 2^31).
__device__ __forceinline__ uint32_t rne_shr32(uint32_t x, uint32_t s)
{
    return (x + ((1u << (s - 1)) - 1u) + ((x >> s) & 1u)) >> s;
}
__device__ __forceinline__ uint64_t rne_shr64(uint64_t x, uint32_t s)
{
    return (x + ((1ull << (s - 1)) - 1ull) + ((x >> s) & 1ull)) >> s;
}

// ---------------------------------------------------------------------------------------
// Block scale encoding.
// ---------------------------------------------------------------------------------------

// E4M3 / UE5M3 code nearest to v >= 0 given in fp32 (3 mantissa bits, subnormals,
// saturation at the largest finite code).  Branch-free: the significand is shifted right by
// 20 (normal target) or more (subnormal target; the shift saturates at 31, which yields 0
// for any 24-bit significand), rounded to nearest even, and added to the exponent field.
template <int FMT>
__device__ __forceinline__ uint32_t fp8_code_f32(float v)
{
    constexpr int bias = ScaleFmt<FMT>::bias;
    const uint32_t b = f2u(v);
    const int e = (int)(b >> 23);                      // 0 for zero / fp32 subnormal
    const uint32_t sig = (b & 0x7FFFFFu) | 0x800000u;  // value = sig * 2^(e - 150)
    const int et = e - 127 + bias;                     // target exponent field if normal
    int sh = 148 - bias - e;                           // subnormal step is 2^(-2-bias)
    sh = sh < 20 ? 20 : (sh > 31 ? 31 : sh);
    const uint32_t base = et > 1 ? (uint32_t)(et - 1) << 3 : 0u;
    const uint32_t code = base + rne_shr32(sig, (uint32_t)sh);  // a carry moves to et + 1
    return code < ScaleFmt<FMT>::maxcode ? code : ScaleFmt<FMT>::maxcode;
}

// Same from an fp64 value (used with a per-tensor scale, where v = a / (6 g) is formed in
// fp64 by a correctly rounded division, which decides every midpoint exactly).
template <int FMT>
__device__ __forceinline__ uint32_t fp8_code_f64(double v)
{
    constexpr int bias = ScaleFmt<FMT>::bias;
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int e = (int)((b >> 52) & 0x7FF);
    if (e == 0) return 0;
    const uint64_t sig = (b & 0xFFFFFFFFFFFFFull) | (1ull << 52);  // value = sig * 2^(e-1075)
    const int et = e - 1023 + bias;
    uint64_t code;
    if (et >= 1) {
        if (et > 40) return ScaleFmt<FMT>::maxcode;
        code = ((uint64_t)(et - 1) << 3) + rne_shr64(sig, 49);
    } else {
        const int sh = 1073 - bias - e;
        code = sh > 63 ? 0ull : rne_shr64(sig, (uint32_t)sh);
    }
    return code < ScaleFmt<FMT>::maxcode ? (uint32_t)code : ScaleFmt<FMT>::maxcode;
}

// E4M3 / UE5M3 byte -> fp32 value (exact).  E4M3 bytes 0x80..0xFE are negative values;
// the quantizer never writes them, but dequantization honours them.
template <int FMT>
__device__ __forceinline__ float fp8_value(uint32_t code)
{
    constexpr int bias = ScaleFmt<FMT>::bias;
    const uint32_t sign = FMT == FMT_E4M3 ? (code & 0x80u) << 24 : 0u;
    const uint32_t E = FMT == FMT_E4M3 ? (code >> 3) & 15u : code >> 3, M = code & 7u;
    const uint32_t normal = ((E - bias + 127) << 23) | (M << 20);
    const uint32_t sub = f2u((float)M * u2f((uint32_t)(127 - 2 - bias) << 23));  // M * 2^(-2-bias)
    return u2f(sign | (E ? normal : sub));
}

// E8M0 byte of the power of two nearest to a / 6 (ties up), from the fp32 bits of
// a = |absmax|: with a = f * 2^ea, f in [1, 2), the midpoint 1.5 * 2^k of a/6 is a = 9 * 2^k,
// so k = ea - 3 + [f >= 1.125] and byte = k + 127, clamped to [0, 254].
__device__ __forceinline__ uint32_t e8m0_code_absmax(uint32_t abits)
{
    const int e = (int)(abits >> 23);
    const int byte = e - 3 + ((abits & 0x7FFFFFu) >= 0x100000u ? 1 : 0);
    return byte < 0 ? 0u : (byte > 254 ? 254u : (uint32_t)byte);
}

// E8M0 byte nearest to v >= 0 given in fp64 (ties up).
__device__ __forceinline__ uint32_t e8m0_code_f64(double v)
{
    if (v == 0.0) return 0;
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int k = (int)((b >> 52) & 0x7FF) - 1023 + ((b & 0xFFFFFFFFFFFFFull) >= (1ull << 51) ? 1 : 0);
    const int byte = k + 127;
    return byte < 0 ? 0u : (byte > 254 ? 254u : (uint32_t)byte);
}

// 2^(byte - 127) as fp32 (byte 0 is the fp32 denormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t byte)
{
    return byte ? u2f(byte << 23) : u2f(0x00400000u);
}
__device__ __forceinline__ double e8m0_value_f64(uint32_t byte)
{
    return __builtin_bit_cast(double, (uint64_t)(byte + 1023 - 127) << 52);
}

// Scale byte of a block from its absmax bits (fp32 bits of a >= 0), for g == 1.
template <int FMT>
__device__ __forceinline__ uint32_t scale_code_g1(uint32_t abits)
{
    if constexpr (FMT == FMT_E8M0) {
        return e8m0_code_absmax(abits);
    } else {
        // fl32(fl64(a) * fl64(1/6)) decides every FP8 midpoint exactly: it equals a midpoint
        // m (5 significant bits) only when a = 6 m, and otherwise stays on a's side of it
        // (|a/6 - m| >= ulp(a)/6 while both roundings move it by less than ulp(a)/8).
        return fp8_code_f32<FMT>((float)((double)u2f(abits) * (1.0 / 6.0)));
    }
}

// Scale byte for a per-tensor scale g (six_g = 6 * g, exact in fp64).
template <int FMT>
__device__ __forceinline__ uint32_t scale_code_g(uint32_t abits, double six_g)
{
    const double v = (double)u2f(abits) / six_g;
    if constexpr (FMT == FMT_E8M0) return e8m0_code_f64(v);
    else return fp8_code_f64<FMT>(v);
}

// Decoded scale as fp32 (exact; E8M0 byte 0 is the fp32 denormal 2^-127).
template <int FMT>
__device__ __forceinline__ float scale_value_f32(uint32_t byte)
{
    if constexpr (FMT == FMT_E8M0) return e8m0_value(byte);
    else return fp8_value<FMT>(byte);
}

// Decoded scale as fp64 (exact).
template <int FMT>
__device__ __forceinline__ double scale_value_f64(uint32_t byte)
{
    if constexpr (FMT == FMT_E8M0) return e8m0_value_f64(byte);
    else return (double)fp8_value<FMT>(byte);
}

// ---------------------------------------------------------------------------------------
// Element encoding with g == 1.
//
// s = m * 2^E with m in {1, 1.125, ..., 1.875}.  The hardware converter divides by 2^E
// exactly, so the element path feeds it x' = x / m, formed as fma(x, chi, x * clo) where
// chi + clo approximates 1/m to ~2^-48: every tie x = t * s lands exactly on t * 2^E and
// every other input stays on its side of the decision points (checked exhaustively over
// all bf16 inputs for all eight m).  E8M0 has m = 1 and feeds x directly.
// ---------------------------------------------------------------------------------------

struct EncG1 {
    float pow2;  // 2^E for the converter
    float chi;   // 1/m, high part (0 when the block scale is 0)
    float clo;   // 1/m, low part
};

// chi = 1/m rounded down to fp32 and clo = fl32(1/m - chi) >= 0, for m = 1 + mi/8.  Both
// parts are non-negative so that x' keeps the sign of x, also for x = -0.
static __constant__ uint32_t kRecipParts[8][2] = {
    {0x3f800000u, 0x00000000u}, {0x3f638e38u, 0x33638e39u}, {0x3f4cccccu, 0x334ccccdu},
    {0x3f3a2e8bu, 0x3322e8bau}, {0x3f2aaaaau, 0x332aaaabu}, {0x3f1d89d8u, 0x331d89d9u},
    {0x3f124924u, 0x33124925u}, {0x3f088888u, 0x33088889u}};

__device__ __forceinline__ void recip_parts(uint32_t mi, float& chi, float& clo)
{
    chi = u2f(kRecipParts[mi][0]);
    clo = u2f(kRecipParts[mi][1]);
}

template <int FMT>
__device__ __forceinline__ EncG1 enc_params_g1(uint32_t byte)
{
    EncG1 p;
    if constexpr (FMT == FMT_E8M0) {
        p.pow2 = e8m0_value(byte);
        p.chi = 1.0f;
        p.clo = 0.0f;
    } else {
        const uint32_t sb = f2u(fp8_value<FMT>(byte));
        float chi, clo;
        recip_parts((sb >> 20) & 7u, chi, clo);
        const bool zero = sb == 0;  // flushed block: x' = +-0 -> codes 0 / 8
        p.pow2 = zero ? 1.0f : u2f(sb & 0x7F800000u);
        p.chi = zero ? 0.0f : chi;
        p.clo = zero ? 0.0f : clo;
    }
    return p;
}

// Two fp32 elements -> one code byte (lo element in the low nibble), g == 1.
template <int FMT>
__device__ __forceinline__ uint32_t enc_pair_g1(float lo, float hi, const EncG1& p, uint32_t old,
                                                int sel_dummy = 0)
{
    (void)sel_dummy;
    if constexpr (FMT != FMT_E8M0) {
        lo = __builtin_fmaf(lo, p.chi, lo * p.clo);
        hi = __builtin_fmaf(hi, p.chi, hi * p.clo);
    }
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, lo, hi, p.pow2, 0) & 0xFFu;
}

// ---------------------------------------------------------------------------------------
// Element encoding with a per-tensor scale g != 1: compare |x| with the exact decision
// points t * s * g (t = 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; formed exactly in fp64).
// Each becomes an fp32 threshold u with  [|x| passes t*s*g]  <=>  [|x| > u]:
//   strict ">" points (ties go down): u = largest fp32 <= t*s*g;
//   ">=" points (ties go up):         u = that value, minus one ulp if it equals t*s*g.
// The code magnitude is the number of thresholds |x| exceeds.
// ---------------------------------------------------------------------------------------

struct EncG {
    uint32_t u[7];  // fp32 bit patterns, compared as unsigned integers with |x|'s bits
};

__device__ __forceinline__ uint32_t rd32_bits(double t)  // t > 0
{
    float f = (float)t;
    uint32_t b = f2u(f);
    if ((double)f > t) b -= 1u;  // also maps +Inf (t beyond FLT_MAX) to FLT_MAX
    return b;
}

// The seven thresholds for a block whose s * g is sg (exact in fp64, > 0).
__device__ __forceinline__ void enc_thresholds(double sg, uint32_t (&u)[7])
{
    const double t[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
    for (int i = 0; i < 7; ++i) {
        const double tt = t[i] * sg;
        uint32_t b = rd32_bits(tt);
        if ((i & 1) && (double)u2f(b) == tt) b -= 1u;  // ">=" points: 0.75, 1.75, 3.5
        u[i] = b;
    }
}

template <int FMT>
__device__ __forceinline__ EncG enc_params_g(uint32_t byte, double g)
{
    EncG p;
    const double s = scale_value_f64<FMT>(byte);
    if (s == 0.0) {
#pragma unroll
        for (int i = 0; i < 7; ++i) p.u[i] = 0x7F800000u;  // nothing exceeds +Inf
        return p;
    }
    enc_thresholds(s * g, p.u);
    return p;
}

// The same thresholds from a per-workgroup table.  Every scale value s of the three formats
// is (1 + j/8) 2^e with j its three mantissa bits as an fp32 number, and while the thresholds
// for s = 1 + j/8 and their 2^e multiples are all normal fp32 numbers, rounding down and the
// one-ulp step of the ">=" points commute with the factor 2^e: the thresholds for s are the
// table's row j with e added to each exponent field.  tab[8 j + i] holds threshold i for
// s = 1 + j/8 (enc_thresholds((1 + j/8) g)); a block outside that range (s = 0, an fp32-subnormal
// s, a table row or a result beyond the normal range) takes enc_params_g.
template <int FMT>
__device__ __forceinline__ EncG enc_params_g_tab(uint32_t byte, double g, const uint32_t* tab)
{
    const uint32_t sb = f2u(scale_value_f32<FMT>(byte));
    const int es = (int)(sb >> 23);
    const uint32_t* row = tab + 8 * ((sb >> 20) & 7u);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(row);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 4);
    const int e = es - 127, e0 = (int)(lo.x >> 23), e6 = (int)(hi.z >> 23);
    if (es == 0 || es >= 255 || e0 < 1 || e0 + e < 1 || e6 > 253 || e6 + e > 254) return enc_params_g<FMT>(byte, g);
    const uint32_t d = (uint32_t)e << 23;
    EncG p;
    p.u[0] = lo.x + d;
    p.u[1] = lo.y + d;
    p.u[2] = lo.z + d;
    p.u[3] = lo.w + d;
    p.u[4] = hi.x + d;
    p.u[5] = hi.y + d;
    p.u[6] = hi.z + d;
    return p;
}

__device__ __forceinline__ uint32_t enc_elem_g(uint32_t xbits32, const EncG& p)
{
    const uint32_t a = xbits32 & 0x7FFFFFFFu;
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 7; ++i) c += (a > p.u[i]) ? 1u : 0u;
    return c | ((xbits32 >> 28) & 8u);
}

// bf16 input: the same decisions on packed 16-bit magnitudes.  A bf16 pattern has a zero
// low half, so |x| > u  <=>  X > (u >> 16) with X the 15-bit magnitude of x.  The thresholds
// are non-decreasing, so the count of those below X comes from a three-step search: X > U3
// gives code bit 2; then U1 or U5 gives bit 1; then U0, U2, U4 or U6 gives bit 0.  Two
// elements are decided at once, one per 16-bit half: X > U is the sign of U - X (both below
// 2^15), spread over its half by an arithmetic shift into a 0 / 0xFFFF mask that selects the
// next threshold with a bitfield insert.
struct EncG16 {
    uint32_t p[7];  // U_i in both halves
};

__device__ __forceinline__ EncG16 enc_params_g16(const EncG& e)
{
    EncG16 q;
#pragma unroll
    for (int i = 0; i < 7; ++i) q.p[i] = (e.u[i] >> 16) * 0x00010001u;
    return q;
}

typedef __attribute__((ext_vector_type(2))) short i16x2;

// 0xFFFF in each half where X > U
__device__ __forceinline__ uint32_t gt_mask16(uint32_t pu, uint32_t x)
{
    const u16x2 d = __builtin_bit_cast(u16x2, pu) - __builtin_bit_cast(u16x2, x);
    uint32_t m = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, d) >> 15);
    // opaque to the optimizer: left alone it rewrites the mask selects below into per-half
    // compares and selects, several times the instruction count
    asm("" : "+v"(m));
    return m;
}

__device__ __forceinline__ uint32_t sel32(uint32_t m, uint32_t a, uint32_t b) { return (m & a) | (~m & b); }

// Codes of the two bf16 elements of word w: element 0 (low half) in bits 0..3, element 1 in
// bits 16..19.
__device__ __forceinline__ uint32_t enc_pair_g16(uint32_t w, const EncG16& q)
{
    const uint32_t x = w & 0x7FFF7FFFu;
    const uint32_t m2 = gt_mask16(q.p[3], x);
    const uint32_t m1 = gt_mask16(sel32(m2, q.p[5], q.p[1]), x);
    const uint32_t t3 = sel32(m1, sel32(m2, q.p[6], q.p[2]), sel32(m2, q.p[4], q.p[0]));
    const uint32_t m0 = gt_mask16(t3, x);
    return (m2 & 0x00040004u) | (m1 & 0x00020002u) | (m0 & 0x00010001u) | ((w >> 12) & 0x00080008u);
}

// Four such results (elements 0..7 of a code word, two per result) -> the code word.
__device__ __forceinline__ uint32_t pack_pairs_g16(uint32_t z0, uint32_t z1, uint32_t z2, uint32_t z3)
{
    uint32_t a = z0 | (z1 << 8);  // nibbles of elements 0, 2 at bits 0, 8; 1, 3 at 16, 24
    uint32_t b = z2 | (z3 << 8);
    a |= a >> 12;                 // elements 0..3 in the low 16 bits
    b |= b >> 12;
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}

// Byte offset of the scale of (row, 32-element block kb) in the tiled scale layout with ks
// 256-k stages per row tile (the layout is described with kTileBytes in mx_internal.h).
__device__ __forceinline__ uint64_t tiled_scale_off(uint32_t row, uint32_t kb, uint32_t ks)
{
    const uint32_t r = row & 255u;
    return ((uint64_t)(row >> 8) * ks + (kb >> 3)) * 2048u + ((r >> 7) << 10) + ((r & 31u) << 5) +
           (((r >> 5) & 3u) << 3) + (kb & 7u);
}

// Byte offset of the scale of (row, 32-element block kb) in the preshuffled layout with cb
// 2048-k chunks per 8-row group (the layout is described with kPreBytes in mx_internal.h).
__device__ __forceinline__ uint64_t pre_scale_off(uint32_t row, uint32_t kb, uint32_t cb)
{
    return ((uint64_t)(row >> 3) * cb + (kb >> 6)) * 512u + ((kb & 63u) << 3) + (row & 7u);
}

// ---------------------------------------------------------------------------------------
// Buffer loads: a resource descriptor carries a byte range, and lanes whose offset is out of
// range read zero without a branch (used for masked rows and k-tails).
// ---------------------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;  // an offset beyond every range this library builds

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t bload32(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload16(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload8(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint64_t bload64(rsrc_t r, uint32_t off)
{
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    return (uint64_t)v.x | ((uint64_t)v.y << 32);
}

// Buffer stores: a lane whose offset is out of range writes nothing.
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore32(rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore64(rsrc_t r, uint32_t off, u32x2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore128(rsrc_t r, uint32_t off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
// The same store marked non-temporal (cache-policy bit 1, "nt"): output that no later work
// in the launch reads, kept from displacing the operand tiles in the L2.
__device__ __forceinline__ void bstore128_nt(rsrc_t r, uint32_t off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 2);
}

// ---------------------------------------------------------------------------------------
// Dequantization helpers.
// ---------------------------------------------------------------------------------------

// For g == 1: e * s = (e * 2^E) * m, both steps exact (m = 0 for a flushed block).
struct DecG1 {
    float pow2;
    float mant;
};

template <int FMT>
__device__ __forceinline__ DecG1 dec_params_g1(uint32_t byte)
{
    DecG1 p;
    if constexpr (FMT == FMT_E8M0) {
        p.pow2 = e8m0_value(byte);
        p.mant = 1.0f;
    } else {
        // s = mant * pow2 with mant = +-(1 + M/8) carrying the sign of s, or mant = +-0
        const uint32_t sb = f2u(fp8_value<FMT>(byte));
        const bool zero = (sb & 0x7FFFFFFFu) == 0;
        p.pow2 = zero ? 1.0f : u2f(sb & 0x7F800000u);
        p.mant = zero ? u2f(sb) : u2f((sb & 0x807FFFFFu) | 0x3F800000u);
    }
    return p;
}

}  // namespace mxk
