// mx_fp8.hip -- the FP8 weight fallback: E4M3 elements in the MX block structure.
//
// hotelren.com/news/2192771, article "量化技术演进与微缩量化原理": section 5.3 item 1 (a layer
// whose weights have a standard deviation below 1e-4 comes out of FP4 quantization as zeros;
// the remedy named there is FP8) and section 6 item 1 (key layers kept in FP8).  The format
// keeps everything of the FP4 path but the element: per block of `block` elements along k a
// scale in one of the three scale formats, the value nearest to absmax / (448 g) (448 being
// the largest E4M3 magnitude, where FP4 divides by 6), and one E4M3 byte per element, the
// value nearest to |x| / (s g), clipped at 448, ties to the even code, sign kept; a zero scale
// flushes the block to +-0.
//
// Element rounding is exact: a quotient estimate q = |x| * fl(1/(s g)) in fp64 picks a code,
// which an exact comparison of |x| with the neighbouring decision points (midpoint * s * g,
// at most 33 significant bits, exact in fp64) corrects by at most one step.
//
// The W8A16 product Y = X . dequant(W8)^T runs on bf16 matrix cores: e * s (at most 8
// significant bits) is exact in bf16 for |e * s| >= 2^-133, g multiplies the fp32 sums.
#include <cmath>

#include "mx_device.h"
#include "mx_internal.h"
#include "mx_wdeq.h"

namespace mxk {
namespace f8 {

constexpr int THREADS = 256;

// E4M3 magnitude of code c in 0..127 as an exact double (127 reads as 480, the pattern's
// value were it not NaN; callers treat 0x7F separately).
__device__ __forceinline__ double mag(uint32_t c)
{
    const uint32_t e = c >> 3, m = c & 7u;
    const double p = __builtin_bit_cast(double, (uint64_t)(1023 + (int)e - 10) << 52);  // 2^(e-10)
    return e == 0 ? (double)c * 0x1p-9 : (double)(8u + m) * p;
}

// E4M3 magnitude code (0..126) nearest to a / S: ties to even, clipped at 448.  a >= 0;
// S > 0 is exact; rS is fl(1/S).
__device__ __forceinline__ uint32_t code_of(double a, double S, double rS)
{
    const double q = a * rS;
    uint32_t c;
    if (q >= 448.0) {
        c = 126;
    } else if (q < 0x1p-6) {
        c = (uint32_t)__builtin_rint(q * 512.0);  // subnormal codes 0..7 (8 is 2^-6)
    } else {
        const int e = (int)((__builtin_bit_cast(uint64_t, q) >> 52) & 0x7FF) - 1023;  // -6 .. 8
        const double t = q * __builtin_bit_cast(double, (uint64_t)(1023 + 3 - e) << 52);  // [8, 16)
        const int cc = (e + 7) * 8 + (int)__builtin_rint(t) - 8;
        c = cc > 126 ? 126u : (uint32_t)cc;
    }
    if (c < 126) {
        const double up = (mag(c) + mag(c + 1)) * 0.5 * S;
        if (a > up || (a == up && (c & 1u))) ++c;
    }
    if (c > 0) {
        const double dn = (mag(c - 1) + mag(c)) * 0.5 * S;
        if (a < dn || (a == dn && (c & 1u))) --c;
    }
    return c;
}

struct Blk {
    double S, rS;  // s * g and its reciprocal (S == 0: flushed)
};

template <int FMT>
__device__ __forceinline__ Blk block_params(uint32_t sbyte, double g)
{
    Blk p;
    p.S = scale_value_f64<FMT>(sbyte) * g;
    p.rS = p.S != 0.0 ? 1.0 / p.S : 0.0;
    return p;
}

// E4M3 byte of an element with fp32 bit pattern xb
__device__ __forceinline__ uint32_t elem_byte(uint32_t xb, const Blk& p)
{
    const uint32_t sign = (xb >> 24) & 0x80u;
    if (p.S == 0.0) return sign;
    return sign | code_of((double)u2f(xb & 0x7FFFFFFFu), p.S, p.rS);
}

// ---------------------------------------------------------------------------------------
// quantize, fast path: one lane per 8 consecutive elements (16-byte bf16 or 2 x 16-byte fp32
// loads, 8 code bytes stored); blocks of 4 are two per lane, blocks of 8 one per lane, larger
// ones span BLOCK / 8 adjacent lanes that combine their absmax with lane shuffles.
// ---------------------------------------------------------------------------------------
// bf16 input, g == 1: the hardware converter (divides by the power of two of its scale
// argument, rounds to nearest even, keeps the sign; quotients past 464 it turns into NaN
// rather than 448, so the input is first clamped to +-448 times that power of two) after the
// exact pre-scale by 1/m of the FP4 path for E4M3 / UE5M3 scale mantissas m: for bf16 inputs the
// pre-scaled value lies on the same side of every decision point as the exact quotient and
// lands exactly on a tie when the quotient is one (the same argument as for the E2M1 grid,
// whose decision points are a subset of finer ones; checked by the parity tests around
// every decision point of every scale mantissa).
typedef __attribute__((ext_vector_type(2))) short i16x2;

template <int FMT, int SEL>
__device__ __forceinline__ i16x2 enc_fp8_pair(i16x2 old, uint32_t wd, const EncG1& p, float lim)
{
    float lo = u2f(wd << 16), hi = u2f(wd & 0xFFFF0000u);
    if constexpr (FMT != FMT_E8M0) {
        lo = __builtin_fmaf(lo, p.chi, lo * p.clo);
        hi = __builtin_fmaf(hi, p.chi, hi * p.clo);
    }
    lo = __builtin_amdgcn_fmed3f(lo, -lim, lim);
    hi = __builtin_amdgcn_fmed3f(hi, -lim, lim);
    return __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, lo, hi, p.pow2, SEL != 0);
}

template <int BLOCK, int FMT, bool BF16, bool HW>
__global__ __launch_bounds__(THREADS) void quantize_fp8_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                               FastDiv upr_div, uint32_t upr, uint32_t total,
                                                               double g, uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales, int64_t k)
{
    constexpr int NB = BLOCK < 8 ? 8 / BLOCK : 1;
    constexpr int EPB = 8 / NB;
    constexpr int LANES = BLOCK > 8 ? BLOCK / 8 : 1;
    const uint32_t u = blockIdx.x * THREADS + threadIdx.x;
    const bool act = u < total;
    const uint32_t row = act ? upr_div.div(u) : 0u;
    const uint32_t c8 = act ? u - row * upr : 0u;

    uint32_t xb[8];
    if (act) {
        const u32x4* p = reinterpret_cast<const u32x4*>(x + (int64_t)row * ldx_bytes + (int64_t)c8 * (BF16 ? 16 : 32));
        if constexpr (BF16) {
            const u32x4 v = p[0];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xb[2 * j] = w[j] << 16;
                xb[2 * j + 1] = w[j] & 0xFFFF0000u;
            }
        } else {
            const u32x4 v0 = p[0], v1 = p[1];
            const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) xb[j] = w[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xb[j] = 0u;
    }

    uint32_t amax[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < EPB; ++e) {
            const uint32_t a = xb[b * EPB + e] & 0x7FFFFFFFu;
            m = a > m ? a : m;
        }
        amax[b] = m;
    }
    if constexpr (LANES > 1) {
#pragma unroll
        for (int off = 1; off < LANES; off <<= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)amax[0], off);
            amax[0] = o > amax[0] ? o : amax[0];
        }
    }

    uint32_t sb[NB];
    u32x2 cv;
    if constexpr (HW) {  // bf16 input, g == 1
        i16x2 h0 = {0, 0}, h1 = {0, 0};
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            sb[b] = scale_code_g<FMT>(amax[b], 448.0);
            const EncG1 p = enc_params_g1<FMT>(sb[b]);
            const float lim = 448.0f * p.pow2;  // 448 * 2^E (exact, also for 2^-127)
#pragma unroll
            for (int pr = 0; pr < EPB / 2; ++pr) {
                const int j = b * (EPB / 2) + pr;  // element pair j = elements 2j, 2j+1
                const uint32_t wd = (xb[2 * j] >> 16) | (xb[2 * j + 1] & 0xFFFF0000u);
                switch (j) {
                    case 0: h0 = enc_fp8_pair<FMT, 0>(h0, wd, p, lim); break;
                    case 1: h0 = enc_fp8_pair<FMT, 1>(h0, wd, p, lim); break;
                    case 2: h1 = enc_fp8_pair<FMT, 0>(h1, wd, p, lim); break;
                    default: h1 = enc_fp8_pair<FMT, 1>(h1, wd, p, lim); break;
                }
            }
        }
        cv = u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
    } else {
        uint32_t cb[8];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            sb[b] = scale_code_g<FMT>(amax[b], 448.0 * g);
            const Blk p = block_params<FMT>(sb[b], g);
#pragma unroll
            for (int e = 0; e < EPB; ++e) cb[b * EPB + e] = elem_byte(xb[b * EPB + e], p);
        }
        cv = u32x2{cb[0] | (cb[1] << 8) | (cb[2] << 16) | (cb[3] << 24),
                   cb[4] | (cb[5] << 8) | (cb[6] << 16) | (cb[7] << 24)};
    }
    if (!act) return;
    *reinterpret_cast<u32x2*>(codes + (int64_t)row * k + (int64_t)c8 * 8) = cv;
    uint8_t* sp = scales + (int64_t)row * (k / BLOCK);
    if constexpr (NB == 2) {
        *reinterpret_cast<uint16_t*>(sp + c8 * 2) = (uint16_t)(sb[0] | (sb[1] << 8));
    } else {
        if (LANES == 1 || (c8 % LANES) == 0) sp[c8 / LANES] = (uint8_t)sb[0];
    }
}

// bf16 input, g == 1, k % 32 == 0: a lane takes 32 elements (four 16-byte loads, two 16-byte
// code stores), so that the block scale (an fp64 division) and the addressing are paid once per
// 32 elements instead of per 8; blocks of up to 32 are lane-local, larger ones span BLOCK / 32
// lanes (absmax by shuffles).  Elements go through the hardware converter as above.
template <int BLOCK, int FMT>
__global__ __launch_bounds__(THREADS) void quantize_fp8_hw32_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                                    FastDiv gpr_div, uint32_t gpr, uint32_t total,
                                                                    uint8_t* __restrict__ codes,
                                                                    uint8_t* __restrict__ scales, int64_t k)
{
    constexpr int NB = BLOCK <= 32 ? 32 / BLOCK : 1;  // blocks (or block parts) per lane
    constexpr int WPB = 16 / NB;                       // bf16 pairs (words) per lane-local part
    constexpr int LANES = BLOCK > 32 ? BLOCK / 32 : 1;
    const uint32_t u = blockIdx.x * THREADS + threadIdx.x;
    const bool act = u < total;
    const uint32_t row = act ? gpr_div.div(u) : 0u;
    const uint32_t gc = act ? u - row * gpr : 0u;  // the lane holds elements 32 gc .. +31

    uint32_t w[16];  // word j: elements 2j (low half), 2j + 1
    if (act) {
        const u32x4* p = reinterpret_cast<const u32x4*>(x + (int64_t)row * ldx_bytes + (int64_t)gc * 64);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 v = p[q];
            w[4 * q] = v.x;
            w[4 * q + 1] = v.y;
            w[4 * q + 2] = v.z;
            w[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) w[j] = 0u;
    }

    uint32_t amax[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        u16x2 m = __builtin_bit_cast(u16x2, w[b * WPB] & 0x7FFF7FFFu);
#pragma unroll
        for (int j = 1; j < WPB; ++j)
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[b * WPB + j] & 0x7FFF7FFFu));
        amax[b] = (uint32_t)(m.x > m.y ? m.x : m.y) << 16;
    }
    if constexpr (LANES > 1) {
#pragma unroll
        for (int off = 1; off < LANES; off <<= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)amax[0], off);
            amax[0] = o > amax[0] ? o : amax[0];
        }
    }

    uint32_t sb[NB];
    i16x2 h[8];  // code dword d: elements 4d .. 4d + 3
#pragma unroll
    for (int d = 0; d < 8; ++d) h[d] = i16x2{0, 0};
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        sb[b] = scale_code_g<FMT>(amax[b], 448.0);
        const EncG1 p = enc_params_g1<FMT>(sb[b]);
        const float lim = 448.0f * p.pow2;  // 448 * 2^E (exact, also for 2^-127)
#pragma unroll
        for (int jj = 0; jj < WPB; ++jj) {
            const int j = b * WPB + jj;  // word j -> half j % 2 of code dword j / 2
            if (j & 1) h[j >> 1] = enc_fp8_pair<FMT, 1>(h[j >> 1], w[j], p, lim);
            else h[j >> 1] = enc_fp8_pair<FMT, 0>(h[j >> 1], w[j], p, lim);
        }
    }
    if (!act) return;
    u32x4* cp = reinterpret_cast<u32x4*>(codes + (int64_t)row * k + (int64_t)gc * 32);
    // non-temporal: the codes are not read again by this launch
    __builtin_nontemporal_store(u32x4{__builtin_bit_cast(uint32_t, h[0]), __builtin_bit_cast(uint32_t, h[1]),
                                      __builtin_bit_cast(uint32_t, h[2]), __builtin_bit_cast(uint32_t, h[3])}, cp);
    __builtin_nontemporal_store(u32x4{__builtin_bit_cast(uint32_t, h[4]), __builtin_bit_cast(uint32_t, h[5]),
                                      __builtin_bit_cast(uint32_t, h[6]), __builtin_bit_cast(uint32_t, h[7])}, cp + 1);
    uint8_t* sp = scales + (int64_t)row * (k / BLOCK);
    if constexpr (NB == 1) {
        if (LANES == 1 || (gc % LANES) == 0) sp[gc / LANES] = (uint8_t)sb[0];
    } else if constexpr (NB == 2) {
        *reinterpret_cast<uint16_t*>(sp + gc * 2) = (uint16_t)(sb[0] | (sb[1] << 8));
    } else if constexpr (NB == 4) {
        *reinterpret_cast<uint32_t*>(sp + gc * 4) = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
    } else {
        *reinterpret_cast<u32x2*>(sp + gc * 8) = u32x2{sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24),
                                                       sb[4] | (sb[5] << 8) | (sb[6] << 16) | (sb[7] << 24)};
    }
}

// quantize, generic path: one thread per block (any k % block == 0, any alignment)
template <int FMT, bool BF16>
__global__ __launch_bounds__(THREADS) void quantize_fp8_generic_kernel(const uint8_t* __restrict__ x, int64_t ldx,
                                                                       int64_t rows, int64_t k, int block, double g,
                                                                       uint8_t* __restrict__ codes,
                                                                       uint8_t* __restrict__ scales)
{
    const int64_t nb = k / block;
    const int64_t id = (int64_t)blockIdx.x * THREADS + threadIdx.x;
    if (id >= rows * nb) return;
    const int64_t r = id / nb, b = id - r * nb;
    const int64_t base = r * ldx + b * block;
    auto bits = [&](int64_t i) -> uint32_t {
        if constexpr (BF16) return (uint32_t)reinterpret_cast<const uint16_t*>(x)[base + i] << 16;
        else return reinterpret_cast<const uint32_t*>(x)[base + i];
    };
    uint32_t amax = 0;
    for (int i = 0; i < block; ++i) {
        const uint32_t a = bits(i) & 0x7FFFFFFFu;
        amax = a > amax ? a : amax;
    }
    const uint32_t sb = scale_code_g<FMT>(amax, 448.0 * g);
    scales[r * nb + b] = (uint8_t)sb;
    const Blk p = block_params<FMT>(sb, g);
    for (int i = 0; i < block; ++i) codes[r * k + b * block + i] = (uint8_t)elem_byte(bits(i), p);
}

// ---------------------------------------------------------------------------------------
// dequantize: y = fl32(e * s * g) (exact product in fp64), bf16 = RNE of that
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float dq_value(uint32_t c, double sg)
{
    const uint32_t m7 = c & 0x7Fu;
    const float f = (float)(mag(m7) * sg);
    return m7 == 0x7Fu ? __builtin_nanf("") : ((c & 0x80u) ? -f : f);  // 0x7F, 0xFF: NaN
}

// |e| of E4M3 magnitude code m (0..0x7E) as fp32, exact
__device__ __forceinline__ float e4m3_mag_f32(uint32_t m)
{
    const uint32_t ex = m >> 3, mn = m & 7u;
    return ex ? u2f(((ex + 120u) << 23) | (mn << 20)) : (float)mn * 0x1p-9f;
}

// The same value in fp32: e * s has at most 8 significant bits and lies in [2^-136, 2^128)
// when s <= 2^118, so it is exact in fp32 (subnormals included) and one fp32 multiply by g
// rounds e * s * g once, as the fp64 form does.  Larger scales (E8M0 bytes above 245) take
// the fp64 form.
__device__ __forceinline__ float dq_value_f32(uint32_t c, float s, float g)
{
    const uint32_t m7 = c & 0x7Fu;
    const float f = (e4m3_mag_f32(m7) * s) * g;
    return m7 == 0x7Fu ? __builtin_nanf("") : ((c & 0x80u) ? -f : f);  // 0x7F, 0xFF: NaN
}

template <int BLOCK, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(THREADS) void dequantize_fp8_kernel(const uint8_t* __restrict__ codes,
                                                                 const uint8_t* __restrict__ scales,
                                                                 FastDiv upr_div, uint32_t upr, uint32_t total,
                                                                 int64_t k, double g, uint8_t* __restrict__ y,
                                                                 int64_t ldy_bytes)
{
    const uint32_t u = blockIdx.x * THREADS + threadIdx.x;  // unit of 8 elements
    if (u >= total) return;
    const uint32_t row = upr_div.div(u), c8 = u - row * upr;
    const u32x2 cv = *reinterpret_cast<const u32x2*>(codes + (int64_t)row * k + (int64_t)c8 * 8);
    const uint8_t* sp = scales + (int64_t)row * (k / BLOCK);
    constexpr int NS = BLOCK < 8 ? 2 : 1;  // scale bytes of the unit
    uint32_t sb[NS];
    if constexpr (BLOCK < 8) {
        sb[0] = sp[c8 * 2];
        sb[1] = sp[c8 * 2 + 1];
    } else {
        sb[0] = sp[(c8 * 8) / BLOCK];
    }
    bool wide = false;  // an E8M0 scale above 2^118
#pragma unroll
    for (int i = 0; i < NS; ++i) wide |= FMT == FMT_E8M0 && sb[i] > 245u;
    float v[8];
    if (!wide) {
        const float gf = (float)g;
        float sf[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) sf[i] = scale_value_f32<FMT>(sb[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t c = ((e < 4 ? cv.x : cv.y) >> (8 * (e & 3))) & 0xFFu;
            v[e] = dq_value_f32(c, sf[BLOCK < 8 ? e / 4 : 0], gf);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t c = ((e < 4 ? cv.x : cv.y) >> (8 * (e & 3))) & 0xFFu;
            v[e] = dq_value(c, scale_value_f64<FMT>(sb[BLOCK < 8 ? e / 4 : 0]) * g);
        }
    }
    if constexpr (OUT_BF16) {
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[2 * j], (__bf16)v[2 * j + 1]});
        *reinterpret_cast<u32x4*>(y + (int64_t)row * ldy_bytes + (int64_t)c8 * 16) = u32x4{o[0], o[1], o[2], o[3]};
    } else {
        u32x4* p = reinterpret_cast<u32x4*>(y + (int64_t)row * ldy_bytes + (int64_t)c8 * 32);
        p[0] = u32x4{f2u(v[0]), f2u(v[1]), f2u(v[2]), f2u(v[3])};
        p[1] = u32x4{f2u(v[4]), f2u(v[5]), f2u(v[6]), f2u(v[7])};
    }
}

// Blocks of 8 or more: each lane takes two units of 8 consecutive elements, 64 units apart
// (a wave covers 128 consecutive units), so that every code load of a wave reads 512
// contiguous bytes and every store writes 1 KB (bf16) or 2 KB (fp32) contiguous.  A unit is
// decoded by the hardware converter with its scale's power of two, then multiplied by the
// scale's mantissa (E4M3 / UE5M3) and by g: e * 2^p is exact in fp32, so is its product with
// the mantissa (at most 8 significant bits), and the product with g is the one fp32 rounding
// -- the same value as the per-element form above.  A unit with a NaN code (0x7F, 0xFF) or,
// for g != 1, an E8M0 scale above 2^118 (where e * s may leave the fp32 range before g brings
// it back) takes the per-element form.
template <int BLOCK, int FMT>
__device__ __forceinline__ void dq8_unit(const u32x2 cv, uint32_t sb, float gf, double g, float (&v)[8])
{
    // bit 7 of a byte of (b & 0x7F) + 1 is set exactly when b & 0x7F == 0x7F, with no carry
    // into the next byte
    const uint32_t nanb = (((cv.x & 0x7F7F7F7Fu) + 0x01010101u) | ((cv.y & 0x7F7F7F7Fu) + 0x01010101u)) & 0x80808080u;
    if (nanb == 0 && !(FMT == FMT_E8M0 && sb > 245u && gf != 1.0f)) {
        const WScale<FMT> ws = wscale<FMT>(sb);
        const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cv.x, ws.pow2, false);
        const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cv.x, ws.pow2, true);
        const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cv.y, ws.pow2, false);
        const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cv.y, ws.pow2, true);
        v[0] = (a.x * ws.mant) * gf; v[1] = (a.y * ws.mant) * gf;
        v[2] = (b.x * ws.mant) * gf; v[3] = (b.y * ws.mant) * gf;
        v[4] = (c.x * ws.mant) * gf; v[5] = (c.y * ws.mant) * gf;
        v[6] = (d.x * ws.mant) * gf; v[7] = (d.y * ws.mant) * gf;
    } else {
        const bool wide = FMT == FMT_E8M0 && sb > 245u;
        const float sf = scale_value_f32<FMT>(sb);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t cb = ((e < 4 ? cv.x : cv.y) >> (8 * (e & 3))) & 0xFFu;
            v[e] = wide ? dq_value(cb, scale_value_f64<FMT>(sb) * g) : dq_value_f32(cb, sf, gf);
        }
    }
}

template <int BLOCK, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(THREADS) void dequantize_fp8_u2_kernel(const uint8_t* __restrict__ codes,
                                                                    const uint8_t* __restrict__ scales,
                                                                    FastDiv upr_div, uint32_t upr, uint32_t total,
                                                                    int64_t k, double g, uint8_t* __restrict__ y,
                                                                    int64_t ldy_bytes)
{
    static_assert(BLOCK >= 8, "one scale per unit");
    const uint32_t t = blockIdx.x * THREADS + threadIdx.x;
    const uint32_t u0 = (t >> 6) * 128 + (t & 63);           // units u0 and u0 + 64
    const float gf = (float)g;
    u32x2 cv[2];
    uint32_t sb[2], row[2], c8[2];
    bool ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // all loads before any arithmetic
        const uint32_t u = u0 + 64 * h;
        ok[h] = u < total;
        const uint32_t uu = ok[h] ? u : 0u;
        row[h] = upr_div.div(uu);
        c8[h] = uu - row[h] * upr;
        cv[h] = *reinterpret_cast<const u32x2*>(codes + (int64_t)row[h] * k + (int64_t)c8[h] * 8);
        sb[h] = scales[(int64_t)row[h] * (k / BLOCK) + (c8[h] * 8) / BLOCK];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (!ok[h]) continue;
        float v[8];
        dq8_unit<BLOCK, FMT>(cv[h], sb[h], gf, g, v);
        if constexpr (OUT_BF16) {
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[2 * j], (__bf16)v[2 * j + 1]});
            // non-temporal stores: 8% faster than plain ones here (bf16 out, 27.3-28.4 -> 25.3-25.8 us)
            __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]},
                                        reinterpret_cast<u32x4*>(y + (int64_t)row[h] * ldy_bytes + (int64_t)c8[h] * 16));
        } else {
            u32x4* p = reinterpret_cast<u32x4*>(y + (int64_t)row[h] * ldy_bytes + (int64_t)c8[h] * 32);
            __builtin_nontemporal_store(u32x4{f2u(v[0]), f2u(v[1]), f2u(v[2]), f2u(v[3])}, p);
            __builtin_nontemporal_store(u32x4{f2u(v[4]), f2u(v[5]), f2u(v[6]), f2u(v[7])}, p + 1);
        }
    }
}

template <int FMT, bool OUT_BF16>
__global__ __launch_bounds__(THREADS) void dequantize_fp8_generic_kernel(const uint8_t* __restrict__ codes,
                                                                         const uint8_t* __restrict__ scales,
                                                                         int64_t rows, int64_t k, int block, double g,
                                                                         uint8_t* __restrict__ y, int64_t ldy)
{
    const int64_t id = (int64_t)blockIdx.x * THREADS + threadIdx.x;
    if (id >= rows * k) return;
    const int64_t r = id / k, c = id - r * k;
    const double sg = scale_value_f64<FMT>(scales[r * (k / block) + c / block]) * g;
    const float v = dq_value(codes[r * k + c], sg);
    if constexpr (OUT_BF16) reinterpret_cast<__bf16*>(y)[r * ldy + c] = (__bf16)v;
    else reinterpret_cast<float*>(y)[r * ldy + c] = v;
}

// ---------------------------------------------------------------------------------------
// W8A16 GEMM / GEMV on bf16 16x16x32 matrix cores.  A workgroup (NW waves) owns NG groups of 16
// weight rows (output columns) and 16 MT activation rows; its waves take every NW-th 128-k
// window.  In a window a lane holds, per row group, weight row lane % 16 and the 32 consecutive
// k 32 (lane / 16) .. +31 (two 16-byte code loads: the four lanes of a row read its 128 bytes),
// dequantizes them to bf16 in registers and feeds four MFMAs with the activations of the same
// k: MFMA i takes k 32 (lane / 16) + 8 i .. +7 from every lane, the same permutation of k for
// both operands, which leaves each dot product unchanged.  The activations of a window are
// loaded once for all NG row groups.  The next window's codes and scales are loaded before the
// current window is computed.  The waves' partial sums meet in LDS.  Requires k % 32 == 0.
// ---------------------------------------------------------------------------------------
template <int BLOCK>
__device__ __forceinline__ uint64_t lane_scales(rsrc_t r, uint32_t off)
{
    if constexpr (BLOCK >= 32) return bload8(r, off);
    else if constexpr (BLOCK == 16) return bload16(r, off);
    else if constexpr (BLOCK == 8) return bload32(r, off);
    else return bload64(r, off);
}

template <int BLOCK, int FMT, int MT, bool OUT_BF16, int NG = 1, int NW = 4>
__global__ __launch_bounds__(64 * NW) void gemm_w8_kernel(const W8Args a)
{
    __shared__ f32x4 red[NW][NG][MT][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t r16 = lane & 15, q = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NG, m0 = (int64_t)blockIdx.y * 16 * MT;
    const uint32_t K = (uint32_t)a.k;
    const uint32_t nrows = (uint32_t)(a.n - n0 < 16 * NG ? a.n - n0 : 16 * NG);
    const uint32_t mrows = (uint32_t)(a.m - m0 < 16 * MT ? a.m - m0 : 16 * MT);
    const rsrc_t wc = make_rsrc(a.wc + n0 * a.k, nrows * K);
    const rsrc_t ws = make_rsrc(a.ws + n0 * (a.k / BLOCK), nrows * (K / BLOCK));
    const rsrc_t xr = make_rsrc(a.x + m0 * a.ldx, (uint32_t)(((int64_t)(mrows - 1) * a.ldx + a.k) * 2));
    const uint32_t nwin = (K + 127) / 128;

    f32x4 acc[NG][MT];
#pragma unroll
    for (int gq = 0; gq < NG; ++gq)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[gq][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto load_w = [&](uint32_t win, uint32_t (&cw)[NG][8], uint64_t (&sb)[NG]) {
        const uint32_t kc = win * 128 + 32 * q;
#pragma unroll
        for (int gq = 0; gq < NG; ++gq) {
            const uint32_t row = 16 * gq + r16;
            const bool ok = kc < K && row < nrows;
            const uint32_t off = ok ? row * K + kc : kOOB;
            const u32x4 c0 = bload128(wc, off), c1 = bload128(wc, ok ? off + 16 : kOOB);
            cw[gq][0] = c0.x; cw[gq][1] = c0.y; cw[gq][2] = c0.z; cw[gq][3] = c0.w;
            cw[gq][4] = c1.x; cw[gq][5] = c1.y; cw[gq][6] = c1.z; cw[gq][7] = c1.w;
            sb[gq] = lane_scales<BLOCK>(ws, ok ? row * (K / BLOCK) + kc / BLOCK : kOOB);
        }
    };

    uint32_t cw[NG][8];
    uint64_t sb[NG];
#pragma unroll
    for (int gq = 0; gq < NG; ++gq) sb[gq] = 0;
    uint32_t win = (uint32_t)wave;
    if (win < nwin) load_w(win, cw, sb);
    for (; win < nwin; win += NW) {
        uint32_t cn[NG][8];
        uint64_t sn[NG];
#pragma unroll
        for (int gq = 0; gq < NG; ++gq) sn[gq] = 0;
        if (win + NW < nwin) load_w(win + NW, cn, sn);
        const uint32_t kc = win * 128 + 32 * q;
        u32x4 xa[MT][4];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const uint32_t xrow = 16 * t + r16;
            const bool ok = kc < K && xrow < mrows;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xa[t][i] = bload128(xr, ok ? (xrow * (uint32_t)a.ldx + kc + 8 * i) * 2 : kOOB);
        }
#pragma unroll
        for (int gq = 0; gq < NG; ++gq) {
            uint32_t wb[16];
            dequant_w8<BLOCK, FMT>(cw[gq], sb[gq], wb);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 bv = {wb[4 * i], wb[4 * i + 1], wb[4 * i + 2], wb[4 * i + 3]};
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[gq][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[t][i]),
                                                                         __builtin_bit_cast(bf16x8, bv), acc[gq][t], 0, 0, 0);
            }
        }
#pragma unroll
        for (int gq = 0; gq < NG; ++gq) {
#pragma unroll
            for (int j = 0; j < 8; ++j) cw[gq][j] = cn[gq][j];
            sb[gq] = sn[gq];
        }
    }
#pragma unroll
    for (int gq = 0; gq < NG; ++gq)
#pragma unroll
        for (int t = 0; t < MT; ++t) red[wave][gq][t][lane] = acc[gq][t];
    __syncthreads();
    // wave w adds the four partials of (row group, m-subtile) pairs w, w + 4, ... and stores
    // them: lane holds C[4 (lane / 16) + i][lane % 16], rows m, columns n
    constexpr uint32_t ESZ = OUT_BF16 ? 2 : 4;
    const rsrc_t yr = make_rsrc(static_cast<uint8_t*>(a.y) + (m0 * a.ldy + n0) * ESZ, 0x7FFFFFFFu);
    for (int pr = wave; pr < NG * MT; pr += NW) {
        const int gq = pr / MT, t = pr % MT;
        f32x4 s = red[0][gq][t][lane];
#pragma unroll
        for (int v = 1; v < NW; ++v) s += red[v][gq][t][lane];
        const uint32_t nn = 16 * gq + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t mm = 16 * t + 4 * q + i;
            const uint32_t off = (mm < mrows && nn < nrows) ? (mm * (uint32_t)a.ldy + nn) * ESZ : kOOB;
            const float v = s[i] * (float)a.g;
            if constexpr (OUT_BF16) bstore16(yr, off, __builtin_bit_cast(uint16_t, (__bf16)v));
            else bstore32(yr, off, f2u(v));
        }
    }
}

// any k % block == 0: one thread per output, fp32 accumulation
template <int FMT, bool OUT_BF16>
__global__ __launch_bounds__(THREADS) void gemm_w8_generic_kernel(const W8Args a)
{
    const int64_t id = (int64_t)blockIdx.x * THREADS + threadIdx.x;
    if (id >= a.m * a.n) return;
    const int64_t m = id / a.n, n = id - m * a.n;
    float acc = 0.0f;
    for (int64_t kk = 0; kk < a.k; ++kk) {
        const double s = scale_value_f64<FMT>(a.ws[n * (a.k / a.block) + kk / a.block]);
        const float w = dq_value(a.wc[n * a.k + kk], s);
        acc = __builtin_fmaf(u2f((uint32_t)a.x[m * a.ldx + kk] << 16), w, acc);
    }
    const float v = acc * (float)a.g;
    if constexpr (OUT_BF16) reinterpret_cast<__bf16*>(a.y)[m * a.ldy + n] = (__bf16)v;
    else reinterpret_cast<float*>(a.y)[m * a.ldy + n] = v;
}

}  // namespace f8

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
template <int FMT, bool BF16>
static hipError_t launch_q8(const QuantArgs& a, hipStream_t st)
{
    const int esz = BF16 ? 2 : 4;
    if (!a.fast) {
        const int64_t nblk = a.rows * (a.k / a.block);
        hipLaunchKernelGGL((f8::quantize_fp8_generic_kernel<FMT, BF16>), dim3((unsigned)((nblk + 255) / 256)),
                           dim3(f8::THREADS), 0, st, static_cast<const uint8_t*>(a.x), a.ldx, a.rows, a.k, a.block,
                           a.g, a.codes, a.scales);
        return hipGetLastError();
    }
    if (BF16 && a.g == 1.0 && a.k % 32 == 0) {  // 32 elements per lane
        const uint32_t gpr = (uint32_t)(a.k / 32), total = (uint32_t)(a.rows * gpr);
        const FastDiv fd = FastDiv::make(gpr);
        const dim3 grid((total + f8::THREADS - 1) / f8::THREADS);
        switch (a.block) {
#define MXH(B)                                                                                                         \
    case B:                                                                                                            \
        hipLaunchKernelGGL((f8::quantize_fp8_hw32_kernel<B, FMT>), grid, dim3(f8::THREADS), 0, st,                       \
                           static_cast<const uint8_t*>(a.x), a.ldx * esz, fd, gpr, total, a.codes, a.scales, a.k); \
        break;
            MXH(4) MXH(8) MXH(16) MXH(32) MXH(64) MXH(128) MXH(256)
#undef MXH
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const uint32_t upr = (uint32_t)(a.k / 8), total = (uint32_t)(a.rows * upr);
    const FastDiv fd = FastDiv::make(upr);
    const dim3 grid((total + f8::THREADS - 1) / f8::THREADS);
#define MXQ8(B)                                                                                              \
    case B:                                                                                                  \
        if (BF16 && a.g == 1.0)                                                                              \
            hipLaunchKernelGGL((f8::quantize_fp8_kernel<B, FMT, BF16, BF16>), grid, dim3(f8::THREADS), 0, st, \
                               static_cast<const uint8_t*>(a.x), a.ldx * esz, fd, upr, total, a.g, a.codes, \
                               a.scales, a.k);                                                               \
        else                                                                                                 \
            hipLaunchKernelGGL((f8::quantize_fp8_kernel<B, FMT, BF16, false>), grid, dim3(f8::THREADS), 0, st, \
                               static_cast<const uint8_t*>(a.x), a.ldx * esz, fd, upr, total, a.g, a.codes, \
                               a.scales, a.k);                                                               \
        break;
    switch (a.block) {
        MXQ8(4) MXQ8(8) MXQ8(16) MXQ8(32) MXQ8(64) MXQ8(128) MXQ8(256)
        default: return hipErrorInvalidValue;
    }
#undef MXQ8
    return hipGetLastError();
}

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t st)
{
#define MXF(F) \
    if (a.fmt == F) return a.bf16 ? launch_q8<F, true>(a, st) : launch_q8<F, false>(a, st);
    MXF(FMT_E4M3) MXF(FMT_UE5M3) MXF(FMT_E8M0)
#undef MXF
    return hipErrorInvalidValue;
}

template <int FMT, bool OUT_BF16>
static hipError_t launch_dq8(const DequantArgs& a, hipStream_t st)
{
    if (!a.fast) {
        const int64_t n = a.rows * a.k;
        hipLaunchKernelGGL((f8::dequantize_fp8_generic_kernel<FMT, OUT_BF16>), dim3((unsigned)((n + 255) / 256)),
                           dim3(f8::THREADS), 0, st, a.codes, a.scales, a.rows, a.k, a.block, a.g,
                           static_cast<uint8_t*>(a.y), a.ldy);
        return hipGetLastError();
    }
    const int64_t ldyb = a.ldy * (OUT_BF16 ? 2 : 4);
    if (a.block >= 8) {
        const uint32_t upr = (uint32_t)(a.k / 8), total = (uint32_t)(a.rows * upr);
        const FastDiv fd = FastDiv::make(upr);
        const dim3 grid((total + 2 * f8::THREADS - 1) / (2 * f8::THREADS));  // two units per lane
#define MXDU(B)                                                                                              \
    case B:                                                                                                  \
        hipLaunchKernelGGL((f8::dequantize_fp8_u2_kernel<B, FMT, OUT_BF16>), grid, dim3(f8::THREADS), 0, st,  \
                           a.codes, a.scales, fd, upr, total, a.k, a.g, static_cast<uint8_t*>(a.y), ldyb);  \
        break;
        switch (a.block) {
            MXDU(8) MXDU(16) MXDU(32) MXDU(64) MXDU(128) MXDU(256)
            default: return hipErrorInvalidValue;
        }
#undef MXDU
        return hipGetLastError();
    }
    const uint32_t upr = (uint32_t)(a.k / 8), total = (uint32_t)(a.rows * upr);
    const FastDiv fd = FastDiv::make(upr);
    const dim3 grid((total + f8::THREADS - 1) / f8::THREADS);
#define MXD8(B)                                                                                              \
    case B:                                                                                                  \
        hipLaunchKernelGGL((f8::dequantize_fp8_kernel<B, FMT, OUT_BF16>), grid, dim3(f8::THREADS), 0, st,   \
                           a.codes, a.scales, fd, upr, total, a.k, a.g, static_cast<uint8_t*>(a.y), ldyb);  \
        break;
    switch (a.block) {
        MXD8(4) MXD8(8) MXD8(16) MXD8(32) MXD8(64) MXD8(128) MXD8(256)
        default: return hipErrorInvalidValue;
    }
#undef MXD8
    return hipGetLastError();
}

hipError_t launch_dequantize_fp8(const DequantArgs& a, hipStream_t st)
{
#define MXF(F) \
    if (a.fmt == F) return a.bf16 ? launch_dq8<F, true>(a, st) : launch_dq8<F, false>(a, st);
    MXF(FMT_E4M3) MXF(FMT_UE5M3) MXF(FMT_E8M0)
#undef MXF
    return hipErrorInvalidValue;
}

// Choice between the pipelined 128 x 256 tile kernel and the 16-row kernel above, from
// measured costs on MI355X: a wave of up to 256 tiles takes about 11 ns per k with E8M0
// scales (17.5 ns with E4M3 / UE5M3 scales, whose dequantization costs more), whatever the
// tile count; the 16-row kernel runs at about 100 TFLOP/s.  Few tiles and small m favour the
// latter (m 128, n 4096, k 4096: 41 against 45 us), many tiles the former (m 2048, n 28672,
// k 8192: 1.0 against 7.9 ms).
static bool w8_prefers_tiled(const W8Args& a)
{
    const double tiles = (double)((a.m + 127) / 128) * (double)((a.n + 255) / 256);
    const double t_tiled = std::ceil(tiles / 256.0) * (double)a.k * (a.fmt == FMT_E8M0 ? 11e-9 : 17.5e-9);
    const double t_rows = 2.0 * (double)a.m * (double)a.n * (double)a.k / 100e12;
    return t_tiled < t_rows;
}

template <int FMT, bool OUT_BF16>
static hipError_t launch_w8(const W8Args& a, hipStream_t st)
{
    if (!a.fast) {
        const int64_t total = a.m * a.n;
        hipLaunchKernelGGL((f8::gemm_w8_generic_kernel<FMT, OUT_BF16>), dim3((unsigned)((total + 255) / 256)),
                           dim3(f8::THREADS), 0, st, a);
        return hipGetLastError();
    }
    // the W4A16 kernels with FP8 codes: the sweeping GEMV (m <= 2, short streams) and the
    // pipelined matrix-core kernel (large products)
    GemmArgs ga{};
    ga.x = a.x;
    ga.m = a.m;
    ga.n = a.n;
    ga.k = a.k;
    ga.ldx = a.ldx;
    ga.wc = a.wc;
    ga.ws = a.ws;
    ga.block = a.block;
    ga.fmt = a.fmt;
    ga.g = (float)a.g;
    ga.y = a.y;
    ga.y_bf16 = a.y_bf16;
    ga.ldy = a.ldy;
    if (w8_uses_sweep(ga)) return launch_gemv_sweep_w8(ga, st);
    if (a.m > 16 && w8_prefers_tiled(a) && a16_uses_tiled(ga)) return launch_gemm_w8_tiled(ga, st);
    // m <= 16: 8 waves per workgroup and as many 16-row groups per workgroup (1, 2 or 4) as keep
    // at least 224 workgroups, which share each activation load among more weight rows
    // (n 14336, m 16: 4 groups, 19.5 against 30.8 us with one group of 4 waves; n 4096: one
    // group, 9.5 against 10.0 us)
    const bool small = a.m <= 16;
    const int ng = !small ? 1 : (a.n + 63) / 64 >= 224 ? 4 : (a.n + 31) / 32 >= 224 ? 2 : 1;
    const dim3 grid((unsigned)((a.n + 16 * ng - 1) / (16 * ng)), (unsigned)((a.m + (small ? 16 : 64) - 1) / (small ? 16 : 64)));
#define MXW8(B)                                                                                                  \
    case B:                                                                                                      \
        if (!small) hipLaunchKernelGGL((f8::gemm_w8_kernel<B, FMT, 4, OUT_BF16, 1, 4>), grid, dim3(256), 0, st, a);   \
        else if (ng == 4) hipLaunchKernelGGL((f8::gemm_w8_kernel<B, FMT, 1, OUT_BF16, 4, 8>), grid, dim3(512), 0, st, a); \
        else if (ng == 2) hipLaunchKernelGGL((f8::gemm_w8_kernel<B, FMT, 1, OUT_BF16, 2, 8>), grid, dim3(512), 0, st, a); \
        else hipLaunchKernelGGL((f8::gemm_w8_kernel<B, FMT, 1, OUT_BF16, 1, 8>), grid, dim3(512), 0, st, a);          \
        break;
    switch (a.block) {
        MXW8(4) MXW8(8) MXW8(16) MXW8(32) MXW8(64) MXW8(128) MXW8(256)
        default: return hipErrorInvalidValue;
    }
#undef MXW8
    return hipGetLastError();
}

hipError_t launch_gemm_w8(const W8Args& a, hipStream_t st)
{
#define MXF(F) \
    if (a.fmt == F) return a.y_bf16 ? launch_w8<F, true>(a, st) : launch_w8<F, false>(a, st);
    MXF(FMT_E4M3) MXF(FMT_UE5M3) MXF(FMT_E8M0)
#undef MXF
    return hipErrorInvalidValue;
}

}  // namespace mxk
