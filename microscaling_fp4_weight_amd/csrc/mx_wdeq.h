// mx_wdeq.h -- weight dequantization into bf16 MFMA operands (device code, W4A16 and W8A16
// kernels).  FP4: a lane's 16 code bytes (32 consecutive k of one weight row) become 16
// dwords of bf16 pairs, e * s exactly: for E8M0 scales v_cvt_scalef32_pk_bf16_fp4 applies
// the power of two; for E4M3 / UE5M3 the conversion applies the scale's power of two and the
// product with its mantissa (at most 6 significant bits) is exact in bf16.  FP8: below.  The
// per-tensor scale is applied by the kernels' epilogues.
#pragma once
#include "mx_device.h"
#include "mx_internal.h"

namespace mxk {

// ---------------------------------------------------------------------------------------
// Weight fragment: 16 code bytes (32 k of one row) -> 16 dwords of bf16 pairs.
// ---------------------------------------------------------------------------------------
template <int FMT>
struct WScale {
    float pow2;
    float mant;
};

template <int FMT>
__device__ __forceinline__ WScale<FMT> wscale(uint32_t byte)
{
    WScale<FMT> s;
    if constexpr (FMT == FMT_E8M0) {
        s.pow2 = e8m0_value(byte);
        s.mant = 1.0f;
    } else {
        const DecG1 p = dec_params_g1<FMT>(byte);
        s.pow2 = p.pow2;
        s.mant = p.mant;
    }
    return s;
}

template <int FMT, int SEL>
__device__ __forceinline__ uint32_t deq_pair_bf16(uint32_t cw, const WScale<FMT>& s)
{
    if constexpr (FMT == FMT_E8M0) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, s.pow2, SEL));
    } else {
        const f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, s.pow2, SEL);
        bf16x2 h;
        h.x = (__bf16)(f.x * s.mant);  // e * s is exact in bf16 (<= 6 significant bits)
        h.y = (__bf16)(f.y * s.mant);
        return __builtin_bit_cast(uint32_t, h);
    }
}

template <int BLOCK, int FMT>
__device__ __forceinline__ void dequant32(const u32x4 cw, uint64_t sbytes, uint32_t d[16])
{
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int sel = 0; sel < 4; ++sel) {
            const int pair = 4 * w + sel;  // elements 2*pair, 2*pair+1 of the 32
            const int sidx = BLOCK >= 32 ? 0 : (2 * pair) / BLOCK;
            const WScale<FMT> s = wscale<FMT>((uint32_t)(sbytes >> (8 * sidx)) & 0xFFu);
            uint32_t v;
            switch (sel) {
                case 0: v = deq_pair_bf16<FMT, 0>(cw[w], s); break;
                case 1: v = deq_pair_bf16<FMT, 1>(cw[w], s); break;
                case 2: v = deq_pair_bf16<FMT, 2>(cw[w], s); break;
                default: v = deq_pair_bf16<FMT, 3>(cw[w], s); break;
            }
            d[pair] = v;
        }
    }
}

// The same 32 codes as e * 2^p (p = the scale's power of two; exact in bf16), returning the
// rest of the scale (its mantissa; 1 for E8M0).  A dot product over one scale block can then
// take the mantissa once, on the block's fp32 sum, instead of once per element: one
// conversion per pair instead of a conversion, two multiplies and a pack.
template <int FMT>
__device__ __forceinline__ float dequant32_pow2(const u32x4 cw, uint32_t byte, uint32_t (&d)[16])
{
    const WScale<FMT> s = wscale<FMT>(byte);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        d[4 * w + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[w], s.pow2, 0));
        d[4 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[w], s.pow2, 1));
        d[4 * w + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[w], s.pow2, 2));
        d[4 * w + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[w], s.pow2, 3));
    }
    return s.mant;
}

// ---------------------------------------------------------------------------------------
// FP8 weight fragment: 32 E4M3 codes (8 dwords, 32 consecutive k of one row) with their scale
// bytes -> 32 bf16 (16 dwords), e * s exact: an E4M3 value has at most 4 significant bits and
// the scale's mantissa at most 4, so every product fits bf16's 8.  For E8M0 scales the
// conversion applies the power of two and rounds straight to bf16 (exact); for E4M3 / UE5M3
// it yields fp32, the mantissa product is exact, and the bf16 is its upper half.
// ---------------------------------------------------------------------------------------
template <int BLOCK, int FMT>
__device__ __forceinline__ void dequant_w8(const uint32_t (&cw)[8], uint64_t sbytes, uint32_t (&out)[16])
{
#pragma unroll
    for (int h = 0; h < 16; ++h) {  // half-dword h: elements 2h, 2h+1
        const int e = 2 * h;
        const uint32_t byte = (uint32_t)(sbytes >> (8 * (BLOCK >= 32 ? 0 : e / BLOCK))) & 0xFFu;
        if constexpr (FMT == FMT_E8M0) {
            const float pow2 = e8m0_value(byte);
            bf16x2 d;
            if (h & 1) d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[h >> 1], pow2, true);
            else d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[h >> 1], pow2, false);
            out[h] = __builtin_bit_cast(uint32_t, d);
        } else {
            const DecG1 p = dec_params_g1<FMT>(byte);
            f32x2 d;
            if (h & 1) d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[h >> 1], p.pow2, true);
            else d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[h >> 1], p.pow2, false);
            const float lo = d.x * p.mant, hi = d.y * p.mant;
            out[h] = (f2u(lo) >> 16) | (f2u(hi) & 0xFFFF0000u);
        }
    }
}

}  // namespace mxk
