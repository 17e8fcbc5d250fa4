// mx_quant.hip -- MX FP4 block quantization and dequantization kernels for gfx950.
//
// Method: hotelren.com/news/2192771, article "量化技术演进与微缩量化原理", section 3.1
// (quantize_block: absmax -> FP8 scale of absmax/6 -> FP4 of x/scale; two-level scaling);
// gtnt.cn/news/16247 "为什么我们需要4-bit浮点量化", sections 2.1 (clip then round) and 4.3
// (two FP4 codes per byte).
//
// Quantize fast path: one lane owns 32 consecutive elements of a row (64 B of bf16 / 128 B
// of fp32, loaded with 128-bit loads) and writes their 16 code bytes with one 128-bit
// non-temporal store.  Blocks of up to 32 elements are lane-local; larger blocks (64..256)
// span 2..8 neighbouring lanes and reduce their absmax with cross-lane shuffles.
// Dequantize fast path: a lane converts 8 consecutive elements (one code dword) per step and
// writes them with one 128-bit (bf16) or two (fp32) non-temporal stores; consecutive lanes
// cover consecutive memory.  (On MI355X, measured: plain loads beat non-temporal loads for
// these streams, non-temporal stores beat plain stores.)  Both require k % 32 == 0 and
// 16-byte aligned rows; the generic path (one thread per block / element pair) covers every
// other valid shape with the same arithmetic.
#include "mx_device.h"
#include "mx_internal.h"

namespace mxk {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------------------
// quantize, fast path
// ---------------------------------------------------------------------------------------
template <int BLOCK, int FMT, bool BF16, bool G1>
__global__ __launch_bounds__(kThreads) void quantize_fast_kernel(
    const uint8_t* __restrict__ x, int64_t ldx_bytes, FastDiv groups_per_row, uint32_t gpr,
    uint32_t total_groups, double g, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t k, uint32_t ts_ks, uint32_t ps_cb)
{
    constexpr int NW = BF16 ? 16 : 32;                    // 32-bit words holding 32 elements
    constexpr int NB = BLOCK <= 32 ? 32 / BLOCK : 1;      // blocks (or block parts) per lane
    constexpr int WPB = NW / NB;                          // words per lane-local block part
    constexpr int LANES = BLOCK > 32 ? BLOCK / 32 : 1;    // lanes sharing one block

    const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
    const bool active = gid < total_groups;
    const uint32_t row = active ? groups_per_row.div(gid) : 0u;
    const uint32_t gc = active ? gid - row * gpr : 0u;

    uint32_t w[NW];
    if (active) {
        const u32x4* p = reinterpret_cast<const u32x4*>(x + (int64_t)row * ldx_bytes +
                                                        (int64_t)gc * (BF16 ? 64 : 128));
#pragma unroll
        for (int j = 0; j < NW / 4; ++j) {
            const u32x4 v = p[j];
            w[4 * j + 0] = v.x;
            w[4 * j + 1] = v.y;
            w[4 * j + 2] = v.z;
            w[4 * j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < NW; ++j) w[j] = 0u;
    }

    // with a per-tensor scale: the element thresholds of the eight scale mantissas, once per
    // workgroup (threads 0-7, one mantissa each), while the loads above are in flight; the
    // barrier leaves the global loads alone (only the table's LDS writes are waited for)
    __shared__ __attribute__((aligned(16))) uint32_t gtab[64];
    if constexpr (!G1) {
        if (threadIdx.x < 8) {
            uint32_t u[7];
            enc_thresholds((1.0 + 0.125 * (double)threadIdx.x) * g, u);
#pragma unroll
            for (int i = 0; i < 7; ++i) gtab[8 * threadIdx.x + i] = u[i];
            gtab[8 * threadIdx.x + 7] = 0u;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this thread's table writes are done
        asm volatile("s_barrier" ::: "memory");
    }

    // absmax bits (fp32 pattern of |x|) per lane-local block part
    uint32_t amax[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if constexpr (BF16) {
            u16x2 m = __builtin_bit_cast(u16x2, w[b * WPB] & 0x7FFF7FFFu);
#pragma unroll
            for (int j = 1; j < WPB; ++j)
                m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[b * WPB + j] & 0x7FFF7FFFu));
            const uint32_t mm = m.x > m.y ? m.x : m.y;
            amax[b] = mm << 16;
        } else {
            uint32_t m = w[b * WPB] & 0x7FFFFFFFu;
#pragma unroll
            for (int j = 1; j < WPB; ++j) {
                const uint32_t a = w[b * WPB + j] & 0x7FFFFFFFu;
                m = a > m ? a : m;
            }
            amax[b] = m;
        }
    }
    if constexpr (LANES > 1) {
#pragma unroll
        for (int off = 1; off < LANES; off <<= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)amax[0], off);
            amax[0] = o > amax[0] ? o : amax[0];
        }
    }

    // scale bytes
    uint32_t sbyte[NB];
    const double six_g = 6.0 * g;
#pragma unroll
    for (int b = 0; b < NB; ++b) sbyte[b] = G1 ? scale_code_g1<FMT>(amax[b]) : scale_code_g<FMT>(amax[b], six_g);

    if (BLOCK == 32 && ts_ks != 0) {  // tiled scale layout (block 32 only)
        if (active) {
            scales[tiled_scale_off(row, gc, ts_ks)] = (uint8_t)sbyte[0];
            // the blocks that pad the row's last stage read as scale byte 0
            for (uint32_t kb = gpr + gc; kb < 8 * ts_ks; kb += gpr) scales[tiled_scale_off(row, kb, ts_ks)] = 0;
        }
    } else if (BLOCK == 32 && ps_cb != 0) {  // preshuffled scale layout (block 32 only)
        if (active) {
            scales[pre_scale_off(row, gc, ps_cb)] = (uint8_t)sbyte[0];
            // the blocks that pad the row's last chunk read as scale byte 0
            for (uint32_t kb = gpr + gc; kb < 64 * ps_cb; kb += gpr) scales[pre_scale_off(row, kb, ps_cb)] = 0;
        }
    } else if (active) {
        uint8_t* sp = scales + (int64_t)row * (k / BLOCK);
        if constexpr (NB == 1) {
            if (LANES == 1 || (gc % LANES) == 0) sp[gc / LANES] = (uint8_t)sbyte[0];
        } else if constexpr (NB == 2) {
            *reinterpret_cast<uint16_t*>(sp + gc * 2) = (uint16_t)(sbyte[0] | (sbyte[1] << 8));
        } else if constexpr (NB == 4) {
            *reinterpret_cast<uint32_t*>(sp + gc * 4) =
                sbyte[0] | (sbyte[1] << 8) | (sbyte[2] << 16) | (sbyte[3] << 24);
        } else {
            const uint32_t lo = sbyte[0] | (sbyte[1] << 8) | (sbyte[2] << 16) | (sbyte[3] << 24);
            const uint32_t hi = sbyte[4] | (sbyte[5] << 8) | (sbyte[6] << 16) | (sbyte[7] << 24);
            const u32x2 sv = {lo, hi};
            *reinterpret_cast<u32x2*>(sp + gc * 8) = sv;
        }
    }

    // element codes: 4 output words of 8 codes each
    uint32_t out[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = 0u;

    if constexpr (G1) {
        EncG1 par[NB];  // all blocks' parameters first: their table loads issue together
#pragma unroll
        for (int b = 0; b < NB; ++b) par[b] = enc_params_g1<FMT>(sbyte[b]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const EncG1& p = par[b];
            if constexpr (BF16) {
                // pair j = elements (2j, 2j+1) = word j
#pragma unroll
                for (int jj = 0; jj < WPB; ++jj) {
                    const int j = b * WPB + jj;
                    uint32_t r;
                    if constexpr (FMT == FMT_E8M0) {
                        const bf16x2 v = __builtin_bit_cast(bf16x2, w[j]);
                        switch (j & 3) {
                            case 0: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out[j >> 2], v, p.pow2, 0); break;
                            case 1: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out[j >> 2], v, p.pow2, 1); break;
                            case 2: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out[j >> 2], v, p.pow2, 2); break;
                            default: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out[j >> 2], v, p.pow2, 3); break;
                        }
                    } else {
                        float lo = u2f(w[j] << 16), hi = u2f(w[j] & 0xFFFF0000u);
                        lo = __builtin_fmaf(lo, p.chi, lo * p.clo);
                        hi = __builtin_fmaf(hi, p.chi, hi * p.clo);
                        switch (j & 3) {
                            case 0: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out[j >> 2], lo, hi, p.pow2, 0); break;
                            case 1: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out[j >> 2], lo, hi, p.pow2, 1); break;
                            case 2: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out[j >> 2], lo, hi, p.pow2, 2); break;
                            default: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out[j >> 2], lo, hi, p.pow2, 3); break;
                        }
                    }
                    out[j >> 2] = r;
                }
            } else {
                // fp32: pair j = words (2j, 2j+1)
#pragma unroll
                for (int jj = 0; jj < WPB / 2; ++jj) {
                    const int j = b * (WPB / 2) + jj;
                    float lo = u2f(w[2 * j]), hi = u2f(w[2 * j + 1]);
                    if constexpr (FMT != FMT_E8M0) {
                        lo = __builtin_fmaf(lo, p.chi, lo * p.clo);
                        hi = __builtin_fmaf(hi, p.chi, hi * p.clo);
                    }
                    uint32_t r;
                    switch (j & 3) {
                        case 0: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out[j >> 2], lo, hi, p.pow2, 0); break;
                        case 1: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out[j >> 2], lo, hi, p.pow2, 1); break;
                        case 2: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out[j >> 2], lo, hi, p.pow2, 2); break;
                        default: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out[j >> 2], lo, hi, p.pow2, 3); break;
                    }
                    out[j >> 2] = r;
                }
            }
        }
    } else if constexpr (BF16) {
        // packed 16-bit decisions, two elements per word; word j holds elements 2j, 2j+1
        uint32_t z[16];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const EncG16 q = enc_params_g16(enc_params_g_tab<FMT>(sbyte[b], g, gtab));
#pragma unroll
            for (int jj = 0; jj < WPB; ++jj) z[b * WPB + jj] = enc_pair_g16(w[b * WPB + jj], q);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = pack_pairs_g16(z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]);
    } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const EncG p = enc_params_g_tab<FMT>(sbyte[b], g, gtab);
            constexpr int EPB = 32 / NB;  // elements per lane-local block part
#pragma unroll
            for (int ee = 0; ee < EPB; ++ee) {
                const int e = b * EPB + ee;
                const uint32_t xb = BF16 ? ((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16)) : w[e];
                out[e >> 3] |= enc_elem_g(xb, p) << (4 * (e & 7));
            }
        }
    }

    if (active) {
        u32x4* cp = reinterpret_cast<u32x4*>(codes + (int64_t)row * (k / 2) + (int64_t)gc * 16);
        const u32x4 ov = {out[0], out[1], out[2], out[3]};
        __builtin_nontemporal_store(ov, cp);
    }
}

// ---------------------------------------------------------------------------------------
// quantize, generic path: one thread per block
// ---------------------------------------------------------------------------------------
template <int FMT, bool BF16, bool G1>
__global__ __launch_bounds__(kThreads) void quantize_generic_kernel(
    const uint8_t* __restrict__ x, int64_t ldx, int64_t rows, int64_t k, int block, double g,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint32_t ts_ks, uint32_t ps_cb)
{
    const int64_t nb = k / block;
    const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
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
    const uint32_t sb = G1 ? scale_code_g1<FMT>(amax) : scale_code_g<FMT>(amax, 6.0 * g);
    if (ts_ks != 0) {  // tiled scale layout (block 32 only)
        scales[tiled_scale_off((uint32_t)r, (uint32_t)b, ts_ks)] = (uint8_t)sb;
        for (int64_t kb = nb + b; kb < 8 * (int64_t)ts_ks; kb += nb) scales[tiled_scale_off((uint32_t)r, (uint32_t)kb, ts_ks)] = 0;
    } else if (ps_cb != 0) {  // preshuffled scale layout (block 32 only)
        scales[pre_scale_off((uint32_t)r, (uint32_t)b, ps_cb)] = (uint8_t)sb;
        for (int64_t kb = nb + b; kb < 64 * (int64_t)ps_cb; kb += nb) scales[pre_scale_off((uint32_t)r, (uint32_t)kb, ps_cb)] = 0;
    } else {
        scales[r * nb + b] = (uint8_t)sb;
    }
    uint8_t* cp = codes + r * (k / 2) + b * (block / 2);
    if constexpr (G1) {
        const EncG1 p = enc_params_g1<FMT>(sb);
        for (int i = 0; i < block; i += 2) cp[i / 2] = (uint8_t)enc_pair_g1<FMT>(u2f(bits(i)), u2f(bits(i + 1)), p, 0u);
    } else {
        const EncG p = enc_params_g<FMT>(sb, g);
        for (int i = 0; i < block; i += 2)
            cp[i / 2] = (uint8_t)(enc_elem_g(bits(i), p) | (enc_elem_g(bits(i + 1), p) << 4));
    }
}

// ---------------------------------------------------------------------------------------
// dequantize, fast path: one lane per 32 consecutive elements
// ---------------------------------------------------------------------------------------
// G1: the converter applies pow2 and mant finishes e * s (exact).  Otherwise pow2 is the scale
// s itself and mant is g: e * s has at most 6 significant bits and lies in [2^-128, 2^128) for
// s <= 2^125, so it is exact in fp32 (subnormals included) and one fp32 multiply rounds e*s*g
// once; sg = s * g in fp64 (non-zero only for E8M0 scales above 2^125) selects the fp64 form.
template <int FMT, bool G1, bool OUT_BF16>
__device__ __forceinline__ void dec_byte_pair(uint32_t cw, int sel, float pow2, float mant,
                                             double sg, float& lo, float& hi)
{
    f32x2 f;
    const float sc = G1 ? pow2 : 1.0f;
    switch (sel) {
        case 0: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 0); break;
        case 1: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 1); break;
        case 2: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 2); break;
        default: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 3); break;
    }
    if constexpr (G1) {
        lo = (FMT == FMT_E8M0) ? f.x : f.x * mant;
        hi = (FMT == FMT_E8M0) ? f.y : f.y * mant;
    } else if (sg == 0.0) {  // one rounding of the exact e * s * g
        lo = (f.x * pow2) * mant;
        hi = (f.y * pow2) * mant;
    } else {
        lo = (float)((double)f.x * sg);
        hi = (float)((double)f.y * sg);
    }
}

constexpr int kDeqUnits = 2;  // 8-element units per lane

// LAY: scale layout, fixed at compile time so that the row-major kernel carries no layout
// branches between its loads (0 row-major, 1 tiled, 2 preshuffled; 1 and 2 with block 32 only)
template <int BLOCK, int FMT, bool G1, bool OUT_BF16, int LAY>
__global__ __launch_bounds__(kThreads) void dequantize_fast_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    FastDiv units_per_row, uint32_t upr, uint32_t total_units, int64_t k, double g,
    uint8_t* __restrict__ y, int64_t ldy_bytes, uint32_t ts_ks, uint32_t ps_cb)
{
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wbase = (blockIdx.x * kThreads + (threadIdx.x & ~63u)) * kDeqUnits;
    // issue every unit's loads first, then convert and store
    uint32_t cw[kDeqUnits], sb[kDeqUnits][2], row[kDeqUnits], c8[kDeqUnits];
    bool act[kDeqUnits];
#pragma unroll
    for (int h = 0; h < kDeqUnits; ++h) {
        const uint32_t u = wbase + h * 64 + lane;  // unit of 8 elements
        act[h] = u < total_units;
        row[h] = act[h] ? units_per_row.div(u) : 0u;
        c8[h] = act[h] ? u - row[h] * upr : 0u;  // the unit holds elements 8*c8 .. 8*c8+7
        cw[h] = 0u;
        sb[h][0] = sb[h][1] = 0u;
        if (act[h]) {
            cw[h] = *reinterpret_cast<const uint32_t*>(codes + (int64_t)row[h] * (k / 2) + (int64_t)c8[h] * 4);
            const uint8_t* sp = scales + (int64_t)row[h] * (k / BLOCK);
            if constexpr (BLOCK == 4) {
                const uint32_t v = *reinterpret_cast<const uint16_t*>(sp + c8[h] * 2);
                sb[h][0] = v & 0xFF;
                sb[h][1] = v >> 8;
            } else if constexpr (LAY == 1) {  // tiled scale layout
                sb[h][0] = sb[h][1] = scales[tiled_scale_off(row[h], c8[h] / 4, ts_ks)];
            } else if constexpr (LAY == 2) {  // preshuffled scale layout
                sb[h][0] = sb[h][1] = scales[pre_scale_off(row[h], c8[h] / 4, ps_cb)];
            } else {
                sb[h][0] = sb[h][1] = sp[(c8[h] * 8) / BLOCK];
            }
        }
    }
#pragma unroll
    for (int h = 0; h < kDeqUnits; ++h) {
        if (!act[h]) continue;
        uint32_t o[OUT_BF16 ? 4 : 8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // pair j = elements 2j, 2j+1 of the unit
            const uint32_t byte = sb[h][BLOCK == 4 ? (j >> 1) : 0];
            if constexpr (OUT_BF16 && G1 && FMT == FMT_E8M0) {
                const float pow2 = e8m0_value(byte);
                bf16x2 hv;
                switch (j) {
                    case 0: hv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[h], pow2, 0); break;
                    case 1: hv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[h], pow2, 1); break;
                    case 2: hv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[h], pow2, 2); break;
                    default: hv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[h], pow2, 3); break;
                }
                o[j] = __builtin_bit_cast(uint32_t, hv);
            } else {
                float pow2 = 1.0f, mant = 1.0f;
                double sg = 0.0;
                if constexpr (G1) {
                    const DecG1 p = dec_params_g1<FMT>(byte);
                    pow2 = p.pow2;
                    mant = p.mant;
                } else if (FMT == FMT_E8M0 && byte > 252u) {
                    sg = scale_value_f64<FMT>(byte) * g;
                } else {
                    pow2 = scale_value_f32<FMT>(byte);
                    mant = (float)g;
                }
                float lo, hi;
                dec_byte_pair<FMT, G1, OUT_BF16>(cw[h], j, pow2, mant, sg, lo, hi);
                if constexpr (OUT_BF16) {
                    bf16x2 hv;
                    hv.x = (__bf16)lo;
                    hv.y = (__bf16)hi;
                    o[j] = __builtin_bit_cast(uint32_t, hv);
                } else {
                    o[2 * j] = f2u(lo);
                    o[2 * j + 1] = f2u(hi);
                }
            }
        }
        u32x4* yp = reinterpret_cast<u32x4*>(y + (int64_t)row[h] * ldy_bytes + (int64_t)c8[h] * (OUT_BF16 ? 16 : 32));
        const u32x4 v0 = {o[0], o[1], o[2], o[3]};
        __builtin_nontemporal_store(v0, yp);
        if constexpr (!OUT_BF16) {
            const u32x4 v1 = {o[4], o[5], o[6], o[7]};
            __builtin_nontemporal_store(v1, yp + 1);
        }
    }
}

// ---------------------------------------------------------------------------------------
// dequantize, generic path: one thread per element pair
// ---------------------------------------------------------------------------------------
template <int FMT, bool G1, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void dequantize_generic_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t rows,
    int64_t k, int block, double g, uint8_t* __restrict__ y, int64_t ldy, uint32_t ts_ks, uint32_t ps_cb)
{
    const int64_t pairs = k / 2;
    const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (id >= rows * pairs) return;
    const int64_t r = id / pairs, j = id - r * pairs;
    const uint32_t cb = codes[r * pairs + j];
    const uint32_t sb = ts_ks != 0   ? scales[tiled_scale_off((uint32_t)r, (uint32_t)(j / 16), ts_ks)]
                        : ps_cb != 0 ? scales[pre_scale_off((uint32_t)r, (uint32_t)(j / 16), ps_cb)]
                                     : scales[r * (k / block) + (2 * j) / block];
    float pow2 = 1.0f, mant = 1.0f;
    double sg = 0.0;
    if constexpr (G1) {
        const DecG1 p = dec_params_g1<FMT>(sb);
        pow2 = p.pow2;
        mant = p.mant;
    } else if (FMT == FMT_E8M0 && sb > 252u) {
        sg = scale_value_f64<FMT>(sb) * g;
    } else {
        pow2 = scale_value_f32<FMT>(sb);
        mant = (float)g;
    }
    float lo, hi;
    dec_byte_pair<FMT, G1, OUT_BF16>(cb, 0, pow2, mant, sg, lo, hi);
    if constexpr (OUT_BF16) {
        uint16_t* yp = reinterpret_cast<uint16_t*>(y) + r * ldy + 2 * j;
        yp[0] = __builtin_bit_cast(uint16_t, (__bf16)lo);
        yp[1] = __builtin_bit_cast(uint16_t, (__bf16)hi);
    } else {
        float* yp = reinterpret_cast<float*>(y) + r * ldy + 2 * j;
        yp[0] = lo;
        yp[1] = hi;
    }
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
template <int FMT, bool BF16, bool G1>
static hipError_t launch_quantize_fmt(const QuantArgs& a, hipStream_t st)
{
    if (a.fast) {
        const uint32_t gpr = (uint32_t)(a.k / 32);
        const uint32_t total = (uint32_t)(a.rows * gpr);
        const dim3 grid((total + kThreads - 1) / kThreads);
        const int64_t ldb = a.ldx * (BF16 ? 2 : 4);
        switch (a.block) {
#define MXQ(B) case B: hipLaunchKernelGGL((quantize_fast_kernel<B, FMT, BF16, G1>), grid, dim3(kThreads), 0, st, \
                   (const uint8_t*)a.x, ldb, FastDiv::make(gpr), gpr, total, a.g, a.codes, a.scales, a.k, a.ts_ks, a.ps_cb); break;
            MXQ(4) MXQ(8) MXQ(16) MXQ(32) MXQ(64) MXQ(128) MXQ(256)
#undef MXQ
            default: return hipErrorInvalidValue;
        }
    } else {
        const int64_t n = a.rows * (a.k / a.block);
        const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
        hipLaunchKernelGGL((quantize_generic_kernel<FMT, BF16, G1>), grid, dim3(kThreads), 0, st,
                           (const uint8_t*)a.x, a.ldx, a.rows, a.k, a.block, a.g, a.codes, a.scales, a.ts_ks, a.ps_cb);
    }
    return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st)
{
    const bool g1 = a.g == 1.0;
#define MXF(F) \
    if (a.fmt == F) { \
        if (a.bf16) return g1 ? launch_quantize_fmt<F, true, true>(a, st) : launch_quantize_fmt<F, true, false>(a, st); \
        return g1 ? launch_quantize_fmt<F, false, true>(a, st) : launch_quantize_fmt<F, false, false>(a, st); \
    }
    MXF(FMT_E4M3) MXF(FMT_UE5M3) MXF(FMT_E8M0)
#undef MXF
    return hipErrorInvalidValue;
}

template <int FMT, bool G1, bool OUT_BF16>
static hipError_t launch_dequantize_fmt(const DequantArgs& a, hipStream_t st)
{
    if (a.fast) {
        const uint32_t upr = (uint32_t)(a.k / 8);
        const uint32_t total = (uint32_t)(a.rows * upr);
        const uint32_t per_wg = kThreads * kDeqUnits;
        const dim3 grid((total + per_wg - 1) / per_wg);
        const int64_t ldb = a.ldy * (OUT_BF16 ? 2 : 4);
        switch (a.block) {
#define MXDL(B, L) hipLaunchKernelGGL((dequantize_fast_kernel<B, FMT, G1, OUT_BF16, L>), grid, dim3(kThreads), 0, st, \
                   a.codes, a.scales, FastDiv::make(upr), upr, total, a.k, a.g, (uint8_t*)a.y, ldb, a.ts_ks, a.ps_cb)
#define MXD(B) case B: MXDL(B, 0); break;
            MXD(4) MXD(8) MXD(16) MXD(64) MXD(128) MXD(256)
            case 32:
                if (a.ts_ks != 0) MXDL(32, 1);
                else if (a.ps_cb != 0) MXDL(32, 2);
                else MXDL(32, 0);
                break;
#undef MXD
#undef MXDL
            default: return hipErrorInvalidValue;
        }
    } else {
        const int64_t n = a.rows * (a.k / 2);
        const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
        hipLaunchKernelGGL((dequantize_generic_kernel<FMT, G1, OUT_BF16>), grid, dim3(kThreads), 0, st,
                           a.codes, a.scales, a.rows, a.k, a.block, a.g, (uint8_t*)a.y, a.ldy, a.ts_ks, a.ps_cb);
    }
    return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t st)
{
    const bool g1 = a.g == 1.0;
#define MXF(F) \
    if (a.fmt == F) { \
        if (a.bf16) return g1 ? launch_dequantize_fmt<F, true, true>(a, st) : launch_dequantize_fmt<F, false, true>(a, st); \
        return g1 ? launch_dequantize_fmt<F, true, false>(a, st) : launch_dequantize_fmt<F, false, false>(a, st); \
    }
    MXF(FMT_E4M3) MXF(FMT_UE5M3) MXF(FMT_E8M0)
#undef MXF
    return hipErrorInvalidValue;
}

}  // namespace mxk
