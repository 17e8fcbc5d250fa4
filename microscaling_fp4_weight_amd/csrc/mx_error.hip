// mx_error.hip -- fused quantize -> dequantize -> error decomposition on the device.
//
// For every block: the scale byte and element codes exactly as mx_quantize makes them (the
// same device encoders), the dequantized values e(c) * s * g, and the squared errors
// (x^ - x)^2 split three ways (hotelren.com/news/2192771, article "量化技术演进与微缩量化原理",
// section 2.2 items 1-3): blocks whose scale is zero (flushed) feed the zero-scale term; in
// the other blocks one element holding the block maximum |x| feeds the max-element term and
// every other element the ordinary-element term.  Elements tied at the maximum have the same
// code magnitude and the same squared error, so which of them counts as "the" maximum does
// not change any sum.  Optionally the dequantized tensor x^ itself is written (the forward
// pass of fake quantization), rounded as mx_dequantize rounds it.
//
// The sums, a separate total, the count of flushed blocks and the count of blocks whose
// maximum is not coded +-6 are reduced in fp64 in an order fixed by the shape (one partial
// per workgroup of a fixed grid, then one workgroup over the partials), so repeated calls
// give identical results.
//
// Exactness: with g == 1 and bf16 input, e * s has at most 6 significant bits and x at most
// 8, within a factor 4 of each other when e != 0, so the fp32 difference e*s - x is exact;
// its square is formed by an fp64 fma.  fp32 input and g != 1 take the difference in fp64,
// where it is exact as well (e * s * g has at most 30 significant bits).
#include "mx_device.h"
#include "mx_internal.h"

namespace mxk {

constexpr int ERR_THREADS = 256;
constexpr int ERR_NP = 6;  // partial sums per workgroup: elem, max, zero, total, flushed, max not 6

// E2M1 magnitudes of codes 0..7 (exact)
__device__ __forceinline__ double e2m1_mag(uint32_t c)
{
    const uint32_t m = c & 7u;
    const double tab[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double v = tab[0];
#pragma unroll
    for (uint32_t i = 1; i < 8; ++i) v = m == i ? tab[i] : v;
    return (c & 8u) ? -v : v;
}

template <bool BF16>
__device__ __forceinline__ uint32_t elem_bits(const uint8_t* p, int i)  // fp32 bit pattern
{
    if constexpr (BF16) return (uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16;
    else return reinterpret_cast<const uint32_t*>(p)[i];
}

// nearest-even bf16 of an fp32 value (finite or +-Inf)
__device__ __forceinline__ uint32_t bf16_bits_rne(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Workgroup reduction of ERR_NP values in a fixed order (wave tree, then the waves in
// order); thread t < ERR_NP returns sum t, the others 0.
__device__ __forceinline__ double wg_reduce(double (&v)[ERR_NP])
{
    __shared__ double red[ERR_THREADS / 64][ERR_NP];
#pragma unroll
    for (int j = 0; j < ERR_NP; ++j)
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v[j] += __shfl_xor(v[j], off);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
#pragma unroll
        for (int j = 0; j < ERR_NP; ++j) red[wave][j] = v[j];
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x < ERR_NP)
#pragma unroll
        for (int w = 0; w < ERR_THREADS / 64; ++w) t += red[w][threadIdx.x];
    return t;
}

// ---------------------------------------------------------------------------------------
// Fast path: one lane per 32 consecutive elements (k % 32 == 0, 16-byte aligned rows), a
// grid-stride loop over the tensor's 32-element groups in which each lane loads its next
// group before working on the current one.  Blocks of 4..32 elements lie in one lane (NB of
// them); larger blocks span BLOCK/32 adjacent lanes, whose absmax and tie counts are
// combined with lane shuffles and whose block-level terms the first lane adds.
// ---------------------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ void load_group(uint32_t (&w)[BF16 ? 16 : 32], const uint8_t* p)
{
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int j = 0; j < (BF16 ? 4 : 8); ++j) {
        const u32x4 v = q[j];  // plain loads: each instruction touches 64-byte runs, merged in cache
        w[4 * j + 0] = v.x;
        w[4 * j + 1] = v.y;
        w[4 * j + 2] = v.z;
        w[4 * j + 3] = v.w;
    }
}

// Encode the pair (lo, hi) -- word wd when bf16 -- into byte SEL of `codes` (g == 1).
template <int FMT, bool BF16, int SEL>
__device__ __forceinline__ uint32_t enc_pair_sel(uint32_t codes, float lo, float hi, uint32_t wd, const EncG1& p)
{
    if constexpr (BF16 && FMT == FMT_E8M0) {
        return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2, wd), p.pow2, SEL);
    } else {
        if constexpr (FMT != FMT_E8M0) {
            lo = __builtin_fmaf(lo, p.chi, lo * p.clo);
            hi = __builtin_fmaf(hi, p.chi, hi * p.clo);
        }
        return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, lo, hi, p.pow2, SEL);
    }
}

// e * scale for the two codes in byte SEL of `codes`
template <int SEL>
__device__ __forceinline__ f32x2 dec_pair_sel(uint32_t codes, float scale)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, scale, SEL);
}

template <int BLOCK, int FMT, bool BF16, bool G1, bool XHAT>
__global__ __launch_bounds__(ERR_THREADS) void quant_error_fast_kernel(
    const uint8_t* __restrict__ x, int64_t ldx_bytes, FastDiv groups_per_row, uint32_t gpr,
    uint32_t total_groups, double g, uint8_t* __restrict__ xh, int64_t ldxh_bytes,
    double* __restrict__ partials)
{
    constexpr int NW = BF16 ? 16 : 32;                // 32-bit words holding 32 elements
    constexpr int NB = BLOCK <= 32 ? 32 / BLOCK : 1;  // blocks (or block parts) per lane
    constexpr int EPB = 32 / NB;                      // elements per lane-local part
    constexpr int LANES = BLOCK > 32 ? BLOCK / 32 : 1;
    constexpr int ESZ = BF16 ? 2 : 4;

    double se = 0.0, sm = 0.0, sz = 0.0, st = 0.0, nzero = 0.0, nnot6 = 0.0;
    const uint32_t stride = gridDim.x * ERR_THREADS;
    uint32_t gid = blockIdx.x * ERR_THREADS + threadIdx.x;
    auto addr = [&](uint32_t gi, uint32_t& row, uint32_t& gc) {
        row = groups_per_row.div(gi);
        gc = gi - row * gpr;
        return x + (int64_t)row * ldx_bytes + (int64_t)gc * (32 * ESZ);
    };
    uint32_t row = 0, gc = 0;
    uint32_t wn[NW];
    if (gid < total_groups) load_group<BF16>(wn, addr(gid, row, gc));
    for (; gid < total_groups; gid += stride) {
        uint32_t w[NW];
#pragma unroll
        for (int j = 0; j < NW; ++j) w[j] = wn[j];
        const uint32_t crow = row, cgc = gc;
        if (gid + stride < total_groups) load_group<BF16>(wn, addr(gid + stride, row, gc));

        // fp32 bits of element e of this lane's 32
        auto xbits = [&](int e) -> uint32_t {
            if constexpr (BF16) return (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16);
            else return w[e];
        };

        // absmax bits per lane-local part
        uint32_t amax[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            uint32_t m = 0;
#pragma unroll
            for (int e = 0; e < EPB; ++e) {
                const uint32_t a = xbits(b * EPB + e) & 0x7FFFFFFFu;
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

        uint32_t xo[XHAT ? NW : 1];  // x^ in the input's element type
        uint32_t cw[4] = {0u, 0u, 0u, 0u};  // the 32 codes, 8 per word
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t sbyte = G1 ? scale_code_g1<FMT>(amax[b]) : scale_code_g<FMT>(amax[b], 6.0 * g);
            const double s64 = scale_value_f64<FMT>(sbyte);
            const bool flushed = s64 == 0.0;
            const float amf = u2f(amax[b]);
            // squared errors of all the lane's elements of the block; an element tied with the
            // maximum (|x| = max) has exactly the maximum's squared error, so the block's
            // maximum term is taken off the total once, below, instead of testing every element
            double acc = 0.0;
            uint32_t cmax;     // code magnitude of the maximum
            double sqm;        // its squared error

            if constexpr (G1) {
                const EncG1 ep = enc_params_g1<FMT>(sbyte);
                const DecG1 dp = dec_params_g1<FMT>(sbyte);
                {
                    const uint32_t cb = enc_pair_g1<FMT>(amf, 0.0f, ep, 0u);
                    cmax = cb & 7u;
                    const f32x2 d = dec_pair_sel<0>(cb, dp.pow2);
                    const double em = (double)d.x * (double)dp.mant - (double)amf;
                    sqm = em * em;
                }
#pragma unroll
                for (int pr = 0; pr < EPB / 2; ++pr) {
                    const int e = b * EPB + 2 * pr;  // pair index e / 2: word e / 8, byte (e / 2) % 4
                    const float lo = u2f(xbits(e)), hi = u2f(xbits(e + 1));
                    const uint32_t wd = BF16 ? w[e >> 1] : 0u;
                    uint32_t& c = cw[e >> 3];
                    f32x2 d;
                    switch ((e >> 1) & 3) {
                        case 0: c = enc_pair_sel<FMT, BF16, 0>(c, lo, hi, wd, ep); d = dec_pair_sel<0>(c, dp.pow2); break;
                        case 1: c = enc_pair_sel<FMT, BF16, 1>(c, lo, hi, wd, ep); d = dec_pair_sel<1>(c, dp.pow2); break;
                        case 2: c = enc_pair_sel<FMT, BF16, 2>(c, lo, hi, wd, ep); d = dec_pair_sel<2>(c, dp.pow2); break;
                        default: c = enc_pair_sel<FMT, BF16, 3>(c, lo, hi, wd, ep); d = dec_pair_sel<3>(c, dp.pow2); break;
                    }
                    const float q0 = FMT == FMT_E8M0 ? d.x : d.x * dp.mant;  // e * s, exact
                    const float q1 = FMT == FMT_E8M0 ? d.y : d.y * dp.mant;
                    double e0, e1;
                    if constexpr (BF16) {
                        e0 = (double)(q0 - lo);  // exact in fp32
                        e1 = (double)(q1 - hi);
                    } else {
                        e0 = (double)q0 - (double)lo;
                        e1 = (double)q1 - (double)hi;
                    }
                    acc = __builtin_fma(e0, e0, acc);
                    acc = __builtin_fma(e1, e1, acc);
                    if constexpr (XHAT) {
                        if constexpr (BF16) xo[e >> 1] = (f2u(q0) >> 16) | (f2u(q1) & 0xFFFF0000u);  // exact
                        else {
                            xo[e] = f2u(q0);
                            xo[e + 1] = f2u(q1);
                        }
                    }
                }
            } else {
                const EncG ep = enc_params_g<FMT>(sbyte, g);
                const double sg = s64 * g;  // exact
                {
                    const uint32_t cm = enc_elem_g(amax[b], ep);
                    cmax = cm & 7u;
                    const double em = e2m1_mag(cm) * sg - (double)amf;
                    sqm = em * em;
                }
#pragma unroll
                for (int pr = 0; pr < EPB / 2; ++pr) {
                    const int e = b * EPB + 2 * pr;
                    const uint32_t b0 = xbits(e), b1 = xbits(e + 1);
                    const uint32_t cb = enc_elem_g(b0, ep) | (enc_elem_g(b1, ep) << 4);
                    const f32x2 d = dec_pair_sel<0>(cb, 1.0f);  // e
                    const double q0 = (double)d.x * sg, q1 = (double)d.y * sg;  // exact
                    const float lo = u2f(b0), hi = u2f(b1);
                    const double e0 = q0 - (double)lo, e1 = q1 - (double)hi;
                    acc = __builtin_fma(e0, e0, acc);
                    acc = __builtin_fma(e1, e1, acc);
                    if constexpr (XHAT) {
                        const float r0 = (float)q0, r1 = (float)q1;  // one rounding of e*s*g
                        if constexpr (BF16) xo[e >> 1] = bf16_bits_rne(r0) | (bf16_bits_rne(r1) << 16);
                        else {
                            xo[e] = f2u(r0);
                            xo[e + 1] = f2u(r1);
                        }
                    }
                }
            }

            // block-level terms: once per block (by the block's first lane when it spans lanes);
            // the block's elements other than one maximum are its ordinary-element term
            bool lead = true;
            if constexpr (LANES > 1) lead = (cgc & (LANES - 1)) == 0;
            st += acc;
            if (flushed) {
                sz += acc;
                nzero += lead ? 1.0 : 0.0;
            } else {
                se += lead ? acc - sqm : acc;
                sm += lead ? sqm : 0.0;
                nnot6 += (lead && cmax != 7u) ? 1.0 : 0.0;
            }
        }

        if constexpr (XHAT) {
            u32x4* op = reinterpret_cast<u32x4*>(xh + (int64_t)crow * ldxh_bytes + (int64_t)cgc * (32 * ESZ));
#pragma unroll
            for (int j = 0; j < NW / 4; ++j) {
                const u32x4 v = {xo[4 * j], xo[4 * j + 1], xo[4 * j + 2], xo[4 * j + 3]};
                op[j] = v;  // plain stores: lanes write 64-byte runs, which L2 merges into full lines
            }
        }
    }
    double v[ERR_NP] = {se, sm, sz, st, nzero, nnot6};
    const double t = wg_reduce(v);
    if (threadIdx.x < ERR_NP) partials[(int64_t)blockIdx.x * ERR_NP + threadIdx.x] = t;
}

// ---------------------------------------------------------------------------------------
// Generic path: one thread per block, any shape and alignment (k even, k % block == 0).
// ---------------------------------------------------------------------------------------
template <int FMT, bool BF16, bool G1>
__global__ __launch_bounds__(ERR_THREADS) void quant_error_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                                  int64_t nb, int64_t nblocks, int block, double g,
                                                                  uint8_t* __restrict__ xh, int64_t ldxh_bytes,
                                                                  double* __restrict__ partials)
{
    constexpr int ESZ = BF16 ? 2 : 4;
    double se = 0.0, sm = 0.0, sz = 0.0, st = 0.0, nzero = 0.0, nnot6 = 0.0;
    const int64_t stride = (int64_t)gridDim.x * ERR_THREADS;
    for (int64_t blk = (int64_t)blockIdx.x * ERR_THREADS + threadIdx.x; blk < nblocks; blk += stride) {
        const int64_t r = blk / nb, b = blk - r * nb;
        const uint8_t* p = x + r * ldx_bytes + b * block * ESZ;
        uint8_t* o = xh ? xh + r * ldxh_bytes + b * block * ESZ : nullptr;
        // block maximum (integer order of sign-cleared bit patterns) and its first index
        uint32_t amax = 0;
        int imax = 0;
        for (int i = 0; i < block; ++i) {
            const uint32_t a = elem_bits<BF16>(p, i) & 0x7FFFFFFFu;
            if (i == 0 || a > amax) {
                imax = i;
                amax = a;
            }
        }
        const uint32_t sbyte = G1 ? scale_code_g1<FMT>(amax) : scale_code_g<FMT>(amax, 6.0 * g);
        const double s = scale_value_f64<FMT>(sbyte);
        const bool flushed = s == 0.0;
        nzero += flushed ? 1.0 : 0.0;
        EncG1 p1;
        EncG pg;
        if constexpr (G1) p1 = enc_params_g1<FMT>(sbyte);
        else pg = enc_params_g<FMT>(sbyte, g);
        for (int i = 0; i < block; i += 2) {
            const uint32_t b0 = elem_bits<BF16>(p, i), b1 = elem_bits<BF16>(p, i + 1);
            uint32_t cb;
            if constexpr (G1) cb = enc_pair_g1<FMT>(u2f(b0), u2f(b1), p1, 0u);
            else cb = enc_elem_g(b0, pg) | (enc_elem_g(b1, pg) << 4);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t c = (cb >> (4 * h)) & 0xFu;
                const double q = e2m1_mag(c) * s * g;  // exact
                const double err = q - (double)u2f(h ? b1 : b0), e2 = err * err;
                st += e2;
                if (flushed) {
                    sz += e2;
                } else if (i + h == imax) {
                    sm += e2;
                    nnot6 += (c & 7u) != 7u ? 1.0 : 0.0;
                } else {
                    se += e2;
                }
                if (o) {
                    const float r32 = (float)q;  // one rounding of e*s*g
                    if constexpr (BF16) reinterpret_cast<uint16_t*>(o)[i + h] = (uint16_t)bf16_bits_rne(r32);
                    else reinterpret_cast<float*>(o)[i + h] = r32;
                }
            }
        }
    }
    double v[ERR_NP] = {se, sm, sz, st, nzero, nnot6};
    const double t = wg_reduce(v);
    if (threadIdx.x < ERR_NP) partials[(int64_t)blockIdx.x * ERR_NP + threadIdx.x] = t;
}

// One workgroup: the partials in a fixed order, then the means.
__global__ __launch_bounds__(ERR_THREADS) void quant_error_finish_kernel(const double* __restrict__ partials,
                                                                         int groups, double n, double nblocks,
                                                                         double* __restrict__ out)
{
    double v[ERR_NP] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int gi = threadIdx.x; gi < groups; gi += ERR_THREADS)
#pragma unroll
        for (int j = 0; j < ERR_NP; ++j) v[j] += partials[(int64_t)gi * ERR_NP + j];
    const double t = wg_reduce(v);
    if (threadIdx.x < 4) out[threadIdx.x] = t / n;  // the four means
    else if (threadIdx.x < ERR_NP) out[threadIdx.x + 1] = t;  // flushed, max not 6
    else if (threadIdx.x == ERR_NP) out[4] = nblocks;
}

// Workgroups of either path for this shape: one thread per block (generic) or per 32
// elements (fast), capped at kErrMaxGroups; the workspace holds ERR_NP doubles for each.
int quant_error_groups(int64_t rows, int64_t k, int block)
{
    const int64_t per_row = (k / block) > (k + 31) / 32 ? (k / block) : (k + 31) / 32;
    const int64_t g = (rows * per_row + ERR_THREADS - 1) / ERR_THREADS;
    return (int)(g < kErrMaxGroups ? g : kErrMaxGroups);
}

static int capped_groups(int64_t units)
{
    const int64_t g = (units + ERR_THREADS - 1) / ERR_THREADS;
    return (int)(g < kErrMaxGroups ? g : kErrMaxGroups);
}

static hipError_t launch_finish(const ErrArgs& a, int groups, hipStream_t st)
{
    hipLaunchKernelGGL(quant_error_finish_kernel, dim3(1), dim3(ERR_THREADS), 0, st, a.partials, groups,
                       (double)(a.rows * a.k), (double)(a.rows * (a.k / a.block)), a.out);
    return hipGetLastError();
}

template <int FMT, bool BF16, bool G1>
static hipError_t launch_err_generic(const ErrArgs& a, hipStream_t st)
{
    const int64_t nb = a.k / a.block, nblocks = a.rows * nb;
    const int groups = capped_groups(nblocks);
    constexpr int ESZ = BF16 ? 2 : 4;
    hipLaunchKernelGGL((quant_error_kernel<FMT, BF16, G1>), dim3(groups), dim3(ERR_THREADS), 0, st,
                       static_cast<const uint8_t*>(a.x), a.ldx * ESZ, nb, nblocks, a.block, a.g,
                       static_cast<uint8_t*>(a.xhat), a.ldxh * ESZ, a.partials);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_finish(a, groups, st);
}

template <int BLOCK, int FMT, bool BF16, bool G1>
static hipError_t launch_err_fast(const ErrArgs& a, hipStream_t st)
{
    constexpr int ESZ = BF16 ? 2 : 4;
    const uint32_t gpr = (uint32_t)(a.k / 32);
    const uint32_t total = (uint32_t)(a.rows * (a.k / 32));
    const int groups = capped_groups(total);
    const FastDiv fd = FastDiv::make(gpr);
    if (a.xhat)
        hipLaunchKernelGGL((quant_error_fast_kernel<BLOCK, FMT, BF16, G1, true>), dim3(groups), dim3(ERR_THREADS), 0, st,
                           static_cast<const uint8_t*>(a.x), a.ldx * ESZ, fd, gpr, total, a.g,
                           static_cast<uint8_t*>(a.xhat), a.ldxh * ESZ, a.partials);
    else
        hipLaunchKernelGGL((quant_error_fast_kernel<BLOCK, FMT, BF16, G1, false>), dim3(groups), dim3(ERR_THREADS), 0, st,
                           static_cast<const uint8_t*>(a.x), a.ldx * ESZ, fd, gpr, total, a.g,
                           static_cast<uint8_t*>(nullptr), (int64_t)0, a.partials);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_finish(a, groups, st);
}

template <int FMT, bool BF16, bool G1>
static hipError_t launch_err(const ErrArgs& a, hipStream_t st)
{
    if (!a.fast) return launch_err_generic<FMT, BF16, G1>(a, st);
    switch (a.block) {
        case 4: return launch_err_fast<4, FMT, BF16, G1>(a, st);
        case 8: return launch_err_fast<8, FMT, BF16, G1>(a, st);
        case 16: return launch_err_fast<16, FMT, BF16, G1>(a, st);
        case 32: return launch_err_fast<32, FMT, BF16, G1>(a, st);
        case 64: return launch_err_fast<64, FMT, BF16, G1>(a, st);
        case 128: return launch_err_fast<128, FMT, BF16, G1>(a, st);
        case 256: return launch_err_fast<256, FMT, BF16, G1>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_quant_error(const ErrArgs& a, hipStream_t st)
{
    const bool g1 = a.g == 1.0;
#define MXF(F)                                                                                        \
    if (a.fmt == F) {                                                                                 \
        if (a.bf16) return g1 ? launch_err<F, true, true>(a, st) : launch_err<F, true, false>(a, st); \
        return g1 ? launch_err<F, false, true>(a, st) : launch_err<F, false, false>(a, st);           \
    }
    MXF(FMT_E4M3) MXF(FMT_UE5M3) MXF(FMT_E8M0)
#undef MXF
    return hipErrorInvalidValue;
}

}  // namespace mxk
