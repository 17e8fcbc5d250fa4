// mx_error.hip -- fused quantize -> dequantize -> error decomposition on the device.
//
// For every block: the scale byte and element codes exactly as mx_quantize makes them (the
// same device encoders), the dequantized values e(c) * s * g in fp64, and the squared errors
// (x^ - x)^2 split three ways (hotelren.com/news/2192771, article "量化技术演进与微缩量化原理",
// section 2.2 items 1-3): blocks whose scale is zero (flushed) feed the zero-scale term; in
// the other blocks the element holding the block maximum (its first occurrence) feeds the
// max-element term and every other element the ordinary-element term.  The sums, a separate
// sum of all squared errors, the count of flushed blocks and the count of blocks whose
// maximum is not coded +-6 are reduced in fp64 with a fixed order (one partial per
// workgroup of a fixed grid, then one workgroup over the partials), so repeated calls give
// identical results.
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

template <int FMT, bool BF16, bool G1>
__global__ __launch_bounds__(ERR_THREADS) void quant_error_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                                  int64_t nb, int64_t nblocks, int block, double g,
                                                                  double* __restrict__ partials)
{
    constexpr int ESZ = BF16 ? 2 : 4;
    double se = 0.0, sm = 0.0, sz = 0.0, st = 0.0, nzero = 0.0, nnot6 = 0.0;
    const int64_t stride = (int64_t)gridDim.x * ERR_THREADS;
    for (int64_t blk = (int64_t)blockIdx.x * ERR_THREADS + threadIdx.x; blk < nblocks; blk += stride) {
        const int64_t r = blk / nb, b = blk - r * nb;
        const uint8_t* p = x + r * ldx_bytes + b * block * ESZ;
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
        if (s == 0.0) {  // flushed block: every element codes to +-0
            nzero += 1.0;
            for (int i = 0; i < block; ++i) {
                const double xv = (double)u2f(elem_bits<BF16>(p, i));
                const double e2 = xv * xv;
                st += e2;
                sz += e2;
            }
            continue;
        }
        if constexpr (G1) {
            const EncG1 q = enc_params_g1<FMT>(sbyte);
            for (int i = 0; i < block; i += 2) {
                const uint32_t b0 = elem_bits<BF16>(p, i), b1 = elem_bits<BF16>(p, i + 1);
                const uint32_t cb = enc_pair_g1<FMT>(u2f(b0), u2f(b1), q, 0u);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t c = (cb >> (4 * h)) & 0xFu;
                    const double xv = (double)u2f(h ? b1 : b0);
                    const double err = e2m1_mag(c) * s * g - xv, e2 = err * err;
                    st += e2;
                    if (i + h == imax) {
                        sm += e2;
                        nnot6 += (c & 7u) != 7u ? 1.0 : 0.0;
                    } else {
                        se += e2;
                    }
                }
            }
        } else {
            const EncG q = enc_params_g<FMT>(sbyte, g);
            for (int i = 0; i < block; ++i) {
                const uint32_t xb = elem_bits<BF16>(p, i);
                const uint32_t c = enc_elem_g(xb, q);
                const double xv = (double)u2f(xb);
                const double err = e2m1_mag(c) * s * g - xv, e2 = err * err;
                st += e2;
                if (i == imax) {
                    sm += e2;
                    nnot6 += (c & 7u) != 7u ? 1.0 : 0.0;
                } else {
                    se += e2;
                }
            }
        }
    }
    // workgroup reduction in a fixed order: wave tree, then the four waves in order
    __shared__ double red[ERR_THREADS / 64][ERR_NP];
    double v[ERR_NP] = {se, sm, sz, st, nzero, nnot6};
#pragma unroll
    for (int j = 0; j < ERR_NP; ++j)
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v[j] += __shfl_xor(v[j], off);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
#pragma unroll
        for (int j = 0; j < ERR_NP; ++j) red[wave][j] = v[j];
    __syncthreads();
    if (threadIdx.x < ERR_NP) {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < ERR_THREADS / 64; ++w) t += red[w][threadIdx.x];
        partials[(int64_t)blockIdx.x * ERR_NP + threadIdx.x] = t;
    }
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
    if (threadIdx.x == 0) {
        double t[ERR_NP];
#pragma unroll
        for (int j = 0; j < ERR_NP; ++j) {
            t[j] = 0.0;
#pragma unroll
            for (int w = 0; w < ERR_THREADS / 64; ++w) t[j] += red[w][j];
        }
        out[0] = t[0] / n;
        out[1] = t[1] / n;
        out[2] = t[2] / n;
        out[3] = t[3] / n;
        out[4] = nblocks;
        out[5] = t[4];
        out[6] = t[5];
    }
}

int quant_error_groups(int64_t rows, int64_t k, int block)
{
    const int64_t nblocks = rows * (k / block);
    const int64_t g = (nblocks + ERR_THREADS - 1) / ERR_THREADS;
    return (int)(g < kErrMaxGroups ? g : kErrMaxGroups);
}

template <int FMT, bool BF16, bool G1>
static hipError_t launch_err(const ErrArgs& a, hipStream_t st)
{
    const int64_t nb = a.k / a.block, nblocks = a.rows * nb;
    const int groups = quant_error_groups(a.rows, a.k, a.block);
    hipLaunchKernelGGL((quant_error_kernel<FMT, BF16, G1>), dim3(groups), dim3(ERR_THREADS), 0, st,
                       static_cast<const uint8_t*>(a.x), a.ldx * (BF16 ? 2 : 4), nb, nblocks, a.block, a.g, a.partials);
    hipLaunchKernelGGL(quant_error_finish_kernel, dim3(1), dim3(ERR_THREADS), 0, st, a.partials, groups,
                       (double)(a.rows * a.k), (double)nblocks, a.out);
    return hipGetLastError();
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
