// mx_stats.hip -- whole-tensor mean, sample standard deviation and max |x| on the device: the
// statistic the block-size policy reads (hotelren.com/news/2192771, article
// "量化技术演进与微缩量化原理", section 6 item 2: the block size follows the tensor's standard
// deviation).
//
// Two passes in fp64, as the textbook defines the quantities: pass 1 sums x (and takes the
// largest |x| bit pattern), pass 2 sums (x - mean)^2 with the mean pass 1 left in device
// memory.  Each pass runs a fixed grid of workgroups over the tensor in units of 8 elements
// (16-byte loads) or, for rows that are not 16-byte aligned or k % 8 != 0, single elements;
// the per-workgroup partials are then added by one workgroup in a fixed order, so repeated
// calls return identical bits.
#include <math.h>

#include "mx_device.h"
#include "mx_internal.h"

namespace mxk {

constexpr int ST_THREADS = 256;

__device__ __forceinline__ double wg_sum(double v, double* red)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < ST_THREADS / 64; ++w) t += red[w];
    __syncthreads();
    return t;
}

__device__ __forceinline__ uint32_t wg_max(uint32_t v, uint32_t* red)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, off);
        v = o > v ? o : v;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < ST_THREADS / 64; ++w) t = red[w] > t ? red[w] : t;
    __syncthreads();
    return t;
}

// The fp32 values of unit u (8 elements when VEC, else 1) handed to f(float, bits).
template <bool BF16, bool VEC, typename F>
__device__ __forceinline__ void visit_unit(const uint8_t* x, int64_t ldx_bytes, FastDiv upr_div, uint32_t upr,
                                           uint32_t u, F&& f)
{
    constexpr int ESZ = BF16 ? 2 : 4;
    const uint32_t row = upr_div.div(u);
    const uint32_t c = u - row * upr;
    if constexpr (VEC) {
        const u32x4* p = reinterpret_cast<const u32x4*>(x + (int64_t)row * ldx_bytes + (int64_t)c * (8 * ESZ));
        if constexpr (BF16) {
            const u32x4 v = p[0];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f(w[j] << 16);
                f(w[j] & 0xFFFF0000u);
            }
        } else {
            const u32x4 v0 = p[0], v1 = p[1];
            const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) f(w[j]);
        }
    } else {
        const uint8_t* p = x + (int64_t)row * ldx_bytes + (int64_t)c * ESZ;
        if constexpr (BF16) f((uint32_t)*reinterpret_cast<const uint16_t*>(p) << 16);
        else f(*reinterpret_cast<const uint32_t*>(p));
    }
}

// pass 1: partials[2 g] = sum of x, partials[2 g + 1] = max |x| (as a double) of workgroup g
template <bool BF16, bool VEC>
__global__ __launch_bounds__(ST_THREADS) void stats_sum_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                                FastDiv upr_div, uint32_t upr, uint32_t total,
                                                                double* __restrict__ partials)
{
    __shared__ double dred[ST_THREADS / 64];
    __shared__ uint32_t ured[ST_THREADS / 64];
    double s = 0.0;
    uint32_t am = 0;
    const uint32_t stride = gridDim.x * ST_THREADS;
    for (uint32_t u = blockIdx.x * ST_THREADS + threadIdx.x; u < total; u += stride)
        visit_unit<BF16, VEC>(x, ldx_bytes, upr_div, upr, u, [&](uint32_t b) {
            s += (double)u2f(b);
            const uint32_t a = b & 0x7FFFFFFFu;
            am = a > am ? a : am;
        });
    const double ts = wg_sum(s, dred);
    const uint32_t tm = wg_max(am, ured);
    if (threadIdx.x == 0) {
        partials[2 * (int64_t)blockIdx.x] = ts;
        partials[2 * (int64_t)blockIdx.x + 1] = (double)u2f(tm);
    }
}

// pass 2: partials[g] = sum of (x - mean)^2 over workgroup g's units
template <bool BF16, bool VEC>
__global__ __launch_bounds__(ST_THREADS) void stats_m2_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                               FastDiv upr_div, uint32_t upr, uint32_t total,
                                                               const double* __restrict__ mean_p,
                                                               double* __restrict__ partials)
{
    __shared__ double dred[ST_THREADS / 64];
    const double mean = *mean_p;
    double s = 0.0;
    const uint32_t stride = gridDim.x * ST_THREADS;
    for (uint32_t u = blockIdx.x * ST_THREADS + threadIdx.x; u < total; u += stride)
        visit_unit<BF16, VEC>(x, ldx_bytes, upr_div, upr, u, [&](uint32_t b) {
            const double d = (double)u2f(b) - mean;
            s = __builtin_fma(d, d, s);
        });
    const double t = wg_sum(s, dred);
    if (threadIdx.x == 0) partials[(int64_t)blockIdx.x] = t;
}

// one workgroup over the partials; PASS 1 writes out[0] = mean and out[2] = max |x|,
// PASS 2 writes out[1] = sqrt(M2 / (n - 1)) (NaN for n == 1)
template <int PASS>
__global__ __launch_bounds__(ST_THREADS) void stats_finish_kernel(const double* __restrict__ partials, int groups,
                                                                   double n, double* __restrict__ out)
{
    __shared__ double dred[ST_THREADS / 64];
    __shared__ uint32_t ured[ST_THREADS / 64];
    constexpr int NP = PASS == 1 ? 2 : 1;
    double s = 0.0, m = 0.0;
    for (int gi = threadIdx.x; gi < groups; gi += ST_THREADS) {
        s += partials[(int64_t)gi * NP];
        if constexpr (PASS == 1) m = partials[(int64_t)gi * NP + 1] > m ? partials[(int64_t)gi * NP + 1] : m;
    }
    const double ts = wg_sum(s, dred);
    if constexpr (PASS == 1) {
        // max of non-negative doubles = max of their bit patterns
        const uint64_t mb = __builtin_bit_cast(uint64_t, m);
        const uint32_t hi = wg_max((uint32_t)(mb >> 32), ured);
        const uint32_t lo = wg_max((uint32_t)(mb >> 32) == hi ? (uint32_t)mb : 0u, ured);
        if (threadIdx.x == 0) {
            out[0] = ts / n;
            out[2] = __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
        }
    } else {
        if (threadIdx.x == 0) out[1] = n > 1.0 ? sqrt(ts / (n - 1.0)) : __builtin_nan("");
    }
}

int stats_groups(int64_t rows, int64_t k)
{
    const int64_t units = rows * ((k % 8 == 0) ? k / 8 : k);  // an upper bound on either path's units
    const int64_t g = (units + ST_THREADS - 1) / ST_THREADS;
    return (int)(g < kStatsMaxGroups ? (g > 0 ? g : 1) : kStatsMaxGroups);
}

template <bool BF16, bool VEC>
static hipError_t launch_stats_t(const StatsArgs& a, hipStream_t st)
{
    constexpr int ESZ = BF16 ? 2 : 4;
    const uint32_t upr = (uint32_t)(VEC ? a.k / 8 : a.k);
    const uint32_t total = (uint32_t)(a.rows * upr);
    const int64_t g = ((int64_t)total + ST_THREADS - 1) / ST_THREADS;
    const int groups = (int)(g < kStatsMaxGroups ? g : kStatsMaxGroups);
    const FastDiv fd = FastDiv::make(upr);
    const uint8_t* x = static_cast<const uint8_t*>(a.x);
    const double n = (double)(a.rows * a.k);
    hipLaunchKernelGGL((stats_sum_kernel<BF16, VEC>), dim3(groups), dim3(ST_THREADS), 0, st, x, a.ldx * ESZ, fd, upr,
                       total, a.partials);
    hipLaunchKernelGGL((stats_finish_kernel<1>), dim3(1), dim3(ST_THREADS), 0, st, a.partials, groups, n, a.out);
    hipLaunchKernelGGL((stats_m2_kernel<BF16, VEC>), dim3(groups), dim3(ST_THREADS), 0, st, x, a.ldx * ESZ, fd, upr,
                       total, a.out, a.partials);
    hipLaunchKernelGGL((stats_finish_kernel<2>), dim3(1), dim3(ST_THREADS), 0, st, a.partials, groups, n, a.out);
    return hipGetLastError();
}

hipError_t launch_tensor_stats(const StatsArgs& a, hipStream_t st)
{
    if (a.bf16) return a.vec ? launch_stats_t<true, true>(a, st) : launch_stats_t<true, false>(a, st);
    return a.vec ? launch_stats_t<false, true>(a, st) : launch_stats_t<false, false>(a, st);
}

}  // namespace mxk
