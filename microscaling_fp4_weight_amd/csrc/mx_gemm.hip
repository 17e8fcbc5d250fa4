// mx_gemm.hip -- Y = X . dequant(Wq)^T for MX FP4 weights on gfx950.
//
// Method: gtnt.cn/news/16247 "为什么我们需要4-bit浮点量化", section 3.1 (dequantize, then
// matmul) and section 4.3 (keep weights quantized; small batches stay quantized, large
// batches dequantize on the fly); hotelren.com/news/2192771, article "量化技术演进与微缩量化
// 原理", section 3.2 item 3 (load FP4 block -> unpack -> load FP8 scale -> multiply ->
// accumulate).  Here the dequantized weights never touch memory: they are produced in
// registers and fed to the matrix cores.
//
// W4A16 (bf16 activations): v_mfma_f32_16x16x32_bf16.  A lane that supplies weights for
// column n reads the 16 code bytes covering 32 consecutive k of row n (one 128-bit load,
// one E8M0 block), converts them with v_cvt_scalef32_pk_bf16_fp4 and feeds four MFMA k-steps.
// The k order inside the 128-wide k-tile is permuted identically for both operands (lane
// group q, step j, element i  <->  k = 32q + 8j + i), which leaves every dot product intact.
// W4A4: v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 operands; in the row-major layout a
// lane's 16 code bytes and its E8M0 byte are exactly one MFMA operand slice and its scale.
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

// Scales covering one lane's 32 k: BLOCK >= 32 -> one byte; else 32/BLOCK bytes packed.
template <int BLOCK>
__device__ __forceinline__ uint64_t load_lane_scales(const uint8_t* p)
{
    if constexpr (BLOCK >= 32) return *p;
    else if constexpr (BLOCK == 16) return *reinterpret_cast<const uint16_t*>(p);
    else if constexpr (BLOCK == 8) return *reinterpret_cast<const uint32_t*>(p);
    else return *reinterpret_cast<const uint64_t*>(p);
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

__device__ __forceinline__ f32x4 mfma_bf16(const uint32_t* a4, const uint32_t* b4, f32x4 c)
{
    const u32x4 av = {a4[0], a4[1], a4[2], a4[3]};
    const u32x4 bv = {b4[0], b4[1], b4[2], b4[3]};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                   __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
}

template <bool OUT_BF16>
__device__ __forceinline__ void store_y(void* y, int64_t ldy, int64_t m, int64_t n, float v)
{
    if constexpr (OUT_BF16) reinterpret_cast<__bf16*>(y)[m * ldy + n] = (__bf16)v;
    else reinterpret_cast<float*>(y)[m * ldy + n] = v;
}

// ---------------------------------------------------------------------------------------
// W4A16 GEMM: workgroup tile 128 x 128, 4 waves in a 2 x 2 grid, each 64 x 64
// (4 x 4 MFMA tiles of 16 x 16), k-tile 128.  X staged through LDS; weights loaded per
// wave straight into registers and dequantized there.
// ---------------------------------------------------------------------------------------
constexpr int TM = 128, TN = 128, TK = 128;
constexpr int XS_STRIDE = TK * 2 + 16;  // bytes per LDS row of the X tile (+16 B against bank conflicts)

template <int BLOCK, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_a16_kernel(const GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t xs[TM * XS_STRIDE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
    const int lr = lane & 15, kq = lane >> 4;
    const int64_t K = a.k;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t k0 = 0; k0 < K; k0 += TK) {
        // X tile -> LDS: 128 rows x 256 B = 2048 chunks of 16 B, 8 per thread
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int chunk = tid + 256 * c;
            const int r = chunk >> 4, c16 = chunk & 15;
            const int64_t gm = m0 + r, gk = k0 + 8 * c16;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (gm < a.m && gk < K) v = *reinterpret_cast<const u32x4*>(a.x + gm * a.ldx + gk);
            *reinterpret_cast<u32x4*>(xs + r * XS_STRIDE + c16 * 16) = v;
        }
        // weights for this wave's 4 n-subtiles
        uint32_t bw[4][16];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
            const int64_t n = n0 + wn * 64 + ns * 16 + lr;
            const int64_t kk = k0 + 32 * kq;
            u32x4 cw = {0u, 0u, 0u, 0u};
            uint64_t sb = 0;
            if (n < a.n && kk < K) {
                cw = *reinterpret_cast<const u32x4*>(a.wc + n * (K / 2) + kk / 2);
                sb = load_lane_scales<BLOCK>(a.ws + n * (K / BLOCK) + kk / BLOCK);
            }
            dequant32<BLOCK, FMT>(cw, sb, bw[ns]);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t af[4][4];
#pragma unroll
            for (int ms = 0; ms < 4; ++ms) {
                const int r = wm * 64 + ms * 16 + lr;
                const u32x4 v = *reinterpret_cast<const u32x4*>(xs + r * XS_STRIDE + (32 * kq + 8 * j) * 2);
                af[ms][0] = v.x; af[ms][1] = v.y; af[ms][2] = v.z; af[ms][3] = v.w;
            }
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = mfma_bf16(af[ms], &bw[ns][4 * j], acc[ms][ns]);
        }
        __syncthreads();
    }
    // epilogue: C layout of a 16x16 tile: lane holds rows 4*(lane/16)+i, column lane%16
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
            const int64_t n = n0 + wn * 64 + ns * 16 + lr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t m = m0 + wm * 64 + ms * 16 + 4 * kq + i;
                if (m < a.m && n < a.n) store_y<OUT_BF16>(a.y, a.ldy, m, n, acc[ms][ns][i] * a.g);
            }
        }
}

// ---------------------------------------------------------------------------------------
// W4A16 GEMV (m <= 16): one MFMA row-tile; a workgroup of 4 waves owns 16 * NS columns,
// the waves take interleaved k-tiles and their partial sums are added through LDS.
// ---------------------------------------------------------------------------------------
constexpr int GEMV_NS = 2;

template <int BLOCK, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemv_a16_kernel(const GemmArgs a)
{
    __shared__ f32x4 red[3][GEMV_NS][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, kq = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * GEMV_NS);
    const int64_t K = a.k;
    const bool mrow = lr < a.m;

    f32x4 acc[GEMV_NS];
#pragma unroll
    for (int ns = 0; ns < GEMV_NS; ++ns) acc[ns] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t k0 = (int64_t)wave * TK; k0 < K; k0 += 4 * TK) {
        const int64_t kk = k0 + 32 * kq;
        const bool kin = kk < K;
        u32x4 cw[GEMV_NS];
        uint64_t sb[GEMV_NS];
#pragma unroll
        for (int ns = 0; ns < GEMV_NS; ++ns) {
            const int64_t n = n0 + ns * 16 + lr;
            cw[ns] = u32x4{0u, 0u, 0u, 0u};
            sb[ns] = 0;
            if (n < a.n && kin) {
                cw[ns] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.wc + n * (K / 2) + kk / 2));
                sb[ns] = load_lane_scales<BLOCK>(a.ws + n * (K / BLOCK) + kk / BLOCK);
            }
        }
        uint32_t xf[16];
        {
            const u32x4* xp = reinterpret_cast<const u32x4*>(a.x + (int64_t)lr * a.ldx + kk);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (mrow && kin) v = xp[j];
                xf[4 * j] = v.x; xf[4 * j + 1] = v.y; xf[4 * j + 2] = v.z; xf[4 * j + 3] = v.w;
            }
        }
#pragma unroll
        for (int ns = 0; ns < GEMV_NS; ++ns) {
            uint32_t bw[16];
            dequant32<BLOCK, FMT>(cw[ns], sb[ns], bw);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[ns] = mfma_bf16(&xf[4 * j], &bw[4 * j], acc[ns]);
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int ns = 0; ns < GEMV_NS; ++ns) red[wave - 1][ns][lane] = acc[ns];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int ns = 0; ns < GEMV_NS; ++ns) {
            f32x4 s = acc[ns] + red[0][ns][lane] + red[1][ns][lane] + red[2][ns][lane];
            const int64_t n = n0 + ns * 16 + lr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t m = 4 * kq + i;
                if (m < a.m && n < a.n) store_y<OUT_BF16>(a.y, a.ldy, m, n, s[i] * a.g);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// W4A4 GEMM: block-scaled FP4 MFMA 16x16x128; workgroup tile 128 x 128 (2 x 2 waves of
// 64 x 64), k-tile 128 = one MFMA k-step.  Each lane loads its 16 code bytes and scale byte
// for every m- and n-subtile straight from the row-major arrays.
// ---------------------------------------------------------------------------------------
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_a4_kernel(const GemmArgs a)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
    const int lr = lane & 15, kq = lane >> 4;
    const int64_t K = a.k;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t k0 = 0; k0 < K; k0 += TK) {
        const int64_t kk = k0 + 32 * kq;
        i32x8 af[4], bf[4];
        int as[4], bs[4];
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
            const int64_t m = m0 + wm * 64 + ms * 16 + lr;
            u32x4 v = {0u, 0u, 0u, 0u};
            int s = 127;
            if (m < a.m && kk < K) {
                v = *reinterpret_cast<const u32x4*>(a.xq_codes + m * (K / 2) + kk / 2);
                s = a.xq_scales[m * (K / 32) + kk / 32];
            }
            af[ms] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            as[ms] = s;
        }
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
            const int64_t n = n0 + wn * 64 + ns * 16 + lr;
            u32x4 v = {0u, 0u, 0u, 0u};
            int s = 127;
            if (n < a.n && kk < K) {
                v = *reinterpret_cast<const u32x4*>(a.wc + n * (K / 2) + kk / 2);
                s = a.ws[n * (K / 32) + kk / 32];
            }
            bf[ns] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            bs[ns] = s;
        }
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int ns = 0; ns < 4; ++ns)
                acc[ms][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[ms], bf[ns], acc[ms][ns], 4, 4, 0, as[ms], 0, bs[ns]);
    }
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
            const int64_t n = n0 + wn * 64 + ns * 16 + lr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t m = m0 + wm * 64 + ms * 16 + 4 * kq + i;
                if (m < a.m && n < a.n) store_y<OUT_BF16>(a.y, a.ldy, m, n, acc[ms][ns][i] * a.g);
            }
        }
}

// ---------------------------------------------------------------------------------------
// Generic path (any shape the fast kernels do not take): one thread per output element,
// fp32 accumulation over element pairs.
// ---------------------------------------------------------------------------------------
template <int FMT, bool A4, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const GemmArgs a)
{
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= a.m * a.n) return;
    const int64_t m = id / a.n, n = id - m * a.n;
    const int64_t K = a.k;
    float acc = 0.0f;
    for (int64_t kp = 0; kp < K / 2; ++kp) {
        const uint32_t cb = a.wc[n * (K / 2) + kp];
        const uint32_t sbyte = a.ws[n * (K / a.block) + (2 * kp) / a.block];
        float w0, w1;
        if constexpr (FMT == FMT_E8M0) {
            const f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cb, e8m0_value(sbyte), 0);
            w0 = f.x; w1 = f.y;
        } else {
            const DecG1 p = dec_params_g1<FMT>(sbyte);
            const f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cb, p.pow2, 0);
            w0 = f.x * p.mant; w1 = f.y * p.mant;
        }
        float x0, x1;
        if constexpr (A4) {
            const uint32_t xb = a.xq_codes[m * (K / 2) + kp];
            const f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(
                xb, e8m0_value(a.xq_scales[m * (K / 32) + (2 * kp) / 32]), 0);
            x0 = f.x; x1 = f.y;
        } else {
            x0 = u2f((uint32_t)a.x[m * a.ldx + 2 * kp] << 16);
            x1 = u2f((uint32_t)a.x[m * a.ldx + 2 * kp + 1] << 16);
        }
        acc = __builtin_fmaf(x0, w0, acc);
        acc = __builtin_fmaf(x1, w1, acc);
    }
    store_y<OUT_BF16>(a.y, a.ldy, m, n, acc * a.g);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint8_t* y, int64_t m, int64_t n, int64_t ldy, int esize)
{
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= m * n) return;
    const int64_t r = id / n, c = id - r * n;
    if (esize == 2) reinterpret_cast<uint16_t*>(y)[r * ldy + c] = 0;
    else reinterpret_cast<uint32_t*>(y)[r * ldy + c] = 0;
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
hipError_t launch_fill_zero(void* y, int64_t m, int64_t n, int64_t ldy, bool bf16, hipStream_t st)
{
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((m * n + 255) / 256)), dim3(256), 0, st,
                       (uint8_t*)y, m, n, ldy, bf16 ? 2 : 4);
    return hipGetLastError();
}

template <int FMT, bool OUT_BF16>
static hipError_t launch_a16_fmt(const GemmArgs& a, hipStream_t st)
{
    const bool fast = (a.k % 32 == 0) && ((a.ldx * 2) % 16 == 0) && ((uintptr_t)a.x % 16 == 0);
    if (!fast) {
        const int64_t total = a.m * a.n;
        hipLaunchKernelGGL((gemm_generic_kernel<FMT, false, OUT_BF16>), dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, st, a);
        return hipGetLastError();
    }
    if (a.m <= 16) {
        const dim3 grid((unsigned)((a.n + 16 * GEMV_NS - 1) / (16 * GEMV_NS)));
        switch (a.block) {
#define MXV(B) case B: hipLaunchKernelGGL((gemv_a16_kernel<B, FMT, OUT_BF16>), grid, dim3(256), 0, st, a); break;
            MXV(4) MXV(8) MXV(16) MXV(32) MXV(64) MXV(128) MXV(256)
#undef MXV
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((a.n + TN - 1) / TN), (unsigned)((a.m + TM - 1) / TM));
    switch (a.block) {
#define MXG(B) case B: hipLaunchKernelGGL((gemm_a16_kernel<B, FMT, OUT_BF16>), grid, dim3(256), 0, st, a); break;
        MXG(4) MXG(8) MXG(16) MXG(32) MXG(64) MXG(128) MXG(256)
#undef MXG
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_a16(const GemmArgs& a, hipStream_t st)
{
#define MXF(F) if (a.fmt == F) return a.y_bf16 ? launch_a16_fmt<F, true>(a, st) : launch_a16_fmt<F, false>(a, st);
    MXF(FMT_E4M3) MXF(FMT_UE5M3) MXF(FMT_E8M0)
#undef MXF
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_a4(const GemmArgs& a, hipStream_t st)
{
    // activations were quantized into the workspace (block 32, E8M0) by the caller
    const dim3 grid((unsigned)((a.n + TN - 1) / TN), (unsigned)((a.m + TM - 1) / TM));
    if (a.y_bf16) hipLaunchKernelGGL((gemm_a4_kernel<true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((gemm_a4_kernel<false>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace mxk
