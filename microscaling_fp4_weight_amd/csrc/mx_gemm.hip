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
// W4A16 GEMV (m <= 16): one MFMA row-tile.  A workgroup owns 16 output columns; its
// GEMV_WAVES waves take contiguous k ranges.  Each wave keeps GEMV_DEPTH k-tiles of weight
// and activation loads in flight (a rolling prefetch: tile t + GEMV_DEPTH is requested as
// soon as tile t has been consumed); the waves' partial sums are added through LDS.
// ---------------------------------------------------------------------------------------
constexpr int GEMV_WAVES = 4;
constexpr int GEMV_DEPTH = 4;

template <int BLOCK>
struct GemvTile {
    u32x4 cw;         // 32 weight codes of row n
    uint64_t sb;      // their scale byte(s)
    u32x4 xv[4];      // 32 activations of row lr (zero for rows >= m)
};

// Scales covering one lane's 32 k through a buffer resource (zero when out of range).
template <int BLOCK>
__device__ __forceinline__ uint64_t bload_lane_scales(rsrc_t r, uint32_t off)
{
    if constexpr (BLOCK >= 32) return bload8(r, off);
    else if constexpr (BLOCK == 16) return bload16(r, off);
    else if constexpr (BLOCK == 8) return bload32(r, off);
    else return bload64(r, off);
}

struct GemvRows {
    rsrc_t w, s, x;          // this workgroup's 16 weight rows, their scales, the activations
    uint32_t woff, soff, xoff;  // this lane's row offsets (bytes)
    uint32_t K;
};

template <int BLOCK>
__device__ __forceinline__ void gemv_load(GemvTile<BLOCK>& t, int64_t tile, int64_t t1, int kq,
                                          const GemvRows& r)
{
    const uint32_t kk = (uint32_t)tile * TK + 32 * kq;
    const bool ok = tile < t1 && kk < r.K;
    t.cw = bload128(r.w, ok ? r.woff + kk / 2 : kOOB);
    t.sb = bload_lane_scales<BLOCK>(r.s, ok ? r.soff + kk / BLOCK : kOOB);
#pragma unroll
    for (int j = 0; j < 4; ++j) t.xv[j] = bload128(r.x, ok ? r.xoff + (kk + 8 * j) * 2 : kOOB);
}

template <int BLOCK, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_a16_kernel(const GemmArgs a)
{
    __shared__ f32x4 red[GEMV_WAVES - 1][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, kq = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t n = n0 + lr;
    const uint32_t K = (uint32_t)a.k;
    const int64_t KT = (a.k + TK - 1) / TK;
    const int64_t per = (KT + GEMV_WAVES - 1) / GEMV_WAVES;
    const int64_t t0 = wave * per;
    const int64_t t1 = t0 + per < KT ? t0 + per : KT;
    const uint32_t rows = (uint32_t)(a.n - n0 < 16 ? a.n - n0 : 16);

    GemvRows r;
    r.w = make_rsrc(a.wc + n0 * (a.k / 2), rows * (K / 2));
    r.s = make_rsrc(a.ws + n0 * (a.k / BLOCK), rows * (K / BLOCK));
    r.x = make_rsrc(a.x, (uint32_t)(a.m * a.ldx * 2));
    r.woff = lr * (K / 2);
    r.soff = lr * (K / BLOCK);
    r.xoff = (uint32_t)(lr * a.ldx * 2);
    r.K = K;

    GemvTile<BLOCK> buf[GEMV_DEPTH];
#pragma unroll
    for (int p = 0; p < GEMV_DEPTH; ++p) gemv_load<BLOCK>(buf[p], t0 + p, t1, kq, r);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t tb = t0; tb < t1; tb += GEMV_DEPTH) {
#pragma unroll
        for (int p = 0; p < GEMV_DEPTH; ++p) {
            uint32_t bw[16];
            dequant32<BLOCK, FMT>(buf[p].cw, buf[p].sb, bw);
            const u32x4 x0 = buf[p].xv[0], x1 = buf[p].xv[1], x2 = buf[p].xv[2], x3 = buf[p].xv[3];
            gemv_load<BLOCK>(buf[p], tb + p + GEMV_DEPTH, t1, kq, r);
            const uint32_t xf[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                     x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = mfma_bf16(&xf[4 * j], &bw[4 * j], acc);
        }
    }
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < GEMV_WAVES - 1; ++w) acc += red[w][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = 4 * kq + i;
            if (m < a.m && n < a.n) store_y<OUT_BF16>(a.y, a.ldy, m, n, acc[i] * a.g);
        }
    }
}

// ---------------------------------------------------------------------------------------
// W4A16 GEMV for m <= 4 on the vector ALUs.  A workgroup owns DOT_ROWS weight rows; its 4
// waves split k into contiguous ranges of 2048-element chunks.  In a chunk, lane l holds the
// 32 activations k = c*2048 + 32 l .. +31 of every row of X in registers (reused for all
// DOT_ROWS weight rows) and, per weight row, loads that row's 16 code bytes for the same k
// -- one load instruction reads 1 KB of contiguous codes.  Products are accumulated with
// v_dot2_f32_bf16 into per-lane partial sums, which are reduced across the wave and then
// across the 4 waves at the end.
// ---------------------------------------------------------------------------------------
constexpr int DOT_ROWS = 8;
constexpr int DOT_WAVES = 4;
constexpr int DOT_CHUNK = 2048;

template <int BLOCK, int FMT, int MM, bool OUT_BF16>
__global__ __launch_bounds__(64 * DOT_WAVES) void gemv_dot_kernel(const GemmArgs a)
{
    __shared__ float red[DOT_WAVES][DOT_ROWS * MM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * DOT_ROWS;
    const uint32_t K = (uint32_t)a.k;
    const uint32_t nrows = (uint32_t)(a.n - n0 < DOT_ROWS ? a.n - n0 : DOT_ROWS);
    const int64_t KC = (a.k + DOT_CHUNK - 1) / DOT_CHUNK;
    const int64_t per = (KC + DOT_WAVES - 1) / DOT_WAVES;
    const int64_t c0 = wave * per;
    const int64_t c1 = c0 + per < KC ? c0 + per : KC;

    const rsrc_t wr = make_rsrc(a.wc + n0 * (a.k / 2), nrows * (K / 2));
    const rsrc_t sr = make_rsrc(a.ws + n0 * (a.k / BLOCK), nrows * (K / BLOCK));
    const rsrc_t xr = make_rsrc(a.x, (uint32_t)(a.m * a.ldx * 2));

    float acc[DOT_ROWS][MM];
#pragma unroll
    for (int r = 0; r < DOT_ROWS; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[r][m] = 0.0f;

    for (int64_t c = c0; c < c1; ++c) {
        const uint32_t kk = (uint32_t)c * DOT_CHUNK + 32 * lane;
        const bool ok = kk < K;
        u32x4 cw[DOT_ROWS];
        uint64_t sb[DOT_ROWS];
#pragma unroll
        for (int r = 0; r < DOT_ROWS; ++r) {
            cw[r] = bload128(wr, ok ? r * (K / 2) + kk / 2 : kOOB);
            sb[r] = bload_lane_scales<BLOCK>(sr, ok ? r * (K / BLOCK) + kk / BLOCK : kOOB);
        }
        uint32_t xf[MM][16];
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 v = bload128(xr, ok && m < a.m ? (uint32_t)(m * a.ldx * 2) + (kk + 8 * j) * 2 : kOOB);
                xf[m][4 * j] = v.x; xf[m][4 * j + 1] = v.y; xf[m][4 * j + 2] = v.z; xf[m][4 * j + 3] = v.w;
            }
#pragma unroll
        for (int r = 0; r < DOT_ROWS; ++r) {
            uint32_t bw[16];
            dequant32<BLOCK, FMT>(cw[r], sb[r], bw);
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[r][m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xf[m][i]),
                                                                __builtin_bit_cast(bf16x2, bw[i]),
                                                                acc[r][m], false);
        }
    }
    // reduce over the 64 lanes, then over the waves
#pragma unroll
    for (int r = 0; r < DOT_ROWS; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            float v = acc[r][m];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            acc[r][m] = v;
        }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < DOT_ROWS; ++r)
#pragma unroll
            for (int m = 0; m < MM; ++m) red[wave][r * MM + m] = acc[r][m];
    }
    __syncthreads();
    if (tid < DOT_ROWS * MM) {
        const int r = tid / MM, m = tid % MM;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < DOT_WAVES; ++w) v += red[w][tid];
        if (m < a.m && (uint32_t)r < nrows) store_y<OUT_BF16>(a.y, a.ldy, m, n0 + r, v * a.g);
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
    if (a.m <= 4) {
        const dim3 grid((unsigned)((a.n + DOT_ROWS - 1) / DOT_ROWS));
        switch (a.block) {
#define MXD1(B) case B: \
    if (a.m == 1) hipLaunchKernelGGL((gemv_dot_kernel<B, FMT, 1, OUT_BF16>), grid, dim3(64 * DOT_WAVES), 0, st, a); \
    else hipLaunchKernelGGL((gemv_dot_kernel<B, FMT, 4, OUT_BF16>), grid, dim3(64 * DOT_WAVES), 0, st, a); \
    break;
            MXD1(4) MXD1(8) MXD1(16) MXD1(32) MXD1(64) MXD1(128) MXD1(256)
#undef MXD1
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (a.m <= 16) {
        const dim3 grid((unsigned)((a.n + 15) / 16));
        switch (a.block) {
#define MXV(B) case B: hipLaunchKernelGGL((gemv_a16_kernel<B, FMT, OUT_BF16>), grid, dim3(64 * GEMV_WAVES), 0, st, a); break;
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
    if (a4_uses_mfma(a)) return launch_gemm_a4_mfma(a, st);
    if (a.ws_tiled) return hipErrorInvalidValue;  // the direct kernel reads row-major scales
    const dim3 grid((unsigned)((a.n + TN - 1) / TN), (unsigned)((a.m + TM - 1) / TM));
    if (a.y_bf16) hipLaunchKernelGGL((gemm_a4_kernel<true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((gemm_a4_kernel<false>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace mxk
