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
#include "mx_wdeq.h"

namespace mxk {


// Scales covering one lane's 32 k: BLOCK >= 32 -> one byte; else 32/BLOCK bytes packed.
template <int BLOCK>
__device__ __forceinline__ uint64_t load_lane_scales(const uint8_t* p)
{
    if constexpr (BLOCK >= 32) return *p;
    else if constexpr (BLOCK == 16) return *reinterpret_cast<const uint16_t*>(p);
    else if constexpr (BLOCK == 8) return *reinterpret_cast<const uint32_t*>(p);
    else return *reinterpret_cast<const uint64_t*>(p);
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

// Scales covering one lane's 32 k through a buffer resource (zero when out of range).
template <int BLOCK>
__device__ __forceinline__ uint64_t bload_lane_scales(rsrc_t r, uint32_t off)
{
    if constexpr (BLOCK >= 32) return bload8(r, off);
    else if constexpr (BLOCK == 16) return bload16(r, off);
    else if constexpr (BLOCK == 8) return bload32(r, off);
    else return bload64(r, off);
}

// ---------------------------------------------------------------------------------------
// W4A16 GEMV for 2 <= m <= 16 with the activations in LDS.  The activations (m rows of X)
// are what every workgroup needs in full while it needs only its own weight rows, so they are
// brought into LDS once per workgroup and 4096-element chunk (LDS-DMA, 1 KB per load) instead
// of being re-read per 16-row weight tile through the load unit.  A workgroup owns up to 16
// weight tiles of 16 rows (tile t of workgroup b is b + t * grid); its 8 waves split each
// chunk's k four ways.  For a tile, a lane holds weight row lane%16 and the 32 consecutive k
// 32*(lane/16) .. +31 of every 128-k step (one 16-byte code load), dequantizes them in
// registers, and feeds 16x16x32 bf16 MFMAs with the matching activations from LDS: k is
// permuted the same way for both operands, which leaves the dot product unchanged.  The next
// tile's weight loads are in flight while a tile is computed.  Partial sums of the 8 waves
// meet in LDS at the end.
// ---------------------------------------------------------------------------------------
constexpr int GL_WAVES = 8;                       // two per SIMD
constexpr int GL_KC = 4096;                       // k per LDS chunk of X
constexpr int GL_PITCH = 2 * GL_KC + 16;          // LDS bytes per X row (padded: rows start 4 banks apart)
constexpr int GL_TMAX = 16;                       // 16-row weight tiles per workgroup
constexpr int GL_KTW = GL_KC / TK / GL_WAVES;     // 128-k steps per wave per chunk
constexpr int GL_RED = GL_WAVES * GL_TMAX * 64 * 16;  // bytes of the cross-wave reduction

template <int BLOCK>
struct GlW {
    u32x4 cw[GL_KTW];      // 32 codes of the lane's row per 128-k step
    uint64_t sb[GL_KTW];   // their scale byte(s) (blocks below 32)
    u32x4 srow;            // blocks of 32 and more: the row's scale bytes of the wave's k range
};

// Scale byte(s) of the lane's 32 k in 128-k step kt (kq = lane / 16).  For blocks of 32 and
// more, the 512 k of a wave's range have at most 16 scale bytes per row, which one load per
// lane brings at once (the four lanes of a row read the same bytes) instead of one scattered
// byte per step; k past the end gets the format's byte for 1.0 (its codes are zero, so any
// finite scale gives zero products).
template <int BLOCK, int FMT>
__device__ __forceinline__ uint64_t gl_scale(const GlW<BLOCK>& w, int kt, int kq, bool ok)
{
    if constexpr (BLOCK >= 32) {
        constexpr uint32_t one = FMT == FMT_E8M0 ? 127u : FMT == FMT_E4M3 ? 0x38u : 0x78u;
        const int dw = (kt * TK / BLOCK) / 4;                     // dword holding the byte (constant once kt is)
        const uint32_t idx = (uint32_t)(kt * TK + 32 * kq) / BLOCK;
        const uint32_t v = dw == 0 ? w.srow.x : dw == 1 ? w.srow.y : dw == 2 ? w.srow.z : w.srow.w;
        return ok ? (v >> (8 * (idx & 3))) & 0xFFu : one;
    } else {
        return w.sb[kt];
    }
}

template <int BLOCK>
__device__ __forceinline__ void gl_load(GlW<BLOCK>& w, const GemmArgs& a, uint32_t tile, uint32_t k0,
                                        int lr, int kq)
{
    const uint32_t K = (uint32_t)a.k;
    const int64_t n0 = (int64_t)tile * 16;
    const uint32_t rows = (uint32_t)(a.n - n0 < 16 ? a.n - n0 : 16);
    const rsrc_t wr = make_rsrc(a.wc + n0 * (a.k / 2), rows * (K / 2));
    // the scale range is rounded up to whole dwords: the dword holding a tile's last scale byte
    // lies in the same page as that byte, and bytes past the end are never used
    const rsrc_t sr = make_rsrc(a.ws + n0 * (a.k / BLOCK), (rows * (K / BLOCK) + 3) & ~3u);
#pragma unroll
    for (int kt = 0; kt < GL_KTW; ++kt) {
        const uint32_t kk = k0 + kt * TK + 32 * kq;
        const bool ok = kk < K;
        w.cw[kt] = bload128(wr, ok ? lr * (K / 2) + kk / 2 : kOOB);
        if constexpr (BLOCK < 32) w.sb[kt] = bload_lane_scales<BLOCK>(sr, ok ? lr * (K / BLOCK) + kk / BLOCK : kOOB);
    }
    if constexpr (BLOCK >= 32) {
        static_assert(GL_KTW * TK / BLOCK <= 16, "scale bytes of a wave's range exceed one load");
        constexpr int NB = GL_KTW * TK / BLOCK;                    // 16, 8, 4 or 2 bytes
        // rows of scales need not start on a dword: load whole dwords from the aligned address
        // below and shift the wanted bytes down with v_alignbyte
        const bool in = k0 < K;
        const uint32_t off = lr * (K / BLOCK) + k0 / BLOCK, a0 = off & ~3u, sh = off & 3u;
        if constexpr (NB == 16) {
            const u32x4 lo = bload128(sr, in ? a0 : kOOB);
            const uint32_t hi = bload32(sr, in ? a0 + 16 : kOOB);
            w.srow = u32x4{__builtin_amdgcn_alignbyte(lo.y, lo.x, sh), __builtin_amdgcn_alignbyte(lo.z, lo.y, sh),
                           __builtin_amdgcn_alignbyte(lo.w, lo.z, sh), __builtin_amdgcn_alignbyte(hi, lo.w, sh)};
        } else if constexpr (NB == 8) {
            const uint64_t lo = bload64(sr, in ? a0 : kOOB);
            const uint32_t hi = bload32(sr, in ? a0 + 8 : kOOB);
            const uint32_t l0 = (uint32_t)lo, l1 = (uint32_t)(lo >> 32);
            w.srow = u32x4{__builtin_amdgcn_alignbyte(l1, l0, sh), __builtin_amdgcn_alignbyte(hi, l1, sh), 0u, 0u};
        } else {
            const uint32_t l0 = bload32(sr, in ? a0 : kOOB), l1 = bload32(sr, in ? a0 + 4 : kOOB);
            w.srow = u32x4{__builtin_amdgcn_alignbyte(l1, l0, sh), 0u, 0u, 0u};
        }
    }
}

template <int BLOCK, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(64 * GL_WAVES) void gemv_lds_kernel(const GemmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    typedef __attribute__((address_space(3))) void lds_void;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, kq = lane >> 4;
    const uint32_t K = (uint32_t)a.k, M = (uint32_t)a.m;
    const uint32_t T = (uint32_t)((a.n + 15) / 16), G = gridDim.x;
    const uint32_t ntiles = (T - blockIdx.x + G - 1) / G;  // at most GL_TMAX (launch)
    const rsrc_t xr = make_rsrc(a.x, (uint32_t)(((int64_t)(M - 1) * a.ldx + K) * 2));
    const uint32_t ldx = (uint32_t)a.ldx;
    const uint32_t xrow = (uint32_t)lr < M ? (uint32_t)lr : 0u;  // rows >= m feed outputs never stored

    f32x4 acc[GL_TMAX];
#pragma unroll
    for (int t = 0; t < GL_TMAX; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (uint32_t kc = 0; kc < K; kc += GL_KC) {
        __syncthreads();  // the previous chunk's activations have been read
        // activations k = kc .. kc+4095 of rows m < M: 8 loads of 1 KB per row; k past the end
        // reads as zero, so the weight zeros beyond k never meet stale LDS data
        // every workgroup reads the same activations: start each at a different 1 KB piece so
        // that the requests of concurrent workgroups spread over the L2 channels
        const uint32_t pieces = M * 8, rot = (blockIdx.x * 13u) % pieces;
        for (uint32_t c = (uint32_t)wave; c < pieces; c += GL_WAVES) {
            const uint32_t i = c + rot < pieces ? c + rot : c + rot - pieces;
            const uint32_t m = i >> 3, j = i & 7;
            const uint32_t k = kc + j * 512 + lane * 8;
            const uint32_t off = k < K ? (m * ldx + k) * 2 : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(lds + m * GL_PITCH + j * 1024), 16, off, 0, 0, 0);
        }
        // the first tile's weights travel together with the activations
        const uint32_t kw = (uint32_t)wave * (GL_KC / GL_WAVES);  // this wave's k offset in the chunk
        GlW<BLOCK> buf[2];
        gl_load<BLOCK>(buf[0], a, blockIdx.x, kc + kw, lr, kq);
        __syncthreads();  // (waits for this wave's loads first) every wave's loads have landed
#pragma unroll
        for (int t = 0; t < GL_TMAX; ++t) {
            if ((uint32_t)t >= ntiles) continue;
            if ((uint32_t)t + 1 < ntiles) gl_load<BLOCK>(buf[(t + 1) & 1], a, blockIdx.x + (t + 1) * G, kc + kw, lr, kq);
            const GlW<BLOCK>& w = buf[t & 1];
#pragma unroll
            for (int kt = 0; kt < GL_KTW; ++kt) {
                uint32_t bw[16];
                dequant32<BLOCK, FMT>(w.cw[kt], gl_scale<BLOCK, FMT>(w, kt, kq, kc + kw + kt * TK + 32 * kq < K), bw);
                const uint8_t* xp = lds + xrow * GL_PITCH + (kw + kt * TK + 32 * kq) * 2;
                uint32_t xf[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(xp + 16 * q);
                    xf[4 * q] = v.x; xf[4 * q + 1] = v.y; xf[4 * q + 2] = v.z; xf[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[t] = mfma_bf16(&xf[4 * j], &bw[4 * j], acc[t]);
            }
        }
    }
    // the waves' partial sums meet in LDS ([wave][tile][lane]); wave w finishes tiles w, w+8, ...
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
    for (int t = 0; t < GL_TMAX; ++t)
        if ((uint32_t)t < ntiles) red[(wave * GL_TMAX + t) * 64 + lane] = acc[t];
    __syncthreads();
    for (uint32_t t = (uint32_t)wave; t < ntiles; t += GL_WAVES) {
        f32x4 v = red[t * 64 + lane];
#pragma unroll
        for (int w = 1; w < GL_WAVES; ++w) v += red[(w * GL_TMAX + t) * 64 + lane];
        const int64_t n = (int64_t)(blockIdx.x + t * G) * 16 + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = 4 * kq + i;
            if (m < a.m && n < a.n) store_y<OUT_BF16>(a.y, a.ldy, m, n, v[i] * a.g);
        }
    }
}

// ---------------------------------------------------------------------------------------
// W4A16 GEMV for m = 1 (the template takes up to 4 rows of X) on the vector ALUs.  A workgroup owns DOT_ROWS weight rows; its 4
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

// PRE: weight scales in the preshuffled layout (block 32): the scale bytes of the lane's block
// for all 8 rows of the workgroup are one 8-byte word, one load instead of eight.
template <int BLOCK, int FMT, int MM, bool OUT_BF16, bool PRE = false>
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
    const uint32_t pcb = (uint32_t)((K / 32 + 63) / 64);  // preshuffled: 2048-k chunks per row group
    const rsrc_t sr = PRE ? make_rsrc(a.ws + (n0 / 8) * pcb * 512, pcb * 512)
                          : make_rsrc(a.ws + n0 * (a.k / BLOCK), nrows * (K / BLOCK));
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
        uint64_t sb[PRE ? 1 : DOT_ROWS];
        // preshuffled: the 8 rows' scale bytes as two dwords, each row's byte taken where it
        // is used (64-bit per-row copies made the compiler serialize the chunk's loads)
        uint32_t sv_lo = 0, sv_hi = 0;
        if constexpr (PRE) {
            const uint64_t sv = bload64(sr, ok ? (uint32_t)c * 512 + 8 * lane : kOOB);
            sv_lo = (uint32_t)sv;
            sv_hi = (uint32_t)(sv >> 32);
        }
#pragma unroll
        for (int r = 0; r < DOT_ROWS; ++r) {
            cw[r] = bload128(wr, ok ? r * (K / 2) + kk / 2 : kOOB);
            if constexpr (!PRE) sb[r] = bload_lane_scales<BLOCK>(sr, ok ? r * (K / BLOCK) + kk / BLOCK : kOOB);
        }
        auto sbyte = [&](int r) -> uint32_t {
            if constexpr (PRE) return ((r < 4 ? sv_lo : sv_hi) >> (8 * (r & 3))) & 0xFFu;
            else return (uint32_t)sb[r] & 0xFFu;
        };
        uint32_t xf[MM][16];
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 v = bload128(xr, ok && m < a.m ? (uint32_t)(m * a.ldx * 2) + (kk + 8 * j) * 2 : kOOB);
                xf[m][4 * j] = v.x; xf[m][4 * j + 1] = v.y; xf[m][4 * j + 2] = v.z; xf[m][4 * j + 3] = v.w;
            }
        // all of the chunk's loads are issued before any of its arithmetic (otherwise the
        // scheduler may start on the first rows and issue the activation loads one at a time)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < DOT_ROWS; ++r) {
            uint32_t bw[16];
            if constexpr (BLOCK >= 32 && FMT != FMT_E8M0) {
                // one scale for the lane's 32 k: its mantissa multiplies their fp32 sum once
                const float mant = dequant32_pow2<FMT>(cw[r], sbyte(r), bw);
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    float t = 0.0f;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xf[m][i]),
                                                            __builtin_bit_cast(bf16x2, bw[i]), t, false);
                    acc[r][m] = __builtin_fmaf(t, mant, acc[r][m]);
                }
            } else {
                if constexpr (PRE) dequant32<BLOCK, FMT>(cw[r], (uint64_t)sbyte(r), bw);
                else dequant32<BLOCK, FMT>(cw[r], sb[r], bw);
#pragma unroll
                for (int m = 0; m < MM; ++m)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        acc[r][m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xf[m][i]),
                                                                    __builtin_bit_cast(bf16x2, bw[i]),
                                                                    acc[r][m], false);
            }
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
// W4A16 GEMV for m <= 2 on short streams (the decode shapes): the grid sweeps the code bytes
// in address order.  The codes form a sequence of 1 KB chunks (2048 k of one row, row-major);
// a unit is 8 consecutive chunks (8 KB).  Step i of the persistent grid of G workgroups covers
// units i G .. i G + G - 1, so at any time the whole GPU reads one contiguous slab, which on
// MI355X streams markedly better than many workgroups each reading its own rows (measured:
// n 14336, k 4096: 9.0 against 11.2 us per launch).  Wave w of a workgroup takes chunks 2w,
// 2w+1 of the unit; k / 2048 being 2, 4 or 8, they lie in one row and are the same two chunks
// of k, 2w mod (k / 2048) and the next, at every step, so the wave holds its X for them in
// registers, loaded once (through LDS, once per workgroup).  The next step's codes and scales
// are in flight while a step is computed.  Each wave's partial sums go to LDS; the rows of
// the workgroup's units are summed at the end in a fixed order.
// ---------------------------------------------------------------------------------------
constexpr uint32_t SW_GRID = 1024;
constexpr uint32_t SW_MAX_STEPS = 4;

// MM: rows of X (m == MM).  W8: FP8 (E4M3) codes, a byte per element: a chunk of 2048 k is
// then 2 KB, read as two 1 KB halves, and lane l holds k = 16 l .. 16 l + 15 of each half (two
// 32-blocks, so two scale bytes); with FP4 codes lane l holds k = 32 l .. 32 l + 31 of the chunk.
template <int FMT, bool OUT_BF16, bool PRE, int MM, bool W8>
__global__ __launch_bounds__(256) void gemv_sweep_kernel(const GemmArgs a, uint32_t units)
{
    constexpr int NH = W8 ? 2 : 1;  // code loads per chunk
    __shared__ float part[SW_MAX_STEPS][4][MM];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t K = (uint32_t)a.k, KC = K / 2048, G = gridDim.x;
    const uint32_t c0 = (2 * (uint32_t)wave) & (KC - 1);  // the wave's first chunk of k
    const uint32_t rowb = W8 ? K : K / 2;                   // code bytes per row

    const rsrc_t wr = make_rsrc(a.wc, (uint32_t)(a.n * rowb));
    const rsrc_t sr = PRE ? make_rsrc(a.ws, (uint32_t)(((a.n + 7) / 8) * KC * 512))
                          : make_rsrc(a.ws, (uint32_t)(a.n * (a.k / 32)));
    const uint32_t nsteps = (units - blockIdx.x + G - 1) / G;  // units blockIdx.x + i G < units

    auto load = [&](uint32_t i, u32x4 (&cw)[2][NH], uint32_t (&sb)[2]) {
        const uint32_t row = ((blockIdx.x + i * G) * 8 + 2 * wave) / KC;
        const bool ok = i < nsteps;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t c = c0 + h;
            if constexpr (W8) {
#pragma unroll
                for (int e = 0; e < 2; ++e) cw[h][e] = bload128(wr, ok ? row * rowb + c * 2048 + e * 1024 + lane * 16 : kOOB);
                const uint32_t so = row * (K / 32) + c * 64 + (lane >> 1);
                sb[h] = bload8(sr, ok ? so : kOOB) | (bload8(sr, ok ? so + 32 : kOOB) << 8);
            } else {
                cw[h][0] = bload128(wr, ok ? row * rowb + c * 1024 + lane * 16 : kOOB);
                const uint32_t so = PRE ? ((row >> 3) * KC + c) * 512 + lane * 8 + (row & 7)
                                        : row * (K / 32) + c * 64 + lane;
                sb[h] = bload8(sr, ok ? so : kOOB);
            }
        }
    };
    u32x4 cw[2][NH], cn[2][NH];
    uint32_t sb[2], sn[2];
    // X of the wave's chunk pair in the order of the lane's 32 k (piece j = 8 k).  The m rows
    // of X are staged once per workgroup through LDS (m k / 8 pieces of 16 bytes, m k 2 bytes
    // of dynamic LDS): each wave needs all of it when k / 2048 is 2, and fetching it once per
    // workgroup instead of once per wave cuts its L2 traffic fourfold (measured: n 4096, k 4096,
    // m 1: 5.4 -> 4.6 us).
    extern __shared__ u32x4 xs[];
    uint32_t xq[MM][2][16];
    {
        // X by LDS-DMA (lane i of a load writes 16 bytes at the wave's base + 16 i; the piece
        // count, m k / 8, is a multiple of 512), then step 0's codes and scales, so that the
        // weights' HBM latency overlaps the staging; wait for this wave's X loads only (the
        // NLOAD weight loads issued after them may stay in flight), then the barrier.
        typedef __attribute__((address_space(3))) void lds_void;
        const rsrc_t xr = make_rsrc(a.x, (uint32_t)(((int64_t)(MM - 1) * a.ldx + a.k) * 2));
        const uint32_t npieces = MM * (K / 8);
        for (uint32_t t0 = (uint32_t)wave * 64; t0 < npieces; t0 += 256) {
            const uint32_t t = t0 + lane, m = t / (K / 8), p = t - m * (K / 8);
            const uint32_t off = t < npieces ? (uint32_t)(m * a.ldx * 2) + p * 16 : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(xs + t0), 16, off, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        load(0, cw, sb);
        __builtin_amdgcn_sched_barrier(0);
        constexpr int NLOAD = 2 * (NH + (W8 ? 2 : 1));  // vector-memory instructions of load()
        __builtin_amdgcn_s_waitcnt((NLOAD & 0xF) | ((NLOAD >> 4) << 14) | (0x7 << 4) | (0xF << 8));
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t kx = W8 ? (c0 + h) * 2048 + (j >> 1) * 1024 + 16 * lane + 8 * (j & 1)
                                           : (c0 + h) * 2048 + 32 * lane + 8 * j;
                    const u32x4 v = xs[m * (K / 8) + kx / 8];
                    xq[m][h][4 * j] = v.x;
                    xq[m][h][4 * j + 1] = v.y;
                    xq[m][h][4 * j + 2] = v.z;
                    xq[m][h][4 * j + 3] = v.w;
                }
    }
    for (uint32_t i = 0; i < nsteps; ++i) {
        load(i + 1, cn, sn);
        float acc[MM];
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[m] = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t bw[16];
            if constexpr (W8 && FMT != FMT_E8M0) {
                // the lane's two 16-element pieces, each inside its own 32-element block (pairs
                // 0-7: first scale byte, 8-15: second): each pair as e * 2^p in bf16 (exact),
                // each piece's scale mantissa once on its fp32 sum
                const uint32_t c8[8] = {cw[h][0].x, cw[h][0].y, cw[h][0].z, cw[h][0].w,
                                        cw[h][1].x, cw[h][1].y, cw[h][1].z, cw[h][1].w};
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const DecG1 p = dec_params_g1<FMT>((sb[h] >> (8 * q)) & 0xFFu);
#pragma unroll
                    for (int hh = 0; hh < 8; ++hh) {
                        const int pr = 8 * q + hh;
                        const bf16x2 v = (pr & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8[pr >> 1], p.pow2, true)
                                                  : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8[pr >> 1], p.pow2, false);
                        bw[pr] = __builtin_bit_cast(uint32_t, v);
                    }
#pragma unroll
                    for (int m = 0; m < MM; ++m) {
                        float u = 0.0f;
#pragma unroll
                        for (int hh = 0; hh < 8; ++hh)
                            u = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xq[m][h][8 * q + hh]),
                                                                __builtin_bit_cast(bf16x2, bw[8 * q + hh]), u, false);
                        acc[m] = __builtin_fmaf(u, p.mant, acc[m]);
                    }
                }
                continue;
            } else if constexpr (W8) {
                const uint32_t c8[8] = {cw[h][0].x, cw[h][0].y, cw[h][0].z, cw[h][0].w,
                                        cw[h][1].x, cw[h][1].y, cw[h][1].z, cw[h][1].w};
                dequant_w8<16, FMT>(c8, sb[h], bw);  // elements 0..15: first byte, 16..31: second
            } else if constexpr (FMT != FMT_E8M0) {
                // one scale for the lane's 32 k: its mantissa multiplies their fp32 sum once
                const float mant = dequant32_pow2<FMT>(cw[h][0], sb[h] & 0xFFu, bw);
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    float u = 0.0f;
#pragma unroll
                    for (int t = 0; t < 16; ++t)
                        u = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xq[m][h][t]),
                                                            __builtin_bit_cast(bf16x2, bw[t]), u, false);
                    acc[m] = __builtin_fmaf(u, mant, acc[m]);
                }
                continue;
            } else {
                dequant32<32, FMT>(cw[h][0], sb[h], bw);
            }
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    acc[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xq[m][h][t]),
                                                             __builtin_bit_cast(bf16x2, bw[t]), acc[m], false);
        }
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            float v = acc[m];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            if (lane == 0) part[i][wave][m] = v;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int e = 0; e < NH; ++e) cw[h][e] = cn[h][e];
            sb[h] = sn[h];
        }
    }
    __syncthreads();
    // a unit holds 8 / KC rows; row rr of it sums the partials of waves rr KC/2 .. +KC/2-1
    const uint32_t rpu = 8 / KC;
    if (threadIdx.x < nsteps * rpu * MM) {
        const uint32_t m = threadIdx.x % MM, ir = threadIdx.x / MM, i = ir / rpu, rr = ir - i * rpu;
        float v = 0.0f;
        for (uint32_t w = rr * (KC / 2); w < (rr + 1) * (KC / 2); ++w) v += part[i][w][m];
        store_y<OUT_BF16>(a.y, a.ldy, m, (int64_t)(blockIdx.x + i * G) * rpu + rr, v * a.g);
    }
}

// the sweep's shape conditions; returns the unit count (0: not applicable)
static uint32_t sweep_units(const GemmArgs& a)
{
    if (a.m < 1 || a.m > 2 || a.block != 32) return 0;
    if (a.k != 4096 && a.k != 8192 && a.k != 16384) return 0;  // 2, 4 or 8 chunks per row
    if (((a.m - 1) * a.ldx + a.k) * 2 >= (int64_t(1) << 31)) return 0;
    const int64_t chunks = a.n * (a.k / 2048);
    if (chunks % 8 != 0) return 0;
    const int64_t units = chunks / 8;
    const int64_t g = units < SW_GRID ? units : SW_GRID;
    if (units == 0 || (units + g - 1) / g > SW_MAX_STEPS) return 0;
    return (uint32_t)units;
}

template <int FMT, bool OUT_BF16, int MM, bool W8>
static hipError_t launch_sweep(const GemmArgs& a, uint32_t units, hipStream_t st)
{
    const dim3 grid(units < SW_GRID ? units : SW_GRID);
    const size_t lds = (size_t)MM * a.k * 2;  // X; at most 64 KB (m <= 2, k <= 16384)
    // allow the full 64 KB of dynamic LDS next to the static partial sums
    static LdsLimit lim_pre, lim;
    if (const hipError_t e = lim_pre.ensure((const void*)gemv_sweep_kernel<FMT, OUT_BF16, true, MM, false>, 65536, st);
        e != hipSuccess)
        return e;
    if (const hipError_t e = lim.ensure((const void*)gemv_sweep_kernel<FMT, OUT_BF16, false, MM, W8>, 65536, st);
        e != hipSuccess)
        return e;
    if (!W8 && a.ws_pre) hipLaunchKernelGGL((gemv_sweep_kernel<FMT, OUT_BF16, true, MM, false>), grid, dim3(256), lds, st, a, units);
    else hipLaunchKernelGGL((gemv_sweep_kernel<FMT, OUT_BF16, false, MM, W8>), grid, dim3(256), lds, st, a, units);
    return hipGetLastError();
}

bool w8_uses_sweep(const GemmArgs& a) { return !a.ws_pre && sweep_units(a) != 0; }

hipError_t launch_gemv_sweep_w8(const GemmArgs& a, hipStream_t st)
{
    const uint32_t units = sweep_units(a);
    if (units == 0 || a.ws_pre) return hipErrorInvalidValue;
#define MXF(F)                                                                                             \
    if (a.fmt == F) {                                                                                      \
        if (a.m == 1) return a.y_bf16 ? launch_sweep<F, true, 1, true>(a, units, st) : launch_sweep<F, false, 1, true>(a, units, st); \
        return a.y_bf16 ? launch_sweep<F, true, 2, true>(a, units, st) : launch_sweep<F, false, 2, true>(a, units, st);              \
    }
    MXF(FMT_E4M3) MXF(FMT_UE5M3) MXF(FMT_E8M0)
#undef MXF
    return hipErrorInvalidValue;
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
    // the GEMV kernels address X through one buffer resource with 32-bit byte offsets
    const bool x_span_ok = ((a.m - 1) * a.ldx + a.k) * 2 < (int64_t(1) << 31);
    const bool fast = (a.k % 32 == 0) && ((a.ldx * 2) % 16 == 0) && ((uintptr_t)a.x % 16 == 0);
    if (!fast || (a.m <= 16 && !x_span_ok)) {
        const int64_t total = a.m * a.n;
        hipLaunchKernelGGL((gemm_generic_kernel<FMT, false, OUT_BF16>), dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, st, a);
        return hipGetLastError();
    }
    // m = 2 takes the 16-row-unit kernel where it applies (k 4096; 5.5 against 6.4 us at n
    // 4096, even at n 14336), the sweeping kernel otherwise (k 8192 / 16384)
    if (a.m >= 2 && gemv16_applies(a)) return launch_gemv16(a, st);
    if (const uint32_t units = sweep_units(a)) {
        if (a.m == 1) return launch_sweep<FMT, OUT_BF16, 1, false>(a, units, st);
        return launch_sweep<FMT, OUT_BF16, 2, false>(a, units, st);
    }
    if (a.m >= 2 && a.m <= 16) {
        const unsigned tiles = (unsigned)((a.n + 15) / 16);
        unsigned g = tiles < 256 ? tiles : 256;                       // one workgroup per CU
        if (g * GL_TMAX < tiles) g = (tiles + GL_TMAX - 1) / GL_TMAX;  // at most 16 tiles each
        const int need = (int)a.m * GL_PITCH;
        const int lds_bytes = need > GL_RED ? need : GL_RED;
        switch (a.block) {
#define MXL(B) case B: { \
    static LdsLimit lim; \
    if (const hipError_t e = lim.ensure((const void*)gemv_lds_kernel<B, FMT, OUT_BF16>, \
                                        16 * GL_PITCH > GL_RED ? 16 * GL_PITCH : GL_RED, st); e != hipSuccess) \
        return e; \
    hipLaunchKernelGGL((gemv_lds_kernel<B, FMT, OUT_BF16>), dim3(g), dim3(64 * GL_WAVES), lds_bytes, st, a); \
    break; }
            MXL(4) MXL(8) MXL(16) MXL(32) MXL(64) MXL(128) MXL(256)
#undef MXL
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (a.m == 1) {
        const dim3 grid((unsigned)((a.n + DOT_ROWS - 1) / DOT_ROWS));
        switch (a.block) {
#define MXD1(B) case B: \
    if (B == 32 && a.ws_pre) \
        hipLaunchKernelGGL((gemv_dot_kernel<B, FMT, 1, OUT_BF16, true>), grid, dim3(64 * DOT_WAVES), 0, st, a); \
    else \
        hipLaunchKernelGGL((gemv_dot_kernel<B, FMT, 1, OUT_BF16>), grid, dim3(64 * DOT_WAVES), 0, st, a); \
    break;
            MXD1(4) MXD1(8) MXD1(16) MXD1(32) MXD1(64) MXD1(128) MXD1(256)
#undef MXD1
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (a16_uses_tiled(a)) return launch_gemm_a16_tiled(a, st);
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
