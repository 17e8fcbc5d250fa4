// mx_gemm_a16.hip -- W4A16 GEMM for large m on gfx950: Y = X . dequant(Wq)^T with bf16
// activations, fp32 accumulation (gtnt.cn/news/16247 "为什么我们需要4-bit浮点量化", section
// 3.1: dequantize, then matmul; section 4.3: large batches dequantize on the fly;
// hotelren.com/news/2192771, article "量化技术演进与微缩量化原理", section 3.2 item 3: load the
// FP4 block, unpack, apply its scale, multiply, accumulate).  The dequantized weights exist
// only in registers, as the bf16 operands of v_mfma_f32_32x32x16_bf16.
//
// Tiling: a workgroup of 8 waves (two per SIMD) computes a 128 (m) x 256 (n) output tile;
// each wave a 64 x 64 sub-tile of 2 x 2 MFMA results.  The k loop advances 128 elements per
// stage through a 3-deep LDS ring filled by buffer_load ... lds (no register round trip;
// rows and k beyond the tensors read as zero): per stage the activation tile (128 rows x 256
// bytes) and the weight codes (256 rows x 64 bytes); the weight scales arrive per 512 k
// (256 rows x 16 bytes) in a double buffer of their own.  With three stage buffers the loads
// of a stage are issued two stages before it is read.  Within a 64-k window a lane holds 32
// consecutive k of its row for both operands (activations read from LDS, weights dequantized
// from 16 code bytes), and the four MFMA k-steps take them in the same permuted order, which
// leaves every dot product intact.  The MFMA's A operand is the weight fragment, so each
// result tile is transposed (rows n, columns m); the epilogue stages it through LDS and
// writes whole 16-byte chunks.  Workgroups are mapped so that the tiles resident on one XCD
// share a few activation and weight tiles through its L2.
//
// The same kernel serves FP8 (E4M3) weights in the same block structure (the W8A16 product
// of the FP8 fallback): a weight row then brings 128 code bytes per stage, a stage is 64 KB
// and the ring two stages deep (three would not fit in LDS), so the loads of a stage are
// issued one stage before it is read.
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_wdeq.h"

namespace mxk {

namespace a16 {

constexpr int BM = 128, BN = 256, BK = 128;
constexpr int WAVES = 8, THREADS = 64 * WAVES;
constexpr int MI = 2, NJ = 2;                    // per wave: 2 (m) x 2 (n) tiles of 32 x 32
constexpr int XROWB = BK * 2;                    // activation bytes per row per stage (256)
constexpr int X_BYTES = BM * XROWB;              // 32 KB
constexpr int SWIN_K = 512;                      // k per scale window
constexpr int SWIN_BYTES = BN * (SWIN_K / 32);   // 4 KB
constexpr int LOADS_PER_WINDOW = 2;              // per wave

// Stage geometry by weight width: FP4 (W8 false) or FP8 codes.
template <bool W8>
struct Geo {
    static constexpr int WROWB = W8 ? BK : BK / 2;             // code bytes per weight row per stage
    static constexpr int W_BYTES = BN * WROWB;                 // 16 or 32 KB
    static constexpr int STAGE_BYTES = X_BYTES + W_BYTES;      // 48 or 64 KB
    static constexpr int STAGES = W8 ? 2 : 3;
    static constexpr int SWIN_OFF = STAGES * STAGE_BYTES;
    static constexpr int LDS_BYTES = SWIN_OFF + 2 * SWIN_BYTES;  // 155648 or 139264 (of 160 KB)
    static constexpr int WCH = WROWB / 16;                     // 16-byte chunks per weight row
    static constexpr int WRPL = 64 / WCH;                      // weight rows per 1 KB load
    static constexpr int WLOADS = BN / WRPL / WAVES;           // code loads per wave (2 or 4)
    static constexpr int LOADS_PER_STAGE = 4 + WLOADS;         // per wave, with 4 activation loads
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS chunk permutations against bank conflicts: activation rows have 16 chunks of 16 bytes
// (XOR with row % 16); weight rows 4 (FP4: XOR with (row / 4) % 4) or 8 (FP8: XOR with
// (row / 2) % 8), so that the rows sharing a 256-byte line permute their chunks differently.
__device__ __forceinline__ uint32_t xswz(uint32_t row, uint32_t c) { return c ^ (row & 15u); }
template <bool W8>
__device__ __forceinline__ uint32_t wswz(uint32_t row, uint32_t c)
{
    if constexpr (W8) return c ^ ((row >> 1) & 7u);
    else return c ^ ((row >> 2) & 3u);
}

// This wave's share of stage s's loads into the stage buffer at `st`.
// Activations: 32 loads of 4 rows x 256 bytes (lane: row lane/16, LDS chunk lane%16).
// Codes: 16 loads of 16 rows x 64 bytes (FP4; lane: row lane/4, LDS chunk lane%4) or 32 loads
// of 8 rows x 128 bytes (FP8; lane: row lane/8, LDS chunk lane%8).
template <bool W8>
__device__ __forceinline__ void issue_stage(uint8_t* st, int wave, int lane, uint32_t s, rsrc_t xr, rsrc_t wr,
                                            uint32_t ldx, uint32_t K)
{
    using G = Geo<W8>;
    const uint32_t k0 = s * BK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t grp = (uint32_t)(wave * 4 + q);          // 4-row group, 0..31
        const uint32_t row = grp * 4 + (lane >> 4);
        const uint32_t c = xswz(row, lane & 15);
        const uint32_t kk = k0 + 8 * c;
        const uint32_t off = kk < K ? (row * ldx + kk) * 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(st + grp * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < G::WLOADS; ++q) {
        const uint32_t grp = (uint32_t)(wave * G::WLOADS + q);  // group of WRPL rows
        const uint32_t row = grp * G::WRPL + lane / G::WCH;
        const uint32_t c = wswz<W8>(row, lane % G::WCH);
        const uint32_t kk = k0 + (W8 ? 16 : 32) * c;            // first k of chunk c
        const uint32_t off = kk < K ? (W8 ? row * K + kk : row * (K / 2) + kk / 2) : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)(st + X_BYTES + grp * 1024), 16, off, 0, 0, 0);
    }
}

// This wave's share of scale window j (k = 512 j .. +511: 16 bytes per weight row) into the
// window buffer at `sw`: 16 loads of 16 rows x 16 bytes (lane: row lane/4, dword lane%4).
// Requires (k / 32) % 4 == 0 so that every row's window starts on a dword.
__device__ __forceinline__ void issue_window(uint8_t* sw, int wave, int lane, uint32_t j, rsrc_t sr, uint32_t K)
{
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const uint32_t grp = (uint32_t)(wave * 2 + q);          // 16-row group, 0..15
        const uint32_t row = grp * 16 + (lane >> 2);
        const uint32_t off = j * SWIN_K < K ? row * (K / 32) + j * 16 + 4 * (lane & 3) : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void*)(sw + grp * 256), 4, off, 0, 0, 0);
    }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Fragments of one 64-k window w of a stage: per m-block i, 64 activation bytes (k = 64w + 32h
// .. +31 of row m); per n-block jn, 16 (FP4) or 32 (FP8) code bytes (same k of weight row n)
// and the scale byte.
template <bool W8>
struct Frags {
    u32x4 x[MI][4];
    u32x4 w[NJ][W8 ? 2 : 1];
    uint32_t s[NJ];
};

template <bool W8>
__device__ __forceinline__ void read_frags(const uint8_t* st, const uint8_t* swin, uint32_t sbyte, int w,
                                           uint32_t xrow0, uint32_t wrow0, uint32_t h, Frags<W8>& f)
{
    using G = Geo<W8>;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const uint32_t row = xrow0 + 32 * i;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            f.x[i][q] = *reinterpret_cast<const u32x4*>(st + row * XROWB + 16 * xswz(row, 8 * w + 4 * h + q));
    }
#pragma unroll
    for (int jn = 0; jn < NJ; ++jn) {
        const uint32_t row = wrow0 + 32 * jn;
        if constexpr (W8) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
                f.w[jn][c] = *reinterpret_cast<const u32x4*>(st + X_BYTES + row * G::WROWB +
                                                            16 * wswz<W8>(row, 4 * w + 2 * h + c));
        } else {
            f.w[jn][0] = *reinterpret_cast<const u32x4*>(st + X_BYTES + row * G::WROWB + 16 * wswz<W8>(row, 2 * w + h));
        }
        f.s[jn] = swin[row * 16 + sbyte + 2 * w];
    }
}

template <int FMT, bool W8>
__device__ __forceinline__ void mfma_window(f32x16 (&acc)[MI][NJ], const Frags<W8>& f)
{
    uint32_t bw[NJ][16];
#pragma unroll
    for (int jn = 0; jn < NJ; ++jn) {
        if constexpr (W8) {
            const uint32_t cw[8] = {f.w[jn][0].x, f.w[jn][0].y, f.w[jn][0].z, f.w[jn][0].w,
                                    f.w[jn][1].x, f.w[jn][1].y, f.w[jn][1].z, f.w[jn][1].w};
            dequant_w8<32, FMT>(cw, f.s[jn], bw[jn]);
        } else {
            dequant32<32, FMT>(f.w[jn][0], f.s[jn], bw[jn]);
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)          // k-step t takes k 32h + 8t .. +7 of the window
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const u32x4 xv = f.x[i][t];
#pragma unroll
            for (int jn = 0; jn < NJ; ++jn) {
                const u32x4 wv = {bw[jn][4 * t], bw[jn][4 * t + 1], bw[jn][4 * t + 2], bw[jn][4 * t + 3]};
                acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv),
                                                                     __builtin_bit_cast(bf16x8, xv), acc[i][jn], 0, 0, 0);
            }
        }
}

template <int FMT, bool OUT_BF16, bool W8>
__global__ __launch_bounds__(THREADS) void gemm_a16_kernel(const GemmArgs a)
{
    using G = Geo<W8>;
    constexpr int STAGES = G::STAGES, STAGE_BYTES = G::STAGE_BYTES, SWIN_OFF = G::SWIN_OFF;
    constexpr int LOADS_PER_STAGE = G::LOADS_PER_STAGE;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const uint32_t K = (uint32_t)a.k, ldx = (uint32_t)a.ldx;

    // tile mapping: with the n-tile count a multiple of 8, XCD x (= block % 8) takes n-tiles
    // x, x+8, ...; with the m-tile count a multiple of 4 it runs them in groups of 4 m-tiles
    // (all its n-tiles for m-tiles 0-3, then 4-7, ...), so that the ~32 workgroups resident on
    // an XCD share 4 activation tiles (2 MB each at k 8192) and ~8 weight tiles through its L2
    // (fetched from the fabric per 70B-FFN launch: 2.0 GB when each XCD ran all 16 m-tiles of
    // two n-tiles at a time); else, for each n-tile, every m-tile in turn
    const uint32_t MT = (uint32_t)((a.m + BM - 1) / BM), NT = (uint32_t)((a.n + BN - 1) / BN);
    uint32_t mt, nt;
    if ((NT & 7) == 0 && (MT & 3) == 0) {
        const uint32_t x = blockIdx.x & 7, local = blockIdx.x >> 3, NT8 = NT >> 3;
        const uint32_t grp = local / (4 * NT8), r = local - grp * (4 * NT8);
        mt = grp * 4 + (r & 3);
        nt = (r >> 2) * 8 + x;
    } else if ((NT & 7) == 0) {
        const uint32_t x = blockIdx.x & 7, local = blockIdx.x >> 3;
        mt = local % MT;
        nt = (local / MT) * 8 + x;
    } else {
        mt = blockIdx.x % MT;
        nt = blockIdx.x / MT;
    }
    const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN;
    const uint32_t mrows = (uint32_t)(a.m - m0 < BM ? a.m - m0 : BM);
    const uint32_t nrows = (uint32_t)(a.n - n0 < BN ? a.n - n0 : BN);
    const rsrc_t xr = make_rsrc(a.x + m0 * a.ldx, ((mrows - 1) * ldx + K) * 2);
    const uint32_t wrowb = W8 ? K : K / 2;                   // code bytes per weight row
    const rsrc_t wr = make_rsrc(a.wc + n0 * (int64_t)wrowb, nrows * wrowb);
    const rsrc_t sr = make_rsrc(a.ws + n0 * (a.k / 32), nrows * (K / 32));

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Pipeline: one stage (two 64-k windows) per iteration.  The fragments of window 1 are
    // read while window 0's MFMAs run; then, once this stage's reads have completed and the
    // next stage has landed, one barrier publishes it and frees this stage's buffer, which
    // receives the stage three ahead; window 0 of the next stage is read while window 1's MFMAs
    // run.  Scale window j + 1 is requested at stage 4j.  Stages past the end of k load as
    // zeros (out-of-range offsets), so every iteration has the same shape.  With the two-deep
    // FP8 ring the stage awaited at the barrier is the last one issued: every load has to land.
    const int S = (int)((K + BK - 1) / BK);
    issue_window(lds + SWIN_OFF, wave, lane, 0, sr, K);
#pragma unroll
    for (int p = 0; p < STAGES; ++p) issue_stage<W8>(lds + p * STAGE_BYTES, wave, lane, (uint32_t)p, xr, wr, ldx, K);

    const uint32_t r32 = lane & 31, h = lane >> 5;
    const uint32_t xrow0 = wm * 64 + r32, wrow0 = wn * 64 + r32;

    Frags<W8> f0, f1;
    wait_vmcnt<(STAGES - 1) * LOADS_PER_STAGE>();
    barrier_only();
    read_frags(lds, lds + SWIN_OFF, h, 0, xrow0, wrow0, h, f0);

    uint32_t cur = 0;  // byte offset of stage s's buffer
    for (int s = 0; s < S; ++s) {
        const uint32_t nxt = cur + STAGE_BYTES == (uint32_t)(STAGES * STAGE_BYTES) ? 0u : cur + STAGE_BYTES;
        const uint8_t* swin = lds + SWIN_OFF + ((s >> 2) & 1) * SWIN_BYTES;
        const uint32_t sb = 4 * (uint32_t)(s & 3) + h;       // the lane's scale byte in the window row
        read_frags(lds + cur, swin, sb, 1, xrow0, wrow0, h, f1);
        mfma_window<FMT>(acc, f0);
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkm0();
        if constexpr (STAGES == 2) wait_vmcnt<0>();
        else if ((s & 3) == 1) wait_vmcnt<LOADS_PER_STAGE + LOADS_PER_WINDOW>();
        else wait_vmcnt<LOADS_PER_STAGE>();
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
        if ((s & 3) == 0) issue_window(lds + SWIN_OFF + (((s >> 2) + 1) & 1) * SWIN_BYTES, wave, lane, (uint32_t)(s >> 2) + 1, sr, K);
        issue_stage<W8>(lds + cur, wave, lane, (uint32_t)(s + STAGES), xr, wr, ldx, K);
        const int s1 = s + 1;
        const uint8_t* swin1 = lds + SWIN_OFF + ((s1 >> 2) & 1) * SWIN_BYTES;
        read_frags(lds + nxt, swin1, 4 * (uint32_t)(s1 & 3) + h, 0, xrow0, wrow0, h, f0);
        mfma_window<FMT>(acc, f1);
        asm volatile("" ::: "memory");
        cur = nxt;
    }
    wait_vmcnt<0>();

    // Epilogue.  Transposed 32x32 result layout: for tile (i, jn) a lane holds output row
    // m = i*32 + lane%32 and, for group q = e/4, columns n = jn*32 + 8q + 4*(lane/32) + e%4.
    // A wave's 64 x 64 block is staged through LDS (a region per wave, rows padded against
    // bank conflicts) and written back as whole 16-byte chunks.  Out-of-range chunks get an
    // out-of-range offset and are dropped.
    constexpr uint32_t ESZ = OUT_BF16 ? 2 : 4;
    const rsrc_t yr = make_rsrc(static_cast<uint8_t*>(a.y) + (m0 * a.ldy + n0) * ESZ, 0x7FFFFFFFu);
    const uint32_t ldy = (uint32_t)a.ldy;
    constexpr uint32_t CE = 16 / ESZ;
    const bool vec = (ldy % CE) == 0 && (nrows % CE) == 0;
    if (vec) {
        constexpr uint32_t RB = 64 * ESZ;                    // bytes of a wave row (64 columns)
        constexpr uint32_t PITCH = RB + 16;
        constexpr uint32_t CPR = RB / 16;                    // chunks per row (8 or 16)
        constexpr uint32_t RPI = 64 / CPR;                   // rows per store instruction
        static_assert(WAVES * 64 * PITCH <= (uint32_t)G::LDS_BYTES, "epilogue staging exceeds LDS");
        uint8_t* stg = lds + wave * 64 * PITCH;
        barrier_only();  // every wave is done reading the stage buffers
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jn = 0; jn < NJ; ++jn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16& c = acc[i][jn];
                    const float v0 = c[4 * q] * a.g, v1 = c[4 * q + 1] * a.g, v2 = c[4 * q + 2] * a.g, v3 = c[4 * q + 3] * a.g;
                    uint8_t* dst = stg + (i * 32 + r32) * PITCH + (jn * 32 + 8 * q + 4 * h) * ESZ;
                    if constexpr (OUT_BF16) {
                        const u32x2 w = {__builtin_bit_cast(uint32_t, bf16x2{(__bf16)v0, (__bf16)v1}),
                                         __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v2, (__bf16)v3})};
                        *reinterpret_cast<u32x2*>(dst) = w;
                    } else {
                        *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
                    }
                }
#pragma unroll
        for (uint32_t t = 0; t < 64 / RPI; ++t) {
            const uint32_t row = t * RPI + lane / CPR, chunk = lane % CPR;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * PITCH + chunk * 16);
            const uint32_t mm = wm * 64 + row, nn = wn * 64 + chunk * CE;
            const uint32_t off = (mm < mrows && nn < nrows) ? (mm * ldy + nn) * ESZ : kOOB;
            bstore128_nt(yr, off, v);
        }
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const uint32_t mm = wm * 64 + i * 32 + r32;
#pragma unroll
            for (int jn = 0; jn < NJ; ++jn)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t nn = wn * 64 + jn * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                    const uint32_t off = (mm < mrows && nn < nrows) ? (mm * ldy + nn) * ESZ : kOOB;
                    const float v = acc[i][jn][e] * a.g;
                    if constexpr (OUT_BF16) bstore16(yr, off, __builtin_bit_cast(uint16_t, (__bf16)v));
                    else bstore32(yr, off, __builtin_bit_cast(uint32_t, v));
                }
        }
    }
}

template <int FMT, bool OUT_BF16, bool W8>
static hipError_t launch_tiled(const GemmArgs& a, hipStream_t st)
{
    constexpr int LDS = Geo<W8>::LDS_BYTES;
    static LdsLimit lim;
    if (const hipError_t e = lim.ensure((const void*)gemm_a16_kernel<FMT, OUT_BF16, W8>, LDS, st); e != hipSuccess)
        return e;
    const unsigned tiles = (unsigned)(((a.m + BM - 1) / BM) * ((a.n + BN - 1) / BN));
    hipLaunchKernelGGL((gemm_a16_kernel<FMT, OUT_BF16, W8>), dim3(tiles), dim3(THREADS), LDS, st, a);
    return hipGetLastError();
}

}  // namespace a16

bool a16_uses_tiled(const GemmArgs& a)
{
    // block 32 with whole 512-k scale windows (each row's window starts on a dword), 16-byte
    // aligned activation rows, 32-bit offsets within the activation and output tiles
    const int64_t xspan = ((int64_t)(a16::BM - 1) * a.ldx + a.k) * 2;
    const int64_t yspan = ((int64_t)(a16::BM - 1) * a.ldy + a16::BN) * (a.y_bf16 ? 2 : 4);
    return a.block == 32 && a.k % a16::SWIN_K == 0 && (a.ldx * 2) % 16 == 0 &&
           ((uintptr_t)a.x % 16) == 0 && xspan < 0x7FFFFFFF && yspan < 0x7FFFFFFF;
}

hipError_t launch_gemm_a16_tiled(const GemmArgs& a, hipStream_t st)
{
    if (!a16_uses_tiled(a)) return hipErrorInvalidValue;
    if (a16w_uses(a, false)) return launch_gemm_a16w(a, false, st);  // wider wave tiles
    if (a16p_uses(a)) return launch_gemm_a16p(a, st);                 // two workgroups per CU
#define MXF(F) if (a.fmt == F) return a.y_bf16 ? a16::launch_tiled<F, true, false>(a, st) : a16::launch_tiled<F, false, false>(a, st);
    MXF(FMT_E4M3) MXF(FMT_UE5M3) MXF(FMT_E8M0)
#undef MXF
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_w8_tiled(const GemmArgs& a, hipStream_t st)
{
    if (!a16_uses_tiled(a)) return hipErrorInvalidValue;
    if (a16w_uses(a, true)) return launch_gemm_a16w(a, true, st);
#define MXF(F) if (a.fmt == F) return a.y_bf16 ? a16::launch_tiled<F, true, true>(a, st) : a16::launch_tiled<F, false, true>(a, st);
    MXF(FMT_E4M3) MXF(FMT_UE5M3) MXF(FMT_E8M0)
#undef MXF
    return hipErrorInvalidValue;
}
}  // namespace mxk
