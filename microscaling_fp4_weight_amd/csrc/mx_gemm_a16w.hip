// mx_gemm_a16w.hip -- the large-m W4A16 / W8A16 GEMM with wide wave tiles (all E4M3 and UE5M3
// weight scales, and FP8 weights): the
// same product as mx_gemm_a16.hip, Y = X . dequant(Wq)^T with bf16 activations and fp32
// accumulation (gtnt.cn/news/16247 "为什么我们需要4-bit浮点量化", section 3.1: dequantize, then
// matmul; hotelren.com/news/2192771, article "量化技术演进与微缩量化原理", section 3.2 item 3:
// load the FP4 block, unpack, apply its scale, multiply, accumulate).
//
// A scale that is not a power of two costs four vector instructions per dequantized bf16
// pair (fp4 -> fp32 with the scale's power of two, two multiplies by its mantissa, a pack)
// against one for an E8M0 scale.  With 64 x 64 wave tiles every dequantized weight fragment
// feeds two MFMAs and the vector unit, not the matrix core, sets the pace (about 1.4 vector
// cycles per matrix cycle).  Here a wave computes a 128 (m) x 64 (n) tile, so a fragment
// feeds four MFMAs: 8 waves (2 x 4, two per SIMD) compute a 256 x 256 output tile.  k
// advances 64 elements per stage through a 3-deep LDS ring filled by buffer_load ... lds
// (activations 256 rows x 128 bytes, codes 256 rows x 32 (FP4) or 64 (FP8) bytes; rows and k
// beyond the tensors read as zero), and the weight scales arrive per 512 k in a double buffer
// of their own.  Per stage a lane holds 32 consecutive k of its weight row (one 16-byte code
// load, FP8 two), dequantized once into 16 bf16 pairs, and reads its activations per 16-k
// MFMA step, one step ahead of the MFMAs, in the same permuted k order (every dot product is
// unchanged).  The MFMA's A operand is the weight fragment, so each result tile is
// transposed; the epilogue stages it through LDS and writes whole 16-byte chunks.
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_wdeq.h"

namespace mxk {

namespace a16w {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WAVES = 8, THREADS = 64 * WAVES;
constexpr int MI = 4, NJ = 2;                    // per wave: 4 (m) x 2 (n) tiles of 32 x 32
constexpr int XROWB = BK * 2;                    // activation bytes per row per stage (128)
constexpr int X_BYTES = BM * XROWB;              // 32 KB
constexpr int STAGES = 3;
constexpr int SWIN_K = 512;                      // k per scale window
constexpr int SPW = SWIN_K / BK;                 // stages per scale window (8)
constexpr int SWIN_BYTES = BN * (SWIN_K / 32);   // 4 KB
constexpr int LOADS_PER_WINDOW = 2;              // per wave

template <bool W8>
struct Geo {
    static constexpr int WROWB = W8 ? BK : BK / 2;               // code bytes per weight row per stage
    static constexpr int W_BYTES = BN * WROWB;                   // 16 or 8 KB
    static constexpr int STAGE_BYTES = X_BYTES + W_BYTES;        // 48 or 40 KB
    static constexpr int SWIN_OFF = STAGES * STAGE_BYTES;
    static constexpr int LDS_BYTES = SWIN_OFF + 2 * SWIN_BYTES;  // 155648 or 131072 (of 160 KB)
    static constexpr int WCH = WROWB / 16;                       // 16-byte chunks per weight row
    static constexpr int WRPL = 64 / WCH;                        // weight rows per 1 KB load
    static constexpr int WLOADS = BN / WRPL / WAVES;             // code loads per wave (2 or 1)
    static constexpr int LOADS_PER_STAGE = 4 + WLOADS;           // with 4 activation loads
};
static_assert(Geo<true>::LDS_BYTES <= 160 * 1024 && Geo<false>::LDS_BYTES <= 160 * 1024, "LDS ring");

typedef __attribute__((address_space(3))) void lds_void;

// LDS chunk permutations.  A 16-byte LDS read serves 16 lanes at a time, here 16 consecutive
// rows of one chunk column; the XORs give those 16 rows 16 different 16-byte bank groups:
// activation rows are 128 bytes (8 chunks), weight rows 32 (FP4, 2 chunks) or 64 (FP8, 4).
__device__ __forceinline__ uint32_t xswz(uint32_t row, uint32_t c) { return c ^ ((row >> 1) & 7u); }
template <bool W8>
__device__ __forceinline__ uint32_t wswz(uint32_t row, uint32_t c)
{
    if constexpr (W8) return c ^ ((row >> 2) & 3u);
    else return c ^ ((row >> 3) & 1u);
}

// This wave's share of stage s's loads into the stage buffer at `st`.  LDS-DMA writes lane i's
// 16 bytes at 16 i, so LDS slot l % 8 (activations) / l % WCH (codes) of a row receives the
// global chunk the permutation assigns to it.  Activations: 4 loads of 8 rows x 128 bytes.
// Codes: 1 load of 32 rows x 32 bytes (FP4) or 2 loads of 16 rows x 64 bytes (FP8).
template <bool W8>
__device__ __forceinline__ void issue_stage(uint8_t* st, int wave, int lane, uint32_t s, rsrc_t xr, rsrc_t wr,
                                            uint32_t ldx, uint32_t K)
{
    using G = Geo<W8>;
    const uint32_t k0 = s * BK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t grp = (uint32_t)(wave * 4 + q);          // 8-row group, 0..31
        const uint32_t row = grp * 8 + (lane >> 3);
        const uint32_t c = xswz(row, lane & 7);
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

// This wave's share of scale window j (k = 512 j .. +511: 16 bytes per weight row): 2 loads of
// 16 rows x 16 bytes (lane: row lane/4, dword lane%4).  Requires k % 512 == 0.
__device__ __forceinline__ void issue_window(uint8_t* sw, int wave, int lane, uint32_t j, rsrc_t sr, uint32_t K)
{
#pragma unroll
    for (int q = 0; q < LOADS_PER_WINDOW; ++q) {
        const uint32_t grp = (uint32_t)(wave * LOADS_PER_WINDOW + q);  // 16-row group, 0..15
        const uint32_t row = grp * 16 + (lane >> 2);
        const uint32_t off = j * SWIN_K < K ? row * (K / 32) + j * 16 + 4 * (lane & 3) : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void*)(sw + grp * 256), 4, off, 0, 0, 0);
    }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Weight fragments of a stage: per n-block jn, the lane's 32 k (k = 32h .. +31 of the stage) of
// weight row wrow0 + 32 jn -- 16 (FP4) or 32 (FP8) code bytes -- and their scale byte.
template <bool W8>
struct WFrag {
    u32x4 w[NJ][W8 ? 2 : 1];
    uint32_t s[NJ];
};

template <bool W8>
__device__ __forceinline__ void read_w(const uint8_t* st, const uint8_t* swin, uint32_t sbyte, uint32_t wrow0,
                                       uint32_t h, WFrag<W8>& f)
{
    using G = Geo<W8>;
#pragma unroll
    for (int jn = 0; jn < NJ; ++jn) {
        const uint32_t row = wrow0 + 32 * jn;
        if constexpr (W8) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
                f.w[jn][c] = *reinterpret_cast<const u32x4*>(st + X_BYTES + row * G::WROWB +
                                                            16 * wswz<W8>(row, 2 * h + c));
        } else {
            f.w[jn][0] = *reinterpret_cast<const u32x4*>(st + X_BYTES + row * G::WROWB + 16 * wswz<W8>(row, h));
        }
        f.s[jn] = swin[row * 16 + sbyte];
    }
}

// Activations of MFMA step T: per m-block i, k = 32h + 8T .. +7 of row xrow0 + 32 i.
template <int T>
__device__ __forceinline__ void read_x(const uint8_t* st, uint32_t xrow0, uint32_t h, u32x4 (&x)[MI])
{
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const uint32_t row = xrow0 + 32 * i;
        x[i] = *reinterpret_cast<const u32x4*>(st + row * XROWB + 16 * xswz(row, 4 * h + T));
    }
}

template <int FMT, bool W8>
__device__ __forceinline__ void dequant_w(const WFrag<W8>& f, uint32_t (&bw)[NJ][16])
{
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
}

// MFMA step T: the weights' pairs 4T .. 4T+3 (k = 32h + 8T .. +7) against the activations read
// for the same k.
template <int T>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[MI][NJ], const u32x4 (&x)[MI], const uint32_t (&bw)[NJ][16])
{
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jn = 0; jn < NJ; ++jn) {
            const u32x4 wv = {bw[jn][4 * T], bw[jn][4 * T + 1], bw[jn][4 * T + 2], bw[jn][4 * T + 3]};
            acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv),
                                                                 __builtin_bit_cast(bf16x8, x[i]), acc[i][jn], 0, 0, 0);
        }
}

template <int FMT, bool OUT_BF16, bool W8>
__global__ __launch_bounds__(THREADS) void gemm_a16w_kernel(const GemmArgs a)
{
    using G = Geo<W8>;
    constexpr int STAGE_BYTES = G::STAGE_BYTES, SWIN_OFF = G::SWIN_OFF, LPS = G::LOADS_PER_STAGE;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const uint32_t K = (uint32_t)a.k, ldx = (uint32_t)a.ldx;

    // tile mapping: with the n-tile count a multiple of 8, XCD x (= block % 8) takes n-tiles
    // x, x+8, ...; with the m-tile count a multiple of 4 it runs them for 4 m-tiles at a time,
    // so that the workgroups resident on an XCD share a few activation and weight tiles
    // through its L2; else, for each n-tile, every m-tile in turn
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

    // Pipeline, one stage per iteration: dequantize the stage's weights, then MFMA steps 0-2
    // with each step's activations read one step ahead; once this stage's reads have completed
    // and the next stage has landed, one barrier publishes it and frees this stage's buffer,
    // which receives the stage three ahead; the next stage's weights and step-0 activations
    // are read while step 3's MFMAs run.  Scale window j + 1 is requested at stage 8j.  Stages
    // past the end of k load as zeros (out-of-range offsets), so every iteration has the same
    // shape.
    const int S = (int)((K + BK - 1) / BK);
    issue_window(lds + SWIN_OFF, wave, lane, 0, sr, K);
#pragma unroll
    for (int p = 0; p < STAGES; ++p) issue_stage<W8>(lds + p * STAGE_BYTES, wave, lane, (uint32_t)p, xr, wr, ldx, K);

    const uint32_t r32 = lane & 31, h = lane >> 5;
    const uint32_t xrow0 = wm * 128 + r32, wrow0 = wn * 64 + r32;

    WFrag<W8> wf;
    u32x4 xa[MI], xb[MI];
    uint32_t bw[NJ][16];
    wait_vmcnt<(STAGES - 1) * LPS>();
    barrier_only();
    read_w(lds, lds + SWIN_OFF, h, wrow0, h, wf);
    read_x<0>(lds, xrow0, h, xa);

    uint32_t cur = 0;  // byte offset of stage s's buffer
    for (int s = 0; s < S; ++s) {
        const uint32_t nxt = cur + STAGE_BYTES == (uint32_t)(STAGES * STAGE_BYTES) ? 0u : cur + STAGE_BYTES;
        dequant_w<FMT, W8>(wf, bw);
        read_x<1>(lds + cur, xrow0, h, xb);
        mfma_step<0>(acc, xa, bw);
        read_x<2>(lds + cur, xrow0, h, xa);
        mfma_step<1>(acc, xb, bw);
        read_x<3>(lds + cur, xrow0, h, xb);
        mfma_step<2>(acc, xa, bw);
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkm0();
        // stage s+1 must have landed; issued after it: stage s+2 and, when s % 8 == 1, the
        // scale window requested just before stage s+2
        if (s % SPW == 1) wait_vmcnt<LPS + LOADS_PER_WINDOW>();
        else wait_vmcnt<LPS>();
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
        if (s % SPW == 0)
            issue_window(lds + SWIN_OFF + ((s / SPW + 1) & 1) * SWIN_BYTES, wave, lane, (uint32_t)(s / SPW) + 1, sr, K);
        issue_stage<W8>(lds + cur, wave, lane, (uint32_t)(s + STAGES), xr, wr, ldx, K);
        const int s1 = s + 1;
        read_w(lds + nxt, lds + SWIN_OFF + ((s1 / SPW) & 1) * SWIN_BYTES, 2 * (uint32_t)(s1 % SPW) + h, wrow0, h, wf);
        read_x<0>(lds + nxt, xrow0, h, xa);
        mfma_step<3>(acc, xb, bw);
        asm volatile("" ::: "memory");
        cur = nxt;
    }
    wait_vmcnt<0>();

    // Epilogue.  Transposed 32x32 result layout: for tile (i, jn) a lane holds output row
    // m = i*32 + lane%32 and, for group q = e/4, columns n = jn*32 + 8q + 4*(lane/32) + e%4.
    // A wave's 128 x 64 block is staged through LDS in passes of 64 (bf16) or 32 (fp32) rows
    // (a region per wave, rows padded against bank conflicts; the LDS accesses of one wave
    // complete in order, so a pass's writes follow the previous pass's reads) and written back
    // as whole 16-byte chunks.  Out-of-range chunks get an out-of-range offset and are dropped.
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
        constexpr int PASS_ROWS = OUT_BF16 ? 64 : 32;
        constexpr int IPP = PASS_ROWS / 32;                  // 32-row blocks per pass
        constexpr int PASSES = MI / IPP;
        static_assert(WAVES * PASS_ROWS * PITCH <= (uint32_t)G::LDS_BYTES, "epilogue staging exceeds LDS");
        uint8_t* stg = lds + wave * PASS_ROWS * PITCH;
        barrier_only();  // every wave is done reading the stage buffers
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
#pragma unroll
            for (int ii = 0; ii < IPP; ++ii)
#pragma unroll
                for (int jn = 0; jn < NJ; ++jn)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x16& c = acc[pass * IPP + ii][jn];
                        const float v0 = c[4 * q] * a.g, v1 = c[4 * q + 1] * a.g, v2 = c[4 * q + 2] * a.g, v3 = c[4 * q + 3] * a.g;
                        uint8_t* dst = stg + (ii * 32 + r32) * PITCH + (jn * 32 + 8 * q + 4 * h) * ESZ;
                        if constexpr (OUT_BF16) {
                            const u32x2 w = {__builtin_bit_cast(uint32_t, bf16x2{(__bf16)v0, (__bf16)v1}),
                                             __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v2, (__bf16)v3})};
                            *reinterpret_cast<u32x2*>(dst) = w;
                        } else {
                            *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
                        }
                    }
#pragma unroll
            for (uint32_t t = 0; t < PASS_ROWS / RPI; ++t) {
                const uint32_t row = t * RPI + lane / CPR, chunk = lane % CPR;
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * PITCH + chunk * 16);
                const uint32_t mm = wm * 128 + pass * PASS_ROWS + row, nn = wn * 64 + chunk * CE;
                const uint32_t off = (mm < mrows && nn < nrows) ? (mm * ldy + nn) * ESZ : kOOB;
                bstore128_nt(yr, off, v);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const uint32_t mm = wm * 128 + i * 32 + r32;
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
static hipError_t launch(const GemmArgs& a, hipStream_t st)
{
    constexpr int LDS = Geo<W8>::LDS_BYTES;
    // the LDS ring exceeds the default 64 KB dynamic limit
    static LdsLimit lim;
    if (const hipError_t e = lim.ensure((const void*)gemm_a16w_kernel<FMT, OUT_BF16, W8>, LDS, st); e != hipSuccess)
        return e;
    const unsigned tiles = (unsigned)(((a.m + BM - 1) / BM) * ((a.n + BN - 1) / BN));
    hipLaunchKernelGGL((gemm_a16w_kernel<FMT, OUT_BF16, W8>), dim3(tiles), dim3(THREADS), LDS, st, a);
    return hipGetLastError();
}

}  // namespace a16w

bool a16w_uses(const GemmArgs& a, bool w8)
{
    // m above one 128-row tile (smaller m would leave most of a 256-row tile empty); block 32
    // with whole 512-k scale windows, 16-byte aligned activation rows, 32-bit offsets within
    // the activation and output tiles
    const int64_t xspan = ((int64_t)(a16w::BM - 1) * a.ldx + a.k) * 2;
    const int64_t yspan = ((int64_t)(a16w::BM - 1) * a.ldy + a16w::BN) * (a.y_bf16 ? 2 : 4);
    if (!(a.m > 128 && a.block == 32 && a.k % a16w::SWIN_K == 0 && (a.ldx * 2) % 16 == 0 &&
          ((uintptr_t)a.x % 16) == 0 && xspan < 0x7FFFFFFF && yspan < 0x7FFFFFFF))
        return false;
    if (a.fmt != FMT_E8M0) return true;  // E4M3 / UE5M3: the narrow kernels are bound by dequantization
    // FP8 weights with E8M0 scales: the narrow kernel's ring is only two stages deep (64 KB
    // stages); the wide one was faster even with a last round half full (70B-FFN prefill:
    // 855 against 883 us).  FP4 weights with E8M0 scales take the two-workgroup kernel or the
    // 8-wave one: in cycles both beat this one (2048 x 16384 x 8192: 692 k / 780 k cycles per
    // XCD, modelled from the measured rounds, against 814 k measured)
    return w8;
}

hipError_t launch_gemm_a16w(const GemmArgs& a, bool w8, hipStream_t st)
{
    if (!a16w_uses(a, w8)) return hipErrorInvalidValue;
#define MXW(F, W) if (a.fmt == F) return a.y_bf16 ? a16w::launch<F, true, W>(a, st) : a16w::launch<F, false, W>(a, st);
    if (w8) {
        MXW(FMT_E4M3, true) MXW(FMT_UE5M3, true) MXW(FMT_E8M0, true)
    } else {
        MXW(FMT_E4M3, false) MXW(FMT_UE5M3, false) MXW(FMT_E8M0, false)
    }
#undef MXW
    return hipErrorInvalidValue;
}

}  // namespace mxk
