// mx_gemm_a16p.hip -- the large-m W4A16 GEMM with two independent workgroups per CU: the
// same product as mx_gemm_a16.hip, Y = X . dequant(Wq)^T with bf16 activations and fp32
// accumulation (gtnt.cn/news/16247 "为什么我们需要4-bit浮点量化", section 3.1: dequantize, then
// matmul; section 4.3: large batches dequantize on the fly; hotelren.com/news/2192771, article
// "量化技术演进与微缩量化原理", section 3.2 item 3: load the FP4 block, unpack, apply its
// scale, multiply, accumulate).
//
// Why a second kernel for the same tile: in the 8-wave kernel the per-stage barrier keeps the
// two waves of every SIMD in step, so both sit at the barrier at once and the matrix core
// idles there (measured: the main loop ran 182 k cycles per tile against 131 k cycles of MFMA
// work per SIMD, no wave ever waiting on memory).  Here a workgroup is 4 waves (one per
// SIMD) and its LDS ring is small enough for two workgroups per CU; a barrier then stalls only
// one of the two waves a SIMD holds, and the other one's MFMAs fill the gap.
//
// Tiling: a workgroup computes a 128 (m) x 256 (n) output tile; its 4 waves (2 x 2) compute
// 64 x 128 each, 2 x 4 MFMA results of 32 x 32 (bf16 32x32x16).  k advances 64 elements per
// stage through a 3-deep LDS ring filled by buffer_load ... lds (activations 128 rows x 128
// bytes, codes 256 rows x 32 bytes; rows and k beyond the tensors read as zero); the weight
// scales arrive per 256 k (256 rows x 8 bytes) in a double buffer of their own: 76 KB in all.
// Per stage a lane holds 32 consecutive k of its four weight rows (one 16-byte code load each)
// and dequantizes 8 of them per MFMA step, just before the step's MFMAs (16 bf16 registers
// per step instead of 64 per stage); its activations are read per 16-k step, one step ahead,
// in the same permuted k order (every dot product is unchanged).  The MFMA's A operand is the
// weight fragment, so each result tile is transposed; the epilogue stages it through LDS and
// writes whole 16-byte chunks.
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_wdeq.h"

namespace mxk {

namespace a16p {

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int WAVES = 4, THREADS = 64 * WAVES;
constexpr int MI = 2, NJ = 4;                      // per wave: 2 (m) x 4 (n) tiles of 32 x 32
constexpr int XROWB = BK * 2;                      // activation bytes per row per stage (128)
constexpr int X_BYTES = BM * XROWB;                // 16 KB
constexpr int WROWB = BK / 2;                      // code bytes per weight row per stage (32)
constexpr int W_BYTES = BN * WROWB;                // 8 KB
constexpr int STAGE_BYTES = X_BYTES + W_BYTES;     // 24 KB
constexpr int STAGES = 3;
constexpr int SWIN_K = 256;                        // k per scale window
constexpr int SPW = SWIN_K / BK;                   // stages per scale window (4)
constexpr int SWIN_ROWB = SWIN_K / 32;             // scale bytes per weight row per window (8)
constexpr int SWIN_BYTES = BN * SWIN_ROWB;         // 2 KB
constexpr int SWIN_OFF = STAGES * STAGE_BYTES;
constexpr int LDS_BYTES = SWIN_OFF + 2 * SWIN_BYTES;  // 77824: two workgroups fit in 160 KB
constexpr int XLOADS = BM / 8 / WAVES;             // per wave: loads of 8 activation rows (4)
constexpr int WLOADS = BN / 32 / WAVES;            // per wave: loads of 32 weight rows (2)
constexpr int LPS = XLOADS + WLOADS;               // loads per wave per stage
constexpr int LPW = BN / 32 / WAVES;               // per wave: scale loads of 32 rows x 8 bytes (2)
static_assert(2 * LDS_BYTES <= 160 * 1024, "two workgroups per CU");

typedef __attribute__((address_space(3))) void lds_void;

// LDS chunk permutations.  A 16-byte LDS read serves 16 lanes at a time, here 16 consecutive
// rows of one chunk column; the XORs give those 16 rows 16 different 16-byte bank groups:
// activation rows are 128 bytes (8 chunks), weight rows 32 bytes (2 chunks).
__device__ __forceinline__ uint32_t xswz(uint32_t row, uint32_t c) { return c ^ ((row >> 1) & 7u); }
__device__ __forceinline__ uint32_t wswz(uint32_t row, uint32_t c) { return c ^ ((row >> 3) & 1u); }

// This wave's share of stage s's loads into the stage buffer at `st`.  LDS-DMA writes lane i's
// 16 bytes at 16 i, so LDS slot l % 8 (activations) / l % 2 (codes) of a row receives the
// global chunk the permutation assigns to it.  Activations: 4 loads of 8 rows x 128 bytes;
// codes: 2 loads of 32 rows x 32 bytes.
__device__ __forceinline__ void issue_stage(uint8_t* st, int wave, int lane, uint32_t s, rsrc_t xr, rsrc_t wr,
                                            uint32_t ldx, uint32_t K)
{
    const uint32_t k0 = s * BK;
#pragma unroll
    for (int q = 0; q < XLOADS; ++q) {
        const uint32_t grp = (uint32_t)(wave * XLOADS + q);     // 8-row group, 0..15
        const uint32_t row = grp * 8 + (lane >> 3);
        const uint32_t c = xswz(row, lane & 7);
        const uint32_t kk = k0 + 8 * c;
        const uint32_t off = kk < K ? (row * ldx + kk) * 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(st + grp * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < WLOADS; ++q) {
        const uint32_t grp = (uint32_t)(wave * WLOADS + q);     // 32-row group, 0..7
        const uint32_t row = grp * 32 + (lane >> 1);
        const uint32_t c = wswz(row, lane & 1);
        const uint32_t kk = k0 + 32 * c;                        // first k of chunk c
        const uint32_t off = kk < K ? row * (K / 2) + kk / 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)(st + X_BYTES + grp * 1024), 16, off, 0, 0, 0);
    }
}

// This wave's share of scale window j (k = 256 j .. +255: 8 bytes per weight row): 2 loads of
// 32 rows x 8 bytes (lane: row lane/2, dword lane%2).  Requires k % 256 == 0 and (k / 32) % 4
// == 0, so that every row's window starts on a dword.
__device__ __forceinline__ void issue_window(uint8_t* sw, int wave, int lane, uint32_t j, rsrc_t sr, uint32_t K)
{
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
        const uint32_t grp = (uint32_t)(wave * LPW + q);        // 32-row group, 0..7
        const uint32_t row = grp * 32 + (lane >> 1);
        const uint32_t off = j * SWIN_K < K ? row * (K / 32) + j * SWIN_ROWB + 4 * (lane & 1) : kOOB;
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

// Weight fragments of a stage: per n-block jn, the lane's 32 k (k = 32h .. +31 of the stage)
// of weight row wrow0 + 32 jn -- 16 code bytes -- and their scale byte.
struct WFrag {
    u32x4 w[NJ];
    uint32_t s[NJ];
};

__device__ __forceinline__ void read_w(const uint8_t* st, const uint8_t* swin, uint32_t sbyte, uint32_t wrow0,
                                       uint32_t h, WFrag& f)
{
#pragma unroll
    for (int jn = 0; jn < NJ; ++jn) {
        const uint32_t row = wrow0 + 32 * jn;
        f.w[jn] = *reinterpret_cast<const u32x4*>(st + X_BYTES + row * WROWB + 16 * wswz(row, h));
        f.s[jn] = swin[row * SWIN_ROWB + sbyte];
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

// MFMA step: code dword cw[jn] (8 k of weight row jn) dequantized into 4 bf16 pairs, against
// the activations read for the same k.
template <int FMT>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[MI][NJ], const u32x4 (&x)[MI], const uint32_t (&cw)[NJ],
                                          const WScale<FMT> (&ws)[NJ])
{
    u32x4 bw[NJ];
#pragma unroll
    for (int jn = 0; jn < NJ; ++jn)
        bw[jn] = u32x4{deq_pair_bf16<FMT, 0>(cw[jn], ws[jn]), deq_pair_bf16<FMT, 1>(cw[jn], ws[jn]),
                       deq_pair_bf16<FMT, 2>(cw[jn], ws[jn]), deq_pair_bf16<FMT, 3>(cw[jn], ws[jn])};
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jn = 0; jn < NJ; ++jn)
            acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bw[jn]),
                                                                 __builtin_bit_cast(bf16x8, x[i]), acc[i][jn], 0, 0, 0);
}

template <int FMT, bool OUT_BF16>
__global__ __launch_bounds__(THREADS, 2) void gemm_a16p_kernel(const GemmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t K = (uint32_t)a.k, ldx = (uint32_t)a.ldx;

    // tile mapping: with the n-tile count a multiple of 8, XCD x (= block % 8) takes n-tiles
    // x, x+8, ...; with the m-tile count a multiple of 4 it runs them in groups of 4 m-tiles
    // (all its n-tiles for m-tiles 0-3, then 4-7, ...), so that the workgroups resident on an
    // XCD share a few activation and weight tiles through its L2; else, for each n-tile,
    // every m-tile in turn
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
    const rsrc_t wr = make_rsrc(a.wc + n0 * (int64_t)(K / 2), nrows * (K / 2));
    const rsrc_t sr = make_rsrc(a.ws + n0 * (a.k / 32), nrows * (K / 32));

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Pipeline, one stage per iteration: MFMA steps 0-2 with each step's activations read one
    // step ahead; once this stage's reads have completed and the next stage has landed, one
    // barrier publishes it and frees this stage's buffer, which receives the stage three
    // ahead; the next stage's weights and step-0 activations are read while step 3's MFMAs
    // run (step 3's codes and scales are kept aside for it).  Scale window j + 1 is requested
    // at stage 4j.  Stages past the end of k load as zeros (out-of-range offsets), so every
    // iteration has the same shape.
    const int S = (int)((K + BK - 1) / BK);
    issue_window(lds + SWIN_OFF, wave, lane, 0, sr, K);
#pragma unroll
    for (int p = 0; p < STAGES; ++p) issue_stage(lds + p * STAGE_BYTES, wave, lane, (uint32_t)p, xr, wr, ldx, K);

    const uint32_t r32 = lane & 31, h = lane >> 5;
    const uint32_t xrow0 = wm * 64 + r32, wrow0 = wn * 128 + r32;

    WFrag wf;
    u32x4 xa[MI], xb[MI];
    wait_vmcnt<(STAGES - 1) * LPS>();
    barrier_only();
    read_w(lds, lds + SWIN_OFF, h, wrow0, h, wf);
    read_x<0>(lds, xrow0, h, xa);

    uint32_t cur = 0;  // byte offset of stage s's buffer
    for (int s = 0; s < S; ++s) {
        const uint32_t nxt = cur + STAGE_BYTES == (uint32_t)(STAGES * STAGE_BYTES) ? 0u : cur + STAGE_BYTES;
        WScale<FMT> ws[NJ];
        uint32_t c0[NJ], c1[NJ], c2[NJ], c3[NJ];
#pragma unroll
        for (int jn = 0; jn < NJ; ++jn) {
            ws[jn] = wscale<FMT>(wf.s[jn]);
            c0[jn] = wf.w[jn].x; c1[jn] = wf.w[jn].y; c2[jn] = wf.w[jn].z; c3[jn] = wf.w[jn].w;
        }
        read_x<1>(lds + cur, xrow0, h, xb);
        mfma_step<FMT>(acc, xa, c0, ws);
        read_x<2>(lds + cur, xrow0, h, xa);
        mfma_step<FMT>(acc, xb, c1, ws);
        read_x<3>(lds + cur, xrow0, h, xb);
        mfma_step<FMT>(acc, xa, c2, ws);
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkm0();
        // stage s+1 must have landed; issued after it: stage s+2 and, when s % 4 == 1, the
        // scale window requested just before stage s+2
        if (s % SPW == 1) wait_vmcnt<LPS + LPW>();
        else wait_vmcnt<LPS>();
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
        if (s % SPW == 0)
            issue_window(lds + SWIN_OFF + ((s / SPW + 1) & 1) * SWIN_BYTES, wave, lane, (uint32_t)(s / SPW) + 1, sr, K);
        issue_stage(lds + cur, wave, lane, (uint32_t)(s + STAGES), xr, wr, ldx, K);
        const int s1 = s + 1;
        read_w(lds + nxt, lds + SWIN_OFF + ((s1 / SPW) & 1) * SWIN_BYTES, 2 * (uint32_t)(s1 % SPW) + h, wrow0, h, wf);
        read_x<0>(lds + nxt, xrow0, h, xa);
        mfma_step<FMT>(acc, xb, c3, ws);
        asm volatile("" ::: "memory");
        cur = nxt;
    }
    wait_vmcnt<0>();

    // Epilogue.  Transposed 32x32 result layout: for tile (i, jn) a lane holds output row
    // m = i*32 + lane%32 and, for group q = e/4, columns n = jn*32 + 8q + 4*(lane/32) + e%4.
    // A wave's 64 x 128 block is staged through LDS in passes of 64 (bf16) or 32 (fp32) rows
    // (a region per wave, rows padded against bank conflicts; the LDS accesses of one wave
    // complete in order, so a pass's writes follow the previous pass's reads) and written back
    // as whole 16-byte chunks.  Out-of-range chunks get an out-of-range offset and are dropped.
    constexpr uint32_t ESZ = OUT_BF16 ? 2 : 4;
    const rsrc_t yr = make_rsrc(static_cast<uint8_t*>(a.y) + (m0 * a.ldy + n0) * ESZ, 0x7FFFFFFFu);
    const uint32_t ldy = (uint32_t)a.ldy;
    constexpr uint32_t CE = 16 / ESZ;
    const bool vec = (ldy % CE) == 0 && (nrows % CE) == 0;
    if (vec) {
        constexpr uint32_t RB = 128 * ESZ;                   // bytes of a wave row (128 columns)
        constexpr uint32_t PITCH = RB + 16;
        constexpr uint32_t CPR = RB / 16;                    // chunks per row (16 or 32)
        constexpr uint32_t RPI = 64 / CPR;                   // rows per store instruction
        constexpr int PASS_ROWS = OUT_BF16 ? 64 : 32;
        constexpr int IPP = PASS_ROWS / 32;                  // 32-row blocks per pass
        constexpr int PASSES = MI / IPP;
        static_assert(WAVES * PASS_ROWS * PITCH <= (uint32_t)LDS_BYTES, "epilogue staging exceeds LDS");
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
                const uint32_t mm = wm * 64 + pass * PASS_ROWS + row, nn = wn * 128 + chunk * CE;
                const uint32_t off = (mm < mrows && nn < nrows) ? (mm * ldy + nn) * ESZ : kOOB;
                bstore128_nt(yr, off, v);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const uint32_t mm = wm * 64 + i * 32 + r32;
#pragma unroll
            for (int jn = 0; jn < NJ; ++jn)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t nn = wn * 128 + jn * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                    const uint32_t off = (mm < mrows && nn < nrows) ? (mm * ldy + nn) * ESZ : kOOB;
                    const float v = acc[i][jn][e] * a.g;
                    if constexpr (OUT_BF16) bstore16(yr, off, __builtin_bit_cast(uint16_t, (__bf16)v));
                    else bstore32(yr, off, __builtin_bit_cast(uint32_t, v));
                }
        }
    }
}

template <int FMT, bool OUT_BF16>
static hipError_t launch(const GemmArgs& a, hipStream_t st)
{
    // the LDS ring exceeds the default 64 KB dynamic limit
    static LdsLimit lim;
    if (const hipError_t e = lim.ensure((const void*)gemm_a16p_kernel<FMT, OUT_BF16>, LDS_BYTES, st); e != hipSuccess)
        return e;
    const unsigned tiles = (unsigned)(((a.m + BM - 1) / BM) * ((a.n + BN - 1) / BN));
    hipLaunchKernelGGL((gemm_a16p_kernel<FMT, OUT_BF16>), dim3(tiles), dim3(THREADS), LDS_BYTES, st, a);
    return hipGetLastError();
}

}  // namespace a16p

bool a16p_uses(const GemmArgs& a)
{
    // E8M0 scales (with E4M3 / UE5M3 a dequantized pair costs four vector instructions and
    // the 128 x 64 wave tiles of the wide kernel halve them per MFMA), under the conditions of
    // the 8-wave kernel (a16_uses_tiled: block 32, k % 512 == 0, aligned activation rows,
    // 32-bit tile offsets), and more 128 x 256 tiles than CUs: with at most one tile per CU a
    // lone 4-wave workgroup has nothing to hide its barriers behind and the 8-wave kernel is
    // faster (m 256, n 28672, k 8192: 111 against 129 us); from 257 tiles on, the CUs that
    // run two workgroups at once finish first or level (modelled per CU: 346 k cycles for
    // a pair against 390 k for two 8-wave tiles in turn, at k 8192)
    constexpr int64_t CUS = 256;
    const int64_t tiles = ((a.m + a16p::BM - 1) / a16p::BM) * ((a.n + a16p::BN - 1) / a16p::BN);
    return a.fmt == FMT_E8M0 && a.block == 32 && tiles > CUS && a16_uses_tiled(a);
}

hipError_t launch_gemm_a16p(const GemmArgs& a, hipStream_t st)
{
    if (!a16p_uses(a)) return hipErrorInvalidValue;
    return a.y_bf16 ? a16p::launch<FMT_E8M0, true>(a, st) : a16p::launch<FMT_E8M0, false>(a, st);
}

}  // namespace mxk
