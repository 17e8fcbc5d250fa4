// mx_gemm_a4.hip -- W4A4 GEMM on gfx950's block-scaled FP4 matrix cores:
// Y[m][n] = g * sum_k e(xq[m][k]) 2^(sx-127) * e(wq[n][k]) 2^(sw-127)
// (gtnt.cn/news/16247 "为什么我们需要4-bit浮点量化", section 3.1: dequantize then matmul --
// here the matrix cores apply the E8M0 block scales themselves; hotelren.com/news/2192771
// article "量化技术演进与微缩量化原理", section 6 item 1: FP4 activations with block scales).
//
// Tiling: a workgroup computes a 256 x 256 output tile with 4 waves (2 x 2), each a 128 x 128
// sub-tile of 4 x 4 v_mfma_scale_f32_32x32x64_f8f6f4 results (FP4 operands, fp32
// accumulators in AGPRs).  The k loop advances 128 elements per stage; each stage's operand
// tiles (256 rows x 64 code bytes for X and for W, plus 4 E8M0 bytes per row) travel
// HBM -> LDS with buffer_load ... lds (no register round trip; rows or k beyond the tensor
// read as zero), through a 3-deep ring of LDS buffers so that two stages are in flight while
// one is computed.  In LDS, the four 16-byte chunks of each 64-byte row are rotated by
// (row / 4) % 4 so that the fragment reads (32 rows x 16 bytes per half-wave) hit distinct
// banks.  In the row-major layout a lane's 16 code bytes (32 consecutive k of one row) and
// its scale byte are exactly one MFMA operand slice and the scale that goes with it.
// Workgroups are mapped so that the m-tiles sharing a weight tile run on the same XCD.
#include "mx_device.h"
#include "mx_internal.h"

namespace mxk {

namespace a4 {

constexpr int BM = 256, BN = 256, BK = 128, STAGES = 3;
constexpr int ROWB = BK / 2;                       // code bytes per row per stage (64)
constexpr int CODE_BYTES = BM * ROWB;              // 16 KB per operand per stage
constexpr int SCALE_BYTES = BM * (BK / 32);        // 1 KB per operand per stage
constexpr int STAGE_BYTES = 2 * CODE_BYTES + 2 * SCALE_BYTES;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;    // 104448
constexpr int LOADS_PER_STAGE = 10;                // per wave: 4 + 4 code loads, 1 + 1 scale loads

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) { return chunk ^ ((row >> 2) & 3u); }

// Issue one stage's loads (this wave's share) into LDS stage buffer `buf`.
__device__ __forceinline__ void issue_stage(uint8_t* lds, int buf, int wave, int lane, uint32_t k0,
                                            rsrc_t ac, rsrc_t bc, rsrc_t as, rsrc_t bs,
                                            uint32_t K)
{
    uint8_t* st = lds + buf * STAGE_BYTES;
    const uint32_t rowb = K / 2, srow = K / 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t row = (uint32_t)(wave * 4 + q) * 16 + (lane >> 2);   // 16 rows per load
        const uint32_t c = swz(row, lane & 3);                              // global chunk
        const uint32_t kk = k0 + 32 * c;
        const uint32_t off = kk < K ? row * rowb + kk / 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ac, (lds_void*)(st + (wave * 4 + q) * 1024), 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(bc, (lds_void*)(st + CODE_BYTES + (wave * 4 + q) * 1024), 16, off, 0, 0, 0);
    }
    const uint32_t srow_i = (uint32_t)wave * 64 + lane;  // one scale dword (4 bytes = 128 k) per row
    const uint32_t soff = k0 < K ? srow_i * srow + k0 / 32 : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(as, (lds_void*)(st + 2 * CODE_BYTES + wave * 256), 4, soff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(bs, (lds_void*)(st + 2 * CODE_BYTES + SCALE_BYTES + wave * 256), 4, soff, 0, 0, 0);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the memory fence of __syncthreads (which would also wait for
// the prefetches of later stages): each wave has already waited for its own loads of the
// stage about to be read; the clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

template <bool OUT_BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_a4_kernel(const GemmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t K = (uint32_t)a.k;

    // tile mapping: with the n-tile count a multiple of 8, XCD x (= block % 8) takes n-tiles
    // x, x+8, ... and, for each, every m-tile in turn
    const uint32_t MT = (uint32_t)((a.m + BM - 1) / BM), NT = (uint32_t)((a.n + BN - 1) / BN);
    uint32_t mt, nt;
    if ((NT & 7) == 0) {
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
    const rsrc_t ac = make_rsrc(a.xq_codes + m0 * (a.k / 2), mrows * (K / 2));
    const rsrc_t bc = make_rsrc(a.wc + n0 * (a.k / 2), nrows * (K / 2));
    const rsrc_t as = make_rsrc(a.xq_scales + m0 * (a.k / 32), mrows * (K / 32));
    const rsrc_t bs = make_rsrc(a.ws + n0 * (a.k / 32), nrows * (K / 32));

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int S = (int)((K + BK - 1) / BK);
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
        if (p < S) issue_stage(lds, p, wave, lane, (uint32_t)p * BK, ac, bc, as, bs, K);

    const uint32_t r32 = lane & 31, h = lane >> 5;
    for (int s = 0; s < S; ++s) {
        if (s + 1 < S) wait_vmcnt<LOADS_PER_STAGE>();
        else wait_vmcnt<0>();
        barrier_only();
        if (s + STAGES - 1 < S)
            issue_stage(lds, (s + STAGES - 1) % STAGES, wave, lane, (uint32_t)(s + STAGES - 1) * BK, ac, bc, as, bs, K);
        const uint8_t* st = lds + (s % STAGES) * STAGE_BYTES;
        const uint32_t* sa = reinterpret_cast<const uint32_t*>(st + 2 * CODE_BYTES);
        const uint32_t* sbw = reinterpret_cast<const uint32_t*>(st + 2 * CODE_BYTES + SCALE_BYTES);
        uint32_t ascale[4], bscale[4];
        u32x4 fa[2][4], fb[2][4];  // fragments of k-step j in set j (both sets in flight)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t c = 2 * j + h;  // this lane's 16-byte chunk of the 64-byte row
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t ra = wm * 128 + i * 32 + r32;
                const uint32_t rb = wn * 128 + i * 32 + r32;
                fa[j][i] = *reinterpret_cast<const u32x4*>(st + ra * ROWB + 16 * swz(ra, c));
                fb[j][i] = *reinterpret_cast<const u32x4*>(st + CODE_BYTES + rb * ROWB + 16 * swz(rb, c));
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ascale[i] = sa[wm * 128 + i * 32 + r32];
            bscale[i] = sbw[wn * 128 + i * 32 + r32];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {  // two MFMA k-steps of 64
            const uint32_t c = 2 * j + h;
            int asx[4], bsx[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                asx[i] = (int)((ascale[i] >> (8 * c)) & 0xFFu);
                bsx[i] = (int)((bscale[i] >> (8 * c)) & 0xFFu);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jn = 0; jn < 4; ++jn) {
                    const i32x8 av = {(int)fa[j][i].x, (int)fa[j][i].y, (int)fa[j][i].z, (int)fa[j][i].w, 0, 0, 0, 0};
                    const i32x8 bv = {(int)fb[j][jn].x, (int)fb[j][jn].y, (int)fb[j][jn].z, (int)fb[j][jn].w, 0, 0, 0, 0};
                    acc[i][jn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        av, bv, acc[i][jn], 4, 4, 0, asx[i], 0, bsx[jn]);
                }
        }
    }

    // epilogue: 32x32 result layout -- lane holds rows 8*(e/4) + 4*(lane/32) + e%4, column lane%32
    const bool full = m0 + BM <= a.m && n0 + BN <= a.n;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) {
            const int64_t n = n0 + wn * 128 + jn * 32 + r32;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                if (full || (m < a.m && n < a.n)) {
                    const float v = acc[i][jn][e] * a.g;
                    if constexpr (OUT_BF16) reinterpret_cast<__bf16*>(a.y)[m * a.ldy + n] = (__bf16)v;
                    else reinterpret_cast<float*>(a.y)[m * a.ldy + n] = v;
                }
            }
        }
}

}  // namespace a4

hipError_t launch_gemm_a4_mfma(const GemmArgs& a, hipStream_t st)
{
    // the LDS ring exceeds the default 64 KB dynamic limit; raise it once (thread-safe
    // function-local static initialisation)
    static const hipError_t attr_bf16 = hipFuncSetAttribute(
        (const void*)a4::gemm_a4_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, a4::LDS_BYTES);
    static const hipError_t attr_f32 = hipFuncSetAttribute(
        (const void*)a4::gemm_a4_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, a4::LDS_BYTES);
    if (attr_bf16 != hipSuccess || attr_f32 != hipSuccess) return attr_bf16 != hipSuccess ? attr_bf16 : attr_f32;
    const unsigned tiles = (unsigned)(((a.m + a4::BM - 1) / a4::BM) * ((a.n + a4::BN - 1) / a4::BN));
    if (a.y_bf16) hipLaunchKernelGGL(a4::gemm_a4_kernel<true>, dim3(tiles), dim3(256), a4::LDS_BYTES, st, a);
    else hipLaunchKernelGGL(a4::gemm_a4_kernel<false>, dim3(tiles), dim3(256), a4::LDS_BYTES, st, a);
    return hipGetLastError();
}

}  // namespace mxk
