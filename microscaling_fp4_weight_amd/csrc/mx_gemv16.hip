// mx_gemv16.hip -- W4A16 GEMV for decode batches, 2 <= m <= 16, k = 4096, blocks of 32 and
// more: Y = X . dequant(Wq)^T with the weights read once, in address order.
//
// Method: gtnt.cn/news/16247 "为什么我们需要4-bit浮点量化", section 4.3 (small batches keep the
// weights quantized) and section 3.1 (dequantize, then multiply); hotelren.com/news/2192771,
// article "量化技术演进与微缩量化原理", section 3.2 item 3 (load FP4 -> unpack -> scale ->
// multiply -> accumulate).
//
// Work is split in units of 16 weight rows (16 x 2 KB of codes, contiguous): workgroup b takes
// units b, b + G, ..., so at any time the GPU streams one contiguous window of the weight.  Each
// of the 16 waves of a workgroup owns one 256-k slice of every row and keeps the activations of
// that slice in registers for the whole launch, as the B operand of bf16 MFMA 16x16x32 (X rows
// are the 16 columns; rows past m are zero).  A unit's codes reach LDS by LDS-DMA in pieces of
// 8 rows x 128 bytes (whole cache lines; the 16-byte chunks of each row permuted by XOR with
// the row's low bits), and each lane reads back the 16 bytes of its MFMA A-operand row (16
// weight rows per MFMA) without bank conflicts; only the wave itself reads what it loaded, so
// the loop has no barrier.  A wave keeps two of its units in flight: the loads of the next go
// out as soon as one has been computed, so that the GPU streams a window of about two units per
// CU (16 MB at n 14336) rather than requesting the whole weight at once (that was 7% slower at
// n 14336, m 2 to 16).  The waves' partial sums of each unit meet in LDS at the end, in a fixed
// order.
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_wdeq.h"

namespace mxk {
namespace g16 {

constexpr uint32_t KTOT = 4096;  // k handled by this kernel

constexpr int WAVES = 16;                         // waves per workgroup; wave w owns k slice w
constexpr uint32_t GRID_CAP = 256;                // workgroups (one per CU)
constexpr int THREADS = 64 * WAVES;
constexpr uint32_t KCHUNK = KTOT / WAVES;         // k per wave slice (256)
constexpr uint32_t CPR = KCHUNK / 32;             // 16-byte code chunks per row of a slice
constexpr uint32_t RPI = 64 / CPR;                // rows per LDS-DMA instruction
constexpr int NDMA = 16 / RPI;                    // LDS-DMA instructions per unit
constexpr int JP = CPR / 4;                       // code chunks per lane per unit
constexpr uint32_t UNIT_LDS = 16 * KCHUNK / 2;    // bytes of a unit's slice (16 rows)
constexpr uint32_t SCALE_UNIT = 2048;             // LDS bytes per unit for its scales (16 x k/32 at most)

// LDS layout for a workgroup of at most MAXU units, each with buffers of its own: each wave's
// code buffers, then the scales of every unit; the final reduction reuses the code buffers.
template <int MAXU>
struct Lay {
    static constexpr uint32_t WAVE_LDS = MAXU * UNIT_LDS;
    static constexpr uint32_t CODE_LDS = WAVES * WAVE_LDS;
    static constexpr uint32_t BYTES = CODE_LDS + MAXU * SCALE_UNIT;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(MAXU * WAVES * 1024 <= CODE_LDS, "reduction buffer");
};

typedef __attribute__((address_space(3))) void lds_void;

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ f32x4 mfma(const uint32_t* a4, const uint32_t* b4, f32x4 c)
{
    const u32x4 av = {a4[0], a4[1], a4[2], a4[3]};
    const u32x4 bv = {b4[0], b4[1], b4[2], b4[3]};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                   __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
}

template <bool OUT_BF16>
__device__ __forceinline__ void store_out(void* y, int64_t ldy, int64_t m, int64_t n, float v)
{
    if constexpr (OUT_BF16) reinterpret_cast<__bf16*>(y)[m * ldy + n] = (__bf16)v;
    else reinterpret_cast<float*>(y)[m * ldy + n] = v;
}

// A unit's scale bytes (16 rows x k/BLOCK, contiguous in the row-major layout) sit in LDS as
// 16-byte pieces, piece q of row r at slot r PPR + (q ^ (r % PPR)) (PPR pieces per row), so
// that the 16 lanes reading one row each find their bytes in distinct banks.
template <int BLOCK>
struct SC {
    static constexpr uint32_t ROWB = KTOT / BLOCK;              // scale bytes per row
    static constexpr uint32_t PPR = ROWB / 16;                  // 16-byte pieces per row
    static constexpr uint32_t NB = KCHUNK / BLOCK;              // bytes of a wave's slice
    static constexpr int NDMA = (16 * ROWB + 1023) / 1024;      // LDS-DMA loads per unit
};

// The slice's scale bytes of row r of a unit's LDS image (NB bytes, packed from byte 0).
template <int BLOCK>
__device__ __forceinline__ u32x4 lds_slice_scales(const uint8_t* unit_sc, uint32_t r, uint32_t wave)
{
    using S = SC<BLOCK>;
    const uint32_t o = wave * S::NB, q = o / 16;
    const uint8_t* p = unit_sc + 16 * (r * S::PPR + (q ^ (r & (S::PPR - 1)))) + (o % 16);
    if constexpr (S::NB == 16) return *reinterpret_cast<const u32x4*>(p);
    if constexpr (S::NB == 8) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
        return u32x4{v.x, v.y, 0u, 0u};
    }
    if constexpr (S::NB == 4) return u32x4{*reinterpret_cast<const uint32_t*>(p), 0u, 0u, 0u};
    if constexpr (S::NB == 2) return u32x4{*reinterpret_cast<const uint16_t*>(p), 0u, 0u, 0u};
    return u32x4{*p, 0u, 0u, 0u};
}

// Scale byte of 32-k chunk cc of the slice.
template <int BLOCK>
__device__ __forceinline__ uint32_t chunk_scale(const u32x4 s, uint32_t cc)
{
    const uint32_t idx = cc / (BLOCK / 32);
    return (s[idx >> 2] >> (8 * (idx & 3))) & 0xFFu;
}

template <int BLOCK, int FMT, bool OUT_BF16, int MAXU>
__global__ __launch_bounds__(THREADS) void gemv16_kernel(const GemmArgs a)
{
    constexpr int DEPTH = MAXU;
    using LY = Lay<MAXU>;
    constexpr uint32_t WAVE_LDS = LY::WAVE_LDS, CODE_LDS = LY::CODE_LDS;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t r = lane & 15, g = lane >> 4;  // MFMA operand row (A: weight row, B: X row), k group
    const uint32_t N = (uint32_t)a.n, M = (uint32_t)a.m, K = KTOT;
    const uint32_t U = (N + 15) / 16, G = gridDim.x;
    const uint32_t nu = (U - blockIdx.x + G - 1) / G;  // 1..MAXU (launch)
    const uint32_t kw0 = wave * KCHUNK;
    const rsrc_t wr = make_rsrc(a.wc, N * (K / 2));
    const rsrc_t sr = make_rsrc(a.ws, N * (K / BLOCK));
    const rsrc_t xr = make_rsrc(a.x, (uint32_t)(((int64_t)(M - 1) * a.ldx + K) * 2));
    const uint32_t wbase = wave * WAVE_LDS;
    using S = SC<BLOCK>;

    // the scales of every unit slot of the workgroup, by LDS-DMA from waves 0 .. MAXU NDMA - 1
    // (one 1 KB piece each, issued first), visible to all waves after the barrier below.  Every
    // slot is loaded, also past the workgroup's last unit (such loads are out of range: no
    // memory traffic, zeros in LDS), so that the number of loads in flight is the same on every
    // path and each wait below waits for exactly what it needs.
    const bool sc_wave = wave < MAXU * S::NDMA;
    if (sc_wave) {
        const uint32_t i = wave / S::NDMA, part = wave % S::NDMA, u = blockIdx.x + i * G;
        const uint32_t slot = part * 64 + lane, r0 = slot / S::PPR, q = (slot % S::PPR) ^ (r0 & (S::PPR - 1));
        const uint32_t row = u * 16 + r0;
        const uint32_t off = i < nu && r0 < 16 && row < N ? row * S::ROWB + 16 * q : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void*)(lds + CODE_LDS + SCALE_UNIT * i + 1024 * part), 16, off, 0, 0, 0);
    }

    // unit u's codes of this wave's slice into buffer b: LDS-DMA j brings rows RPI j ..
    // RPI j + RPI - 1 (lane -> row RPI j + lane / CPR, chunk (lane % CPR) ^ (row % 8))
    auto issue = [&](uint32_t i, uint32_t b) {
        const uint32_t u = blockIdx.x + i * G;
#pragma unroll
        for (int j = 0; j < NDMA; ++j) {
            const uint32_t row = RPI * j + lane / CPR, c = (lane % CPR) ^ (row & 7), grow = u * 16 + row;
            const uint32_t off = i < nu && grow < N ? grow * (K / 2) + kw0 / 2 + 16 * c : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)(lds + wbase + UNIT_LDS * b + 1024 * j), 16, off, 0, 0, 0);
        }
    };

    // this wave's X slice as B operands: xb[jp][4 t + d] = dword d of X row r at
    // k = kw0 + 32 (4 jp + g) + 8 t.  Loaded as whole 64-byte pieces of a row (load t' of jp:
    // lane (g, r) takes bytes 16 g of the piece of 32-k chunk 4 jp + t'), which leaves piece t'
    // of the lanes of row group g where the MFMA wants piece g of row group t': a 4 x 4
    // transpose across the four 16-lane row groups, done with two rounds of lane swaps.
    uint32_t xb[JP][16];
#pragma unroll
    for (int jp = 0; jp < JP; ++jp) {
        u32x4 v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            v[t] = bload128(xr, r < M ? (uint32_t)(r * a.ldx + kw0 + 32 * (4 * jp + t)) * 2 + 16 * g : kOOB);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int d = 0; d < 4; ++d) xb[jp][4 * t + d] = v[t][d];
    }
    // then the first INFL unit slots (the X loads go first: they hit in L2 and are back before
    // the first unit's codes; issued after the first unit, or later, they delayed the first
    // MFMA).  Every slot up to MAXU is issued in turn, also past the workgroup's last unit
    // (out of range: zeros in LDS, no memory traffic), so that each wait below is a constant.
    constexpr int INFL = DEPTH < 2 ? DEPTH : 2;
#pragma unroll
    for (int i = 0; i < INFL; ++i) issue(i, i);
    // the scale loads were issued before everything else: wait for them alone, then share
    if (sc_wave) wait_vmcnt<INFL * NDMA + 4 * JP>();
    // a barrier without the memory fence of __syncthreads, which would also wait for the code
    // loads still in flight
    asm volatile("s_barrier" ::: "memory");
#pragma unroll
    for (int jp = 0; jp < JP; ++jp)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            // rows 2, 3 of pieces 0 / 1 <-> rows 0, 1 of pieces 2 / 3; then odd rows of pieces
            // 0 / 2 <-> even rows of pieces 1 / 3
            const auto s02 = __builtin_amdgcn_permlane32_swap(xb[jp][d], xb[jp][8 + d], false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(xb[jp][4 + d], xb[jp][12 + d], false, false);
            const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
            const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
            xb[jp][d] = s01[0];
            xb[jp][4 + d] = s01[1];
            xb[jp][8 + d] = s23[0];
            xb[jp][12 + d] = s23[1];
        }

    f32x4 acc[MAXU];
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if ((uint32_t)i >= nu) {
            if (i + INFL < DEPTH) issue(i + INFL, i + INFL);
            continue;
        }
        const uint32_t b = i;
        // unit i's codes have landed (slots i + 1 .. i + INFL - 1 may be in flight)
        constexpr int last = DEPTH - 1;
        if (last - i >= INFL - 1 && INFL > 1) wait_vmcnt<(INFL > 1 ? NDMA : 0)>();
        else wait_vmcnt<0>();
        asm volatile("" ::: "memory");  // the LDS reads below stay after the wait
        const uint8_t* buf = lds + wbase + UNIT_LDS * b + 1024 * (r / RPI) + 16 * ((r % RPI) * CPR);
        const u32x4 sc = lds_slice_scales<BLOCK>(lds + CODE_LDS + SCALE_UNIT * i, r, wave);
        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jp = 0; jp < JP; ++jp) {
            const uint32_t cc = 4 * jp + g;
            const u32x4 cw = *reinterpret_cast<const u32x4*>(buf + 16 * (cc ^ (r & 7)));
            uint32_t bw[16];
            dequant32<BLOCK, FMT>(cw, chunk_scale<BLOCK>(sc, cc), bw);
#pragma unroll
            for (int t = 0; t < 4; ++t) c = mfma(&bw[4 * t], &xb[jp][4 * t], c);
        }
        acc[i] = c;
        if (i + INFL < DEPTH) issue(i + INFL, i + INFL);
    }

    // partial sums of every unit: [unit][wave][lane]; then every thread sums one output over
    // the waves in wave order (fixed, so the result does not depend on timing); the columns
    // of X rows past m are zero padding and are skipped.  The partials overwrite the code
    // buffers, into which a workgroup with fewer units than slots may still have LDS-DMA
    // loads of its unused slots in flight (out of range: they write zeros): wait for them.
    wait_vmcnt<0>();
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
    for (int i = 0; i < MAXU; ++i)
        if ((uint32_t)i < nu) red[(i * WAVES + wave) * 64 + lane] = acc[i];
    __syncthreads();
    const uint32_t t = threadIdx.x;
#pragma unroll
    for (uint32_t t0 = 0; t0 < MAXU * 256; t0 += THREADS) {
        const uint32_t e = t0 + t, i = e / 256, l = (e / 4) % 64, comp = e % 4;  // output (unit, lane, row)
        if (i < nu && l % 16 < M) {
            const float* rf = reinterpret_cast<const float*>(lds);
            float v = rf[((i * WAVES) * 64 + l) * 4 + comp];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) v += rf[((i * WAVES + w) * 64 + l) * 4 + comp];
            // lane l holds column l % 16 (row of X) and weight rows 4 (l / 16) + comp of the unit
            const uint32_t mrow = l % 16, n = (blockIdx.x + i * G) * 16 + 4 * (l / 16) + comp;
            if (mrow < M && n < N) store_out<OUT_BF16>(a.y, a.ldy, mrow, n, v * a.g);
        }
    }
}

}  // namespace g16

bool gemv16_applies(const GemmArgs& a)
{
    if (a.m < 2 || a.m > 16 || a.k != (int64_t)g16::KTOT || a.block < 32) return false;
    if (a.ws_tiled || a.ws_pre) return false;
    if ((a.ldx * 2) % 16 != 0 || (uintptr_t)a.x % 16 != 0) return false;
    if (((a.m - 1) * a.ldx + a.k) * 2 >= (int64_t(1) << 31)) return false;
    if (a.n * (a.k / 2) >= (int64_t(1) << 31)) return false;
    return true;
}

template <int BLOCK, int FMT, bool OUT_BF16, int MAXU>
static hipError_t launch_one(const GemmArgs& a, uint32_t grid, hipStream_t st)
{
    const void* k = (const void*)g16::gemv16_kernel<BLOCK, FMT, OUT_BF16, MAXU>;
    static LdsLimit lim;
    if (const hipError_t e = lim.ensure(k, g16::Lay<MAXU>::BYTES, st); e != hipSuccess) return e;
    hipLaunchKernelGGL((g16::gemv16_kernel<BLOCK, FMT, OUT_BF16, MAXU>), dim3(grid), dim3(g16::THREADS),
                       g16::Lay<MAXU>::BYTES, st, a);
    return hipGetLastError();
}

// One unit per workgroup while the units fit one round of the CUs, else up to four each (two
// in flight at a time).
template <int FMT, bool OUT_BF16>
static hipError_t launch_fmt(const GemmArgs& a, hipStream_t st)
{
    const uint32_t U = (uint32_t)((a.n + 15) / 16);
    const bool one = U <= g16::GRID_CAP;
    const uint32_t G = one ? U : (U + 3) / 4 > g16::GRID_CAP ? (U + 3) / 4 : g16::GRID_CAP;
    switch (a.block) {
#define MXB(B) case B: return one ? launch_one<B, FMT, OUT_BF16, 1>(a, G, st) : launch_one<B, FMT, OUT_BF16, 4>(a, G, st);
        MXB(32) MXB(64) MXB(128) MXB(256)
#undef MXB
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv16(const GemmArgs& a, hipStream_t st)
{
    if (!gemv16_applies(a)) return hipErrorInvalidValue;
#define MXF(F) if (a.fmt == F) return a.y_bf16 ? launch_fmt<F, true>(a, st) : launch_fmt<F, false>(a, st);
    MXF(FMT_E4M3) MXF(FMT_UE5M3) MXF(FMT_E8M0)
#undef MXF
    return hipErrorInvalidValue;
}

}  // namespace mxk
