// mx_gemm_a4.hip -- W4A4 GEMM on gfx950's block-scaled FP4 matrix cores:
// Y[m][n] = g * sum_k e(xq[m][k]) 2^(sx-127) * e(wq[n][k]) 2^(sw-127)
// (gtnt.cn/news/16247 "为什么我们需要4-bit浮点量化", section 3.1: dequantize then matmul --
// here the matrix cores apply the E8M0 block scales themselves; hotelren.com/news/2192771
// article "量化技术演进与微缩量化原理", section 6 item 1: FP4 activations with block scales).
//
// Tiling: a workgroup of 8 waves (two per SIMD, so that one wave's matrix work covers the
// other's waits) computes a 256 x 256 output tile; each wave a 128 x 64 sub-tile of 4 x 2
// v_mfma_scale_f32_32x32x64_f8f6f4 results (FP4 operands, fp32 accumulators).  The k loop
// advances 256 elements per stage; each stage's operand tiles (256 rows x 128 code bytes for
// X and for W, plus 8 E8M0 bytes per row) travel HBM -> LDS with buffer_load ... lds (no
// register round trip; rows or k beyond the tensor read as zero), double-buffered.  A stage
// row is one whole 128-byte cache line, which halves the number of L2 requests against
// 64-byte row pieces.  In LDS, the eight 16-byte chunks of each row are permuted by XOR with
// (row / 2) % 8 so that the fragment reads (16 rows x 16 bytes per group of lanes) hit
// distinct banks.  In the row-major layout a lane's 16 code bytes (32 consecutive k of one
// row) and its scale byte are exactly one MFMA operand slice and the scale that goes with it.
// Workgroups are mapped so that the m-tiles sharing a weight tile run on the same XCD.
#include "mx_device.h"
#include "mx_internal.h"

namespace mxk {

namespace a4 {

constexpr int BM = 256, BK = 256, STAGES = 2;
constexpr int WAVES = 8, THREADS = 64 * WAVES;
constexpr int MI = 4;                              // per wave: 4 x NJ tiles of 32 x 32 (128 m x 32 NJ n)
constexpr int ROWB = BK / 2;                       // code bytes per row per stage (128)
constexpr int SROW = BK / 32;                      // scale bytes per row per stage (8)
constexpr int CODE_BYTES = BM * ROWB;              // 32 KB of activation codes per stage
constexpr int SCALE_BYTES = BM * SROW;             // 2 KB of activation scales per stage

// Weight-side sizes for a tile 128 NJ wide: NJ = 2 is the full 256 x 256 tile, NJ = 1 the
// 256 x 128 half tile that runs the last, partial round of tiles.
template <int NJ>
struct Cfg {
    static constexpr int BN = 128 * NJ;
    static constexpr int WCODE = BN * ROWB;        // weight codes per stage
    static constexpr int WSCALE = BN * SROW;       // weight scales per stage
    static constexpr int SCALE_OFF = CODE_BYTES + WCODE;
    static constexpr int DUMMY = NJ == 1 ? 256 : 0;  // sink of the idle waves' scale loads
    static constexpr int STAGE_BYTES = SCALE_OFF + SCALE_BYTES + WSCALE + DUMMY;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;  // 139264 (NJ 2) or 104960 (NJ 1)
    static constexpr int LOADS_PER_STAGE = 4 + 2 * NJ + 2;  // codes X, codes W, two scale loads
};
constexpr int BN = Cfg<2>::BN;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) { return chunk ^ ((row >> 1) & 7u); }

// Issue this wave's share of one stage's loads into the LDS stage buffer at `st`.
// Codes: each load covers 8 rows x 128 bytes (lane: row lane/8, LDS chunk lane%8).
// Scales: LDS dword p (of 512 per operand) holds dword p%2 (k 128 (p%2) .. +127 of the
// stage) of row 128 (p / 256) + 32 ((p / 2) % 4) + (p / 8) % 32, so that the dwords a lane
// needs (rows i*32 + r of a 128-row half) are contiguous.  That is the order of one (row
// tile, stage) block of the tiled scale layout, so tiled scales arrive with one contiguous
// 256-byte load per wave and operand; row-major scales take one dword per lane from 32 rows
// per load.  The stage index s is also the block index in the tiled layout.
// A half tile (NJ = 1) loads 128 weight rows: two code loads per wave, and its 1 KB of weight
// scales (the half `whalf` of each tiled 2 KB block) by waves 0..3; waves 4..7 issue their
// scale load into a sink region, so that every wave counts the same loads per stage.
template <int NJ, bool W_TILED>
__device__ __forceinline__ void issue_stage(uint8_t* st, int wave, int lane, uint32_t s,
                                            rsrc_t ac, rsrc_t bc, rsrc_t as, rsrc_t bs, uint32_t K,
                                            uint32_t whalf)
{
    using C = Cfg<NJ>;
    const uint32_t rowb = K / 2, srow = K / 32, k0 = s * BK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t grp = (uint32_t)(wave * 4 + q);           // 8-row group, 0..31
        const uint32_t row = grp * 8 + (lane >> 3);
        const uint32_t c = swz(row, lane & 7);                   // global chunk for this LDS slot
        const uint32_t kk = k0 + 32 * c;
        const uint32_t off = kk < K ? row * rowb + kk / 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ac, (lds_void*)(st + grp * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 2 * NJ; ++q) {
        const uint32_t grp = (uint32_t)(wave * 2 * NJ + q);      // 8-row group, 0..16 NJ - 1
        const uint32_t row = grp * 8 + (lane >> 3);
        const uint32_t c = swz(row, lane & 7);
        const uint32_t kk = k0 + 32 * c;
        const uint32_t off = kk < K ? row * rowb + kk / 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(bc, (lds_void*)(st + CODE_BYTES + grp * 1024), 16, off, 0, 0, 0);
    }
    const uint32_t p = (uint32_t)wave * 64 + lane;
    const uint32_t toff = s * 2048u + 4 * p;                     // stages past the end are out of range
    // weight scales: dword pw of this tile's (half) block; idle waves (NJ = 1) use the sink
    const bool wact = NJ == 2 || wave < 4;
    const uint32_t pw = wact ? p : (uint32_t)lane;
    uint32_t soff = s * 2048u + 1024u * whalf + 4 * pw;
    if constexpr (!W_TILED) {
        const uint32_t row = (pw >> 8) * 128 + ((pw >> 1) & 3) * 32 + ((pw >> 3) & 31);
        const uint32_t kk = k0 + 128 * (pw & 1);
        // beyond k: set the top bit (out of every range) arithmetically rather than by a
        // select, which the compiler would otherwise turn into a branch around the load
        const uint32_t beyond = (uint32_t)((int32_t)(K - 1 - kk) >> 31);
        soff = (row * srow + kk / 32) | (beyond & kOOB);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(as, (lds_void*)(st + C::SCALE_OFF + wave * 256), 4, toff, 0, 0, 0);
    uint8_t* wdst = wact ? st + C::SCALE_OFF + SCALE_BYTES + wave * 256 : st + C::SCALE_OFF + SCALE_BYTES + C::WSCALE;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(bs, (lds_void*)wdst, 4, soff, 0, 0, 0);
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

// s_waitcnt lgkmcnt(0) with the other counters left alone: this wave's LDS reads are done.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Scale dwords of a lane: A rows i*32 + r (i = 0..3) as a[0] = {i0 dword 0, i0 dword 1,
// i1 dword 0, i1 dword 1}, a[1] the same for i = 2, 3; B rows jn*32 + r (jn = 0, 1) as b.
struct Scales { u32x4 a[2]; u32x4 b; };  // b: for NJ = 1 only the first two dwords are used

__device__ __forceinline__ int pick_byte(const u32x4 v, int odd, int j, uint32_t h)
{
    const int d = j >> 1;                                    // k-steps 0, 1 -> dword 0; 2, 3 -> 1
    const uint32_t w = odd ? (d ? v.w : v.z) : (d ? v.y : v.x);
    return (int)((w >> (8 * ((2 * j + h) & 3))) & 0xFFu);
}

// One k-step (64 k) of this wave's 4 x 2 block of 32 x 32 MFMA tiles.
// The weight fragment is the MFMA's A operand and the activation fragment its B operand, so
// each tile is computed transposed (rows n, columns m): a lane then holds four consecutive n
// of one output row per group, which the epilogue stages in LDS as one 8- or 16-byte write.
template <int J, int NJ>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[MI][NJ], const u32x4 (&fa)[MI], const u32x4 (&fb)[NJ],
                                          const Scales& sc, uint32_t h)
{
    int asx[MI], bsx[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) asx[i] = pick_byte(sc.a[i >> 1], i & 1, J, h);
#pragma unroll
    for (int jn = 0; jn < NJ; ++jn) bsx[jn] = pick_byte(sc.b, jn, J, h);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jn = 0; jn < NJ; ++jn) {
            // FP4 operands occupy the low four registers of the 8-register operand; the upper
            // four are not read, so they are left undefined rather than zeroed
            const i32x8 av = __builtin_shufflevector((i32x4)fa[i], (i32x4)fa[i], 0, 1, 2, 3, -1, -1, -1, -1);
            const i32x8 bv = __builtin_shufflevector((i32x4)fb[jn], (i32x4)fb[jn], 0, 1, 2, 3, -1, -1, -1, -1);
            acc[i][jn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][jn], 4, 4, 0, bsx[jn], 0, asx[i]);
        }
}

// Fragment reads of k-step J from a stage buffer: rows 32 further are 4096 bytes apart and
// share the chunk permutation, so one base offset per operand serves all of them.
template <int J, int NJ>
__device__ __forceinline__ void read_frags(const uint8_t* st, uint32_t baseA, uint32_t baseB, uint32_t perm,
                                           u32x4 (&fa)[MI], u32x4 (&fb)[NJ])
{
    const uint32_t chunk = 16 * ((2 * J) ^ perm);
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[i] = *reinterpret_cast<const u32x4*>(st + baseA + chunk + i * 32 * ROWB);
#pragma unroll
    for (int jn = 0; jn < NJ; ++jn) fb[jn] = *reinterpret_cast<const u32x4*>(st + CODE_BYTES + baseB + chunk + jn * 32 * ROWB);
}

template <int NJ>
__device__ __forceinline__ void read_scales(const uint8_t* st, uint32_t offSA, uint32_t offSB, Scales& sc)
{
    sc.a[0] = *reinterpret_cast<const u32x4*>(st + offSA);
    sc.a[1] = *reinterpret_cast<const u32x4*>(st + offSA + 16);
    if constexpr (NJ == 2) {
        sc.b = *reinterpret_cast<const u32x4*>(st + offSB);
    } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(st + offSB);
        sc.b = u32x4{v.x, v.y, 0u, 0u};
    }
}

// scheduling: within a k-step, one MFMA, then the fragment reads for the next k-step, then
// the remaining MFMAs, so that the reads' latency hides behind matrix work
#define A4_SCHED_STEP(ID)                                          \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);            \
    __builtin_amdgcn_sched_group_barrier(0x100, MI + NJ, ID);      \
    __builtin_amdgcn_sched_group_barrier(0x008, MI * NJ - 1, ID)

template <bool OUT_BF16, bool W_TILED, int NJ>
__device__ __forceinline__ void gemm_a4_tile(const GemmArgs& a, uint32_t tile_base, uint32_t bid)
{
    using C = Cfg<NJ>;
    constexpr int BN = C::BN;
    constexpr int STAGE_BYTES = C::STAGE_BYTES;
    constexpr int LOADS_PER_STAGE = C::LOADS_PER_STAGE;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // the wave index is uniform across the wave; saying so keeps LDS-DMA destinations scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const uint32_t K = (uint32_t)a.k;

    // tile mapping over full 256 x 256 tiles: with the n-tile count a multiple of 8, XCD x
    // (= tile % 8) takes n-tiles x, x+8, ... and, for each, every m-tile in turn.  The half-tile
    // part (NJ = 1) covers tiles tile_base.. with two workgroups each (bid: the workgroup's index
    // within its part).
    const uint32_t MT = (uint32_t)((a.m + BM - 1) / BM), NT = (uint32_t)((a.n + 255) / 256);
    const uint32_t tile = tile_base + (NJ == 2 ? bid : bid >> 1);
    const uint32_t whalf = NJ == 2 ? 0u : (bid & 1u);
    uint32_t mt, nt;
    if ((NT & 7) == 0) {
        const uint32_t x = tile & 7, local = tile >> 3;
        mt = local % MT;
        nt = (local / MT) * 8 + x;
    } else {
        mt = tile % MT;
        nt = tile / MT;
    }
    const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * 256 + 128 * whalf;
    // the second half of a last n-tile with at most 128 columns holds no column at all: the
    // whole workgroup leaves (uniformly) before it computes any buffer range
    if (n0 >= a.n) return;
    const uint32_t mrows = (uint32_t)(a.m - m0 < BM ? a.m - m0 : BM);
    const uint32_t nrows = (uint32_t)(a.n - n0 < BN ? a.n - n0 : BN);
    const rsrc_t ac = make_rsrc(a.xq_codes + m0 * (a.k / 2), mrows * (K / 2));
    const rsrc_t bc = make_rsrc(a.wc + n0 * (a.k / 2), nrows * (K / 2));
    // activation scales are tiled; weight scales tiled or row-major
    const uint32_t KS = (K + BK - 1) / BK;
    const rsrc_t as = make_rsrc(a.xq_scales + (int64_t)mt * KS * 2048, KS * 2048);
    const rsrc_t bs = W_TILED ? make_rsrc(a.ws + (int64_t)nt * KS * 2048, KS * 2048)
                              : make_rsrc(a.ws + n0 * (a.k / 32), nrows * (K / 32));

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Pipeline: one stage (four k-steps) per iteration; the fragments of a k-step are read
    // from LDS while the MFMAs of the previous k-step run.  Before the last k-step of a stage,
    // once this stage's reads have completed and the next stage has landed, one barrier both
    // publishes the next stage and frees the current buffer, which then receives the stage
    // after next.  Stages past the end of k load as zeros (their offsets are out of range),
    // so every iteration has the same shape.
    const int S = (int)((K + BK - 1) / BK);
    issue_stage<NJ, W_TILED>(lds, wave, lane, 0, ac, bc, as, bs, K, whalf);
    issue_stage<NJ, W_TILED>(lds + STAGE_BYTES, wave, lane, 1, ac, bc, as, bs, K, whalf);

    const uint32_t r32 = lane & 31, h = lane >> 5;
    const uint32_t perm = h ^ ((r32 >> 1) & 7u);              // chunk (2j + h) -> slot (2j) ^ perm
    const uint32_t baseA = (wm * 128 + r32) * ROWB;
    const uint32_t baseB = (wn * 32 * NJ + r32) * ROWB;
    const uint32_t offSA = C::SCALE_OFF + (wm * 256 + r32 * 8) * 4;
    // weight scale dwords of rows wn*32NJ + jn*32 + r: NJ = 2 four from p = 256 (wn/2) + 8 r +
    // 4 (wn%2); NJ = 1 two from p = 8 r + 2 wn
    const uint32_t offSB = C::SCALE_OFF + SCALE_BYTES +
                           (NJ == 2 ? ((wn >> 1) * 256 + r32 * 8 + 4 * (wn & 1)) : (r32 * 8 + 2 * wn)) * 4;

    u32x4 f0a[MI], f0b[NJ], f1a[MI], f1b[NJ];
    Scales sc;
    wait_vmcnt<LOADS_PER_STAGE>();
    barrier_only();
    read_frags<0, NJ>(lds, baseA, baseB, perm, f0a, f0b);
    read_scales<NJ>(lds, offSA, offSB, sc);

    uint32_t cur = 0;  // byte offset of stage s's buffer
    for (int s = 0; s < S; ++s) {
        const uint32_t nxt = cur ^ (uint32_t)STAGE_BYTES;
        read_frags<1, NJ>(lds + cur, baseA, baseB, perm, f1a, f1b);
        mfma_step<0, NJ>(acc, f0a, f0b, sc, h);
        A4_SCHED_STEP(0);
        __builtin_amdgcn_sched_barrier(0);
        read_frags<2, NJ>(lds + cur, baseA, baseB, perm, f0a, f0b);
        mfma_step<1, NJ>(acc, f1a, f1b, sc, h);
        A4_SCHED_STEP(1);
        __builtin_amdgcn_sched_barrier(0);
        read_frags<3, NJ>(lds + cur, baseA, baseB, perm, f1a, f1b);
        mfma_step<2, NJ>(acc, f0a, f0b, sc, h);
        A4_SCHED_STEP(2);
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkm0();
        wait_vmcnt<0>();
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
        issue_stage<NJ, W_TILED>(lds + cur, wave, lane, (uint32_t)(s + STAGES), ac, bc, as, bs, K, whalf);
        Scales sc_n;
        read_frags<0, NJ>(lds + nxt, baseA, baseB, perm, f0a, f0b);
        read_scales<NJ>(lds + nxt, offSA, offSB, sc_n);
        mfma_step<3, NJ>(acc, f1a, f1b, sc, h);
        // next stage's first fragments and scales first, then the stage loads spread between
        // MFMAs so that the matrix pipe stays busy while they are issued
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
        __builtin_amdgcn_sched_group_barrier(0x100, MI + NJ + 3, 3);
        constexpr int SPREAD = LOADS_PER_STAGE / 2 < MI * NJ - 1 ? LOADS_PER_STAGE / 2 : MI * NJ - 1;
#pragma unroll
        for (int g = 0; g < SPREAD; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 3);
        }
        if constexpr (MI * NJ - 1 - SPREAD > 0) __builtin_amdgcn_sched_group_barrier(0x008, MI * NJ - 1 - SPREAD, 3);
        // keep the next stage's reads in this iteration (not sunk into the next one)
        asm volatile("" ::: "memory");
        sc = sc_n;
        cur = nxt;
    }
    wait_vmcnt<0>();

    // Epilogue.  Transposed 32x32 result layout: for tile (i, jn) a lane holds output row
    // m = i*32 + lane%32 and, for group q = e/4, columns n = jn*32 + 8q + 4*(lane/32) + e%4.
    // Rows of a wave's 128 x 64 block are staged through LDS (each wave in a region of its
    // own, 64 rows a pass, rows padded by 16 bytes against bank conflicts so that every
    // read-back stays 16-byte aligned) and written back as whole 16-byte chunks, 128
    // or 256 contiguous bytes per output row.  Stores go through a buffer descriptor;
    // out-of-range chunks get an out-of-range offset and are dropped.
    constexpr uint32_t ESZ = OUT_BF16 ? 2 : 4;
    const rsrc_t yr = make_rsrc(static_cast<uint8_t*>(a.y) + (m0 * a.ldy + n0) * ESZ, 0x7FFFFFFFu);
    const uint32_t ldy = (uint32_t)a.ldy;
    const uint32_t mlim = mrows, nlim = nrows;
    constexpr uint32_t CE = 16 / ESZ;  // elements per 16-byte chunk
    // chunk stores need 16-byte aligned rows and chunks wholly in or out of range
    const bool vec = (ldy % CE) == 0 && (nlim % CE) == 0;
    if (vec) {
        constexpr int PASSES = 2;                             // 64 rows per pass
        constexpr int IPP = MI / PASSES;                      // 32-row blocks per pass
        constexpr uint32_t RB = 32 * NJ * ESZ;                // bytes of a wave row (32 NJ columns)
        constexpr uint32_t PITCH = RB + 16;                   // 16-byte aligned rows for the read-back
        constexpr uint32_t CPR = RB / 16;                     // chunks per row (8 or 16)
        constexpr uint32_t RPI = 64 / CPR;                    // rows per store instruction
        constexpr uint32_t PASS_ROWS = 32 * IPP;
        static_assert(WAVES * PASS_ROWS * PITCH <= (uint32_t)C::LDS_BYTES, "epilogue staging exceeds LDS");
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
            // read back row-contiguous chunks (LDS accesses of one wave complete in order)
#pragma unroll
            for (uint32_t t = 0; t < PASS_ROWS / RPI; ++t) {
                const uint32_t row = t * RPI + lane / CPR, chunk = lane % CPR;
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * PITCH + chunk * 16);
                const uint32_t mm = wm * 128 + pass * PASS_ROWS + row, nn = wn * 32 * NJ + chunk * CE;
                const uint32_t off = (mm < mlim && nn < nlim) ? (mm * ldy + nn) * ESZ : kOOB;
                bstore128_nt(yr, off, v);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const uint32_t mm = wm * 128 + i * 32 + r32;
            const bool mok = mm < mlim;
#pragma unroll
            for (int jn = 0; jn < NJ; ++jn)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t nn = wn * 32 * NJ + jn * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                    const uint32_t off = (mok && nn < nlim) ? (mm * ldy + nn) * ESZ : kOOB;
                    const float v = acc[i][jn][e] * a.g;
                    if constexpr (OUT_BF16) bstore16(yr, off, __builtin_bit_cast(uint16_t, (__bf16)v));
                    else bstore32(yr, off, __builtin_bit_cast(uint32_t, v));
                }
        }
    }
}

// Full tiles 0 .. full - 1 (workgroups 0 .. full - 1), then the remaining tiles as half tiles,
// two workgroups each, in one launch: half tiles start on CUs as the last full tiles finish.
template <bool OUT_BF16, bool W_TILED>
__global__ __launch_bounds__(THREADS) void gemm_a4_merged_kernel(const GemmArgs a, uint32_t full)
{
    if (blockIdx.x < full) gemm_a4_tile<OUT_BF16, W_TILED, 2>(a, 0u, blockIdx.x);
    else gemm_a4_tile<OUT_BF16, W_TILED, 1>(a, full, blockIdx.x - full);
}

}  // namespace a4

template <bool OUT_BF16, bool W_TILED>
static hipError_t launch_merged(const GemmArgs& a, uint32_t full, unsigned groups, hipStream_t st)
{
    // the LDS ring exceeds the default 64 KB dynamic limit
    static LdsLimit lim;
    if (const hipError_t e = lim.ensure((const void*)a4::gemm_a4_merged_kernel<OUT_BF16, W_TILED>,
                                        a4::Cfg<2>::LDS_BYTES, st); e != hipSuccess)
        return e;
    hipLaunchKernelGGL((a4::gemm_a4_merged_kernel<OUT_BF16, W_TILED>), dim3(groups), dim3(a4::THREADS),
                       a4::Cfg<2>::LDS_BYTES, st, a, full);
    return hipGetLastError();
}

// Full 256 x 256 tiles run in whole rounds of kCUs workgroups; when the last round would be at
// most half full, its tiles run instead as twice as many 256 x 128 half tiles, which fill it,
// in the same launch (as two launches, the half tiles waited for the slowest full tile).
constexpr unsigned kCUs = 256;

template <bool OUT_BF16, bool W_TILED>
static hipError_t launch_tiled(const GemmArgs& a, hipStream_t st)
{
    const unsigned tiles = (unsigned)(((a.m + a4::BM - 1) / a4::BM) * ((a.n + 255) / 256));
    const unsigned rem = tiles % kCUs;
    const unsigned full = (rem != 0 && rem <= kCUs / 2) ? tiles - rem : tiles;
    return launch_merged<OUT_BF16, W_TILED>(a, full, full + 2 * (tiles - full), st);
}

bool a4_uses_mfma(const GemmArgs& a)
{
    // k in whole 128-element halves of a stage, 32-bit offsets within an output tile
    const int64_t tile_span = ((int64_t)(a4::BM - 1) * a.ldy + a4::BN) * (a.y_bf16 ? 2 : 4);
    return a.k % 128 == 0 && tile_span < 0x7FFFFFFF;
}

hipError_t launch_gemm_a4_mfma(const GemmArgs& a, hipStream_t st)
{
    if (!a4_uses_mfma(a)) return hipErrorInvalidValue;
    if (a.y_bf16) return a.ws_tiled ? launch_tiled<true, true>(a, st) : launch_tiled<true, false>(a, st);
    return a.ws_tiled ? launch_tiled<false, true>(a, st) : launch_tiled<false, false>(a, st);
}

}  // namespace mxk
