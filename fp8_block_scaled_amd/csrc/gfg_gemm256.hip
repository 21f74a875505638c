// Grouped FP8 (E4M3) block-scaled GEMM on 256 x 256 output tiles for gfx950
// (MI355X): the launches with enough 256 x 256 tiles to keep every CU busy.
//
// Computes the same operation as the kernels of gfg_gemm.hip, the grouped GEMM
// of the first reference page, "Grouped and Batched GEMM kernels with
// blockscaling matching DeepGEMM API" (sections "Summary" and "DeepGEMM
// conformance details"): E4M3 operands, one E8M0 scale per (1,128) block of A
// (stored transposed [K/128][M]) and per (128,128) block of B, contiguous
// (grouped_layout) and masked (masked_m) layouts, bf16 / f16 output.
//
// Why a second tile shape: per 128-K step a CU moves A and B rows through the
// global -> LDS path and the LDS port.  On the 128 x 256 tile that is 48 KB
// for 8.4 MFLOP, and the path, not the matrix cores, sets the step time; the
// 256 x 256 tile moves 64 KB for 16.8 MFLOP, a third less per FLOP.
//
// Design:
//  * 4 wave64s, one per SIMD, each owning a 128 x 128 quarter of the tile
//    (rows 128*(w >> 1) .., columns 128*(w & 1) ..): 256 accumulator registers
//    (64 16x16 blocks) and 192 fragment registers per wave.  Alone on its SIMD,
//    a wave's instruction order is the schedule, so every group of
//    instructions is pinned in place;
//  * v_mfma_scale_f32_16x16x128_f8f6f4 with the E8M0 bytes as hardware scale
//    operands: one instruction per 16 x 16 block and 128-K step, 64 per wave
//    and step;
//  * two 64 KB LDS stages filled by direct-to-LDS loads, A and B rows laid
//    out alike: LDS row R holds tile row R ^ ((R >> 2) & 1), its 16-byte
//    chunks XOR-swizzled by (R >> 2) & 7, so that a lane's four fragment rows
//    (4 apart) share one A-scale dword and the fragment reads and DMA writes
//    are free of bank conflicts;
//  * two barriers per step: the first frees the B rows and half of the A rows
//    of the stage just consumed, whose refill then starts under the first half
//    of the step's MFMAs; the second (after stage k+1 has landed) frees the
//    other A rows.  A wave's load instructions hold up its own MFMA issue, so
//    spreading the step's 16 DMAs over both halves, instead of issuing them
//    all in the second, cut the kernel time by 3 to 9% on the measured
//    workloads;
//  * a persistent grid over (M tile, N tile) work items in the shared
//    XCD-range / grouped-M order; the refills of a tile's last two steps load
//    the next tile's first two stages, and the tile's output stores are
//    issued after them, so neither the next tile's first loads nor the output
//    write stand between two tiles' MFMAs;
//  * the contiguous layout's M tiles follow each expert's run of 128-row
//    tiles in pairs (a run of odd length ends in a 128-row tile);
//  * output through buffer stores of whole 128-byte lines: a DPP exchange
//    between lane pairs turns the MFMA's (row, 4 x 4 columns) per lane into
//    eight complete lines per store instruction, sent non-temporal;
//  * a row that must stay untouched gets an offset past the store window,
//    which the hardware drops, so every wave issues the same number of
//    stores and the vector-memory waits stay exact.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gfg.h"
#include "gfg_device.h"
#include "gfg_internal.h"

namespace gfg {
namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int NTHREADS = 256, WAVES = 4;
constexpr int A_BYTES = BM * BK;                 // 32 KB of A per stage
constexpr int STAGE = A_BYTES + BN * BK;         // + 32 KB of B
constexpr int A_DMA = A_BYTES / 1024 / WAVES;    // 1 KB DMA instructions per wave and stage
constexpr int B_DMA = BN * BK / 1024 / WAVES;
constexpr int CAND_MAX = 4096;                   // candidate M tiles (128-row contiguous, 256-row masked)
constexpr int CPT = CAND_MAX / NTHREADS;         // candidates per thread in the list build

// Vector-memory operations a wave issues, in order: per stage A_DMA + B_DMA
// DMAs (FIRST_HALF_DMA of them before the step's mid barrier) then SL A-scale
// dword loads; per tile boundary, for the contiguous layout, two loads of the
// next tile's grouped_layout rows, then 32 output stores.
constexpr int DMA_OPS = A_DMA + B_DMA;
constexpr int FIRST_HALF_DMA = 12;               // a step's DMAs issued before its mid-step barrier
constexpr int SL = 2;                            // A-scale dwords per stage (two 64-row halves)
template <bool MASKED>
struct Epi {
    static constexpr int OPS = 32 + (MASKED ? 0 : 2);
};

// One work tile: contiguous: first 128-row candidate | (128 rows only) << 12 | expert << 16;
// masked: candidate (group * tiles per group + 256-row index) | valid rows << 12.
struct TileInfo {
    int g;
    int row0;   // first row of the tile inside its region (the group, for the masked layout)
    int lim;    // rows of the tile that may be read and written
    int n0;     // first output column
};

template <bool MASKED>
__device__ __forceinline__ TileInfo tile_info(const Params& p, uint32_t e, int nt) {
    TileInfo t;
    const int c = int(e & 0xFFFu);
    if (MASKED) {
        t.g = c / p.mt_per_group;
        t.row0 = (c - t.g * p.mt_per_group) * BM;
        t.lim = int(e >> 12);
    } else {
        t.g = int(e >> 16);
        t.row0 = c * 128;
        t.lim = min(((e >> 12) & 1u) ? 128 : BM, int(p.rows) - t.row0);
    }
    t.n0 = nt * BN;
    t.g = __builtin_amdgcn_readfirstlane(t.g);
    t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
    t.lim = __builtin_amdgcn_readfirstlane(t.lim);
    t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
    return t;
}

// What the refills of one tile read, as buffer resources: its A rows (rows
// past the tile's readable ones come back as zeros, so no clamp is needed),
// its B rows, its A-scale rows and this wave's B-scale row.
struct Refill {
    __amdgpu_buffer_rsrc_t a_rsrc;
    __amdgpu_buffer_rsrc_t b_rsrc;
    __amdgpu_buffer_rsrc_t sa_rsrc;   // scale_a from the tile's first row of K-block 0 to the region's end
    const uint8_t* sb_row;            // scale_b row (all K-blocks) of this wave's 128-column block
};

template <bool MASKED>
__device__ __forceinline__ Refill make_refill(const Params& p, const TileInfo& t, int wn) {
    Refill r;
    const int KB = p.K / BK;
    const int64_t region = MASKED ? int64_t(t.g) * p.rows : 0;    // first row of the region
    r.a_rsrc = make_rsrc(p.a + (region + t.row0) * p.K, uint32_t(t.lim) * uint32_t(p.K));
    r.b_rsrc = make_rsrc(p.b + (int64_t(t.g) * p.N + t.n0) * p.K, uint32_t(BN) * uint32_t(p.K));
    r.sa_rsrc = make_rsrc(p.a_scale + region * KB + t.row0, uint32_t(int64_t(KB) * p.rows - t.row0));
    r.sb_row = uniform_ptr(p.b_scale + (int64_t(t.g) * (p.N / 128) + t.n0 / 128 + wn) * KB);
    return r;
}

// Block-wide exclusive scan (sum, or max with identity -1) over the NTHREADS threads.
template <bool MAX>
__device__ __forceinline__ int block_exclusive_scan(int v, GFG_LDS int* tmp, int lane, int wave, int* total) {
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x = MAX ? max(x, y) : x + y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    int pre = MAX ? -1 : 0, all = MAX ? -1 : 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        const int tw = tmp[w];
        if (w < wave) pre = MAX ? max(pre, tw) : pre + tw;
        all = MAX ? max(all, tw) : all + tw;
    }
    int ex = __shfl_up(x, 1, 64);
    if (lane == 0) ex = MAX ? -1 : 0;
    __syncthreads();   // tmp is reused by the next scan
    *total = all;
    return MAX ? max(pre, ex) : pre + ex;
}

// LDS layout of a stage: 128-byte rows, A (256 rows) then B (256 rows), both
// as the 128-row kernel's A tile: LDS row R holds tile row a_row(R) =
// R ^ ((R >> 2) & 1) and its physical 16-byte chunk c the logical chunk
// c ^ ((R >> 2) & 7).  A 16x16x128 fragment takes rows 4 apart (row
// 64 h + 4 l16 + f of the wave's 128), so a lane's four rows share one
// A-scale dword, and the row-parity exchange keeps the fragment reads free of
// bank conflicts.  DMA chunk j of wave w fills LDS rows 8 (4 j + w) .. +7;
// with four waves chunk j is chunk 0 moved by 32 j rows (a_row and the chunk
// key do not depend on j).
__device__ __forceinline__ int a_row(int p) { return p ^ ((p >> 2) & 1); }   // an involution
__device__ __forceinline__ int swz_a(int p, int c) { return p * BK + ((c ^ ((p >> 2) & 7)) << 4); }

struct LaneOffsets {
    uint32_t a0;   // A chunk 0; chunk j adds 32 j rows
    uint32_t b0;   // B chunk 0; chunk j adds 32 j rows
    uint32_t K;    // row stride (uniform)
};

// DMA chunk c (0..15) of this wave for stage kb: chunks 0..7 are A's, 8..15 B's.
__device__ __forceinline__ void dma_chunk(const Refill& r, LaneOffsets o, GFG_LDS uint8_t* dst, int kb, int wave,
                                          int c) {
    const uint32_t ks = uint32_t(kb) * BK;
    asm volatile("" : "+v"(o.a0));   // re-added per chunk, not eight offsets held live
    if (c < A_DMA) {
        const int j = c;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r.a_rsrc, (GFG_LDS void*)(dst + (j * WAVES + wave) * 1024), 16,
                                                 o.a0 + uint32_t(32 * j) * o.K, ks, 0, 0);
    } else {
        // every B row of a tile exists, so the chunk's row offset may go into
        // the (unchecked) scalar offset
        const int j = c - A_DMA;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r.b_rsrc, (GFG_LDS void*)(dst + A_BYTES + (j * WAVES + wave) * 1024),
                                                 16, o.b0, ks + uint32_t(32 * j) * o.K, 0, 0);
    }
}

// DMA chunk j (0..7) of this wave's B rows for stage kb, into the B region
// `dst_b` of a stage buffer.
__device__ __forceinline__ void dma_chunk_b(const Refill& r, LaneOffsets o, GFG_LDS uint8_t* dst_b, int kb, int wave,
                                            int j) {
    const uint32_t ks = uint32_t(kb) * BK;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.b_rsrc, (GFG_LDS void*)(dst_b + (j * WAVES + wave) * 1024), 16, o.b0,
                                             ks + uint32_t(32 * j) * o.K, 0, 0);
}

__device__ __forceinline__ void dma_stage(const Refill& r, const LaneOffsets& o, GFG_LDS uint8_t* dst, int kb,
                                          int wave) {
#pragma unroll
    for (int c = 0; c < DMA_OPS; ++c) dma_chunk(r, o, dst, kb, wave, c);
}

// The lane's two A-scale dwords (rows 4 l16 .. +3 of each 64-row half of its
// wave's rows) and the wave's B-scale word.  (The K-block stride goes into
// the vector offset, which the hardware range check covers.)
__device__ __forceinline__ void load_scales(const Refill& r, int kb, int rows, int sa_off, int (&sa)[2], int& sbw,
                                            int& sbs) {
    const uint32_t kofs = uint32_t(kb) * uint32_t(rows);
    sa[0] = int(__builtin_amdgcn_raw_buffer_load_b32(r.sa_rsrc, uint32_t(sa_off) + kofs, 0, 0));
    sa[1] = int(__builtin_amdgcn_raw_buffer_load_b32(r.sa_rsrc, uint32_t(sa_off + 64) + kofs, 0, 0));
    sbw = load_scale_word(r.sb_row, kb);
    sbs = 8 * int((reinterpret_cast<uintptr_t>(r.sb_row) + uintptr_t(kb)) & 3);
}

// The lane index, read afresh where it is used: values derived from it ahead
// of the tile loop would stay live (and be spilled) through the K loop.
__device__ __forceinline__ int lane_now() {
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    return ln;
}

// The lane's DMA source offset of chunk 0 (A and B alike), from the lane index
// read afresh: computed per step, it is not held through the step's first half.
// Chunk 0 of wave w covers LDS rows R = 8 w + (lane >> 3); lane i writes
// physical chunk i % 8, the logical chunk (i % 8) ^ ((R >> 2) & 7) of tile row
// a_row(R).
__device__ __forceinline__ uint32_t dma_lane_offset(int wave, uint32_t K) {
    const int ln = lane_now();
    const int R = 8 * wave + (ln >> 3);
    return uint32_t(a_row(R)) * K + uint32_t(((ln & 7) ^ ((R >> 2) & 7)) << 4);
}

struct Lane {
    // LDS offsets of this lane's fragment rows for the first 64-row half and
    // fragment f = 0 (row p0 + odd for even f, p0 - odd for odd f, then + f
    // rows); logical chunks lq (lo) and lq + 4 (hi).  The second half adds 64
    // rows.  B offsets include the A region.
    int a_lo_e, a_lo_o, a_hi_e, a_hi_o;
    int b_lo_e, b_lo_o, b_hi_e, b_hi_o;
    LaneOffsets off;     // DMA source offsets
    int wave, wm, wn, sa_off;
};

__device__ __forceinline__ int frag_off(int e, int o, int y) {
    const int f = y & 3;
    return ((f & 1) ? o : e) + f * BK + (y >> 2) * 64 * BK;
}

#define GFG_SB() __builtin_amdgcn_sched_barrier(0)


__device__ __forceinline__ u32x4 lds16(const GFG_LDS uint8_t* __restrict__ src, int a) {
    return *reinterpret_cast<const GFG_LDS u32x4*>(src + a);
}
__device__ __forceinline__ v8i join(u32x4 l, u32x4 h) {
    return __builtin_bit_cast(v8i, __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ v4f mfma(const v8i& b, const v8i& a, const v4f& c, int sb, int y, int sa) {
    switch (y & 3) {   // the A-scale byte (op_sel) must be a constant
        case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, 0, sb, 0, sa);
        case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, 0, sb, 1, sa);
        case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, 0, sb, 2, sa);
        default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, 0, sb, 3, sa);
    }
}

// The row mask of a lane: bit y set when its output row for fragment y may be
// written (inside the tile's rows and, for the contiguous layout, of the
// tile's expert).
template <bool MASKED>
__device__ __forceinline__ int row_mask(const Lane& L, const u32x4 (&lay)[2], int lim, int g) {
    int okm = 0;
#pragma unroll
    for (int y = 0; y < 8; ++y)
        okm |= int(L.sa_off + 64 * (y >> 2) + (y & 3) < lim && (MASKED || int(lay[y >> 2][y & 3]) == g)) << y;
    return okm;
}

// One 128-K step k: stage k in `cur` (its B region also as `cur_b`), stage
// k+1 in `nxt`; 64 MFMAs per wave in row order.  On entry af[0..3] and bc hold
// stage k's A fragments 0..3 and B fragments.
//  * start barrier: every wave has read stage k's B and A 0..3 fragments, so
//    their LDS rows (the B region and DMA chunks 0, 1, 4, 5 of A) are free;
//  * first half (fragment rows 0..3): reads stage k's A fragments 4..7 into
//    their slots over the first 8 MFMAs, then refills the free rows with
//    stage kr, one DMA per two MFMAs (12 DMAs);
//  * mid barrier: stage k+1 has landed and every wave has read stage k's
//    A fragments 4..7;
//  * second half (rows 4..7): reads stage k+1's B fragments into bn and its
//    A fragments 0..3 into slots 0..3, and refills the last four A chunks.
// VMWAIT counts the vector-memory operations issued after stage k+1's last
// DMA: the A-scale loads of its step and this step's first-half DMAs, plus
// the tile-boundary operations in the first step of a tile.  The DMAs of a
// half follow its LDS reads of the same buffer: a read issued after a DMA
// into the same buffer would make the compiler wait for the DMA.
// FIRST: the first step of a tile also folds the tile's layout words into
// the row mask right after its mid barrier, so they are not held through the
// step pair.
template <int PAR, int VMWAIT, bool MASKED = false, bool FIRST = false>
__device__ __forceinline__ void k_step(const Lane& L, int rows, GFG_LDS uint8_t* __restrict__ cur,
                                       GFG_LDS uint8_t* __restrict__ cur_b, GFG_LDS uint8_t* __restrict__ nxt, int kr,
                                       const Refill& rf,
                                       v4f (&acc)[8][8], v8i (&af)[8], v8i (&bc)[8], v8i (&bn)[8],
                                       int (&sa)[2][2], int (&sbw)[2], int (&sbs)[2], GFG_LDS uint8_t* okm = nullptr,
                                       const u32x4* lay = nullptr, int lim = 0, int g = 0) {
    const int sb_k = (sbw[PAR] >> sbs[PAR]) & 0xff;
    const int sa0 = sa[PAR][0], sa1 = sa[PAR][1];
    // ---- start barrier: every wave's reads of stage k's B and A 0..3
    // fragments (issued in the previous step's second half) have completed
    GFG_SB();
    GFG_WAITCNT(63, 0);
    __builtin_amdgcn_s_barrier();
    GFG_SB();
    LaneOffsets o;
    o.a0 = o.b0 = dma_lane_offset(L.wave, L.off.K);
    o.K = L.off.K;
    GFG_SB();
    // ---- first half: rows 0..3
    {
        u32x4 r[8];
#pragma unroll
        for (int m = 0; m < 32; ++m) {
            const int y = m >> 3, x = m & 7;
            acc[y][x] = mfma(bc[x], af[y], acc[y][x], sb_k, y, sa0);
            GFG_SB();
            if (m < 8) {
                const int q = m, yy = 4 + (q >> 1);
                r[q] = lds16(cur, (q & 1) ? frag_off(L.a_hi_e, L.a_hi_o, yy) : frag_off(L.a_lo_e, L.a_lo_o, yy));
                GFG_SB();
            }
            if (m >= 8 && !(m & 1)) {
                const int q = (m - 8) >> 1;   // 0..11: A chunks 0, 1, 4, 5 (fragment rows 0..3), then B's
                if (q < 4)
                    dma_chunk(rf, o, cur, kr, L.wave, (q & 1) + 4 * (q >> 1));
                else
                    dma_chunk_b(rf, o, cur_b, kr, L.wave, q - 4);
                GFG_SB();
            }
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) af[4 + f] = join(r[2 * f], r[2 * f + 1]);
    }
    // ---- mid barrier, then the second half: rows 4..7
    GFG_WAITCNT(VMWAIT, 0);
    __builtin_amdgcn_s_barrier();
    GFG_SB();
    if constexpr (FIRST) {
        const u32x4 lw[2] = {lay[0], lay[1]};
        // parked in LDS until the epilogue: a register held through the K
        // loop would be spilled
        okm[L.wave * 64 + lane_now()] = uint8_t(row_mask<MASKED>(L, lw, lim, g));
        GFG_SB();
    }
    {
        u32x4 r[24];
#pragma unroll
        for (int m = 0; m < 32; ++m) {
            const int y = 4 + (m >> 3), x = m & 7;
            acc[y][x] = mfma(bc[x], af[y], acc[y][x], sb_k, y, sa1);
            GFG_SB();
            if ((m & 7) == 1) dma_chunk(rf, o, cur, kr, L.wave, 2 + ((m >> 3) & 1) + 4 * (m >> 4));   // 2, 3, 6, 7
            if (m < 24) {
                if (m < 16) {   // B fragment m >> 1, chunk m & 1
                    const int xx = m >> 1;
                    r[m] = lds16(nxt, (m & 1) ? frag_off(L.b_hi_e, L.b_hi_o, xx) : frag_off(L.b_lo_e, L.b_lo_o, xx));
                } else {        // A fragment (m - 16) >> 1
                    const int yy = (m - 16) >> 1;
                    r[m] = lds16(nxt, (m & 1) ? frag_off(L.a_hi_e, L.a_hi_o, yy) : frag_off(L.a_lo_e, L.a_lo_o, yy));
                }
            }
            GFG_SB();
        }
#pragma unroll
        for (int f = 0; f < 8; ++f) bn[f] = join(r[2 * f], r[2 * f + 1]);
#pragma unroll
        for (int f = 0; f < 4; ++f) af[f] = join(r[16 + 2 * f], r[17 + 2 * f]);
    }
    // stage kr's scales replace stage k's, whose last MFMAs are issued above
    load_scales(rf, kr, rows, L.sa_off, sa[PAR], sbw[PAR], sbs[PAR]);
    GFG_SB();
}

template <bool MASKED, typename OutT>
__global__ __launch_bounds__(NTHREADS, 1) void grouped_fp8_gemm256_kernel(Params p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t smem1[STAGE];
    __shared__ uint32_t work[CAND_MAX];      // work tiles in M order
    __shared__ uint8_t okm_smem[NTHREADS];   // per lane: the row mask of the tile

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    GFG_LDS uint8_t* const buf0 = (GFG_LDS uint8_t*)smem0;
    GFG_LDS uint8_t* const okm_lds = (GFG_LDS uint8_t*)okm_smem;
    GFG_LDS uint8_t* const buf1 = (GFG_LDS uint8_t*)smem1;

    // ---- 1. work tiles (the list build uses stage buffer 0 before the first DMA)
    GFG_LDS int16_t* const expo = reinterpret_cast<GFG_LDS int16_t*>(buf0);   // [CAND_MAX]
    GFG_LDS int* const tmp = reinterpret_cast<GFG_LDS int*>(buf0 + 2 * CAND_MAX);
    const int c0 = tid * CPT;     // this thread's CPT consecutive candidates
    unsigned wmask = 0;           // bit j: candidate c0 + j starts a work tile
    unsigned hmask = 0;           // contiguous: ... that has only 128 rows (its run ends with it)
    if (MASKED) {
        // candidate g * mt_per_group + j: rows [256 j, 256 j + 256) of group g
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = c0 + j;
            if (c < p.n_cand) {
                const int g = c / p.mt_per_group;
                int mm = p.meta[g];
                mm = mm < 0 ? 0 : (mm > p.rows ? int(p.rows) : mm);
                if (mm - (c - g * p.mt_per_group) * BM > 0) wmask |= 1u << j;
            }
        }
    } else {
        // candidate c: the 128-row tile starting at row 128 c; its expert is
        // that of its first row.  A run is a maximal stretch of candidates of
        // one expert; work tiles start at even offsets inside a run.
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = c0 + j;
            if (c < p.n_cand) {
                const int e = p.meta[int64_t(c) * 128];
                expo[c] = int16_t(e >= 0 && e < p.G ? e : -1);
            }
        }
        __syncthreads();
        int last_start = -1;
        int e_prev = (c0 > 0 && c0 - 1 < p.n_cand) ? int(expo[c0 - 1]) : -1;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = c0 + j;
            if (c < p.n_cand) {
                const int e = expo[c];
                if (e >= 0 && e != e_prev) last_start = c;
                e_prev = e;
            }
        }
        int unused;
        int run_start = block_exclusive_scan<true>(last_start, tmp, lane, wave, &unused);
        e_prev = (c0 > 0 && c0 - 1 < p.n_cand) ? int(expo[c0 - 1]) : -1;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = c0 + j;
            if (c < p.n_cand) {
                const int e = expo[c];
                if (e >= 0 && e != e_prev) run_start = c;
                e_prev = e;
                if (e >= 0 && ((c - run_start) & 1) == 0) {
                    wmask |= 1u << j;
                    if (!(c + 1 < p.n_cand && int(expo[c + 1]) == e)) hmask |= 1u << j;
                }
            }
        }
    }
    int n_work;
    int off = block_exclusive_scan<false>(__popc(wmask), tmp, lane, wave, &n_work);
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        if ((wmask >> j) & 1u) {
            const int c = c0 + j;
            uint32_t e;
            if (MASKED) {
                const int g = c / p.mt_per_group;
                int mm = p.meta[g];
                mm = mm < 0 ? 0 : (mm > p.rows ? int(p.rows) : mm);
                e = uint32_t(c) | (uint32_t(min(mm - (c - g * p.mt_per_group) * BM, BM)) << 12);
            } else {
                e = uint32_t(c) | (((hmask >> j) & 1u) << 12) | (uint32_t(int(expo[c])) << 16);
            }
            work[off++] = e;
        }
    n_work = __builtin_amdgcn_readfirstlane(n_work);
    __syncthreads();   // the list is complete, and stage buffer 0 is free for the DMA

    const int NT = p.N / BN;
    const unsigned T = unsigned(n_work) * unsigned(NT);
    TileOrder order;
    order.init(T, p.num_xcd);
    // uniform: kept in scalar registers (in vector registers they are spilled
    // and reloaded at every tile)
    order.x_start = __builtin_amdgcn_readfirstlane(order.x_start);
    order.x_count = __builtin_amdgcn_readfirstlane(order.x_count);
    order.slot = __builtin_amdgcn_readfirstlane(order.slot);
    order.slots = __builtin_amdgcn_readfirstlane(order.slots);
    const unsigned gm = p.group_m > 0 ? unsigned(p.group_m) : 4u;
    unsigned i = order.slot;
    if (i >= order.x_count) return;

    Lane L;
    L.wave = wave;
    L.wm = wave >> 1;
    L.wn = wave & 1;
    const int l16 = lane & 15, lq = lane >> 4, odd = l16 & 1;
    L.sa_off = L.wm * 128 + 4 * l16;
    {
        const int p0 = L.wm * 128 + 4 * l16, pb = L.wn * 128 + 4 * l16;
        L.a_lo_e = swz_a(p0, lq) + odd * BK;
        L.a_lo_o = swz_a(p0, lq) - odd * BK;
        L.a_hi_e = swz_a(p0, lq + 4) + odd * BK;
        L.a_hi_o = swz_a(p0, lq + 4) - odd * BK;
        L.b_lo_e = A_BYTES + swz_a(pb, lq) + odd * BK;
        L.b_lo_o = A_BYTES + swz_a(pb, lq) - odd * BK;
        L.b_hi_e = A_BYTES + swz_a(pb, lq + 4) + odd * BK;
        L.b_hi_o = A_BYTES + swz_a(pb, lq + 4) - odd * BK;
    }
    // DMA sources: chunk 0 of this wave covers LDS rows R = 8 wave + (lane >> 3);
    // lane i writes physical chunk i % 8, the logical chunk (i % 8) ^ ((R >> 2) & 7)
    // of tile row a_row(R).
    {
        const int R = 8 * wave + (lane >> 3);
        const uint32_t ch = uint32_t(((lane & 7) ^ ((R >> 2) & 7)) << 4);
        L.off.a0 = uint32_t(a_row(R)) * uint32_t(p.K) + ch;
        L.off.b0 = uint32_t(a_row(R)) * uint32_t(p.K) + ch;
        L.off.K = uint32_t(p.K);
    }

    const int KB = p.K / BK;   // even and >= 2 (checked on the host)
    __builtin_assume(KB >= 2);
    int mr, nt;
    order.item(i, gm, unsigned(NT), unsigned(n_work), &mr, &nt);
    TileInfo cur = tile_info<MASKED>(p, work[mr], nt);
    Refill rf = make_refill<MASKED>(p, cur, L.wn);

    v4f acc[8][8];
    v8i af[8], bf0[8], bf1[8];
    int sa[2][2], sbw[2], sbs[2];
    u32x4 lay[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    typedef OutT out8 __attribute__((ext_vector_type(8)));
    typedef float f8v __attribute__((ext_vector_type(8)));

    // ---- the first tile's start: stages 0 and 1, then the tile-boundary slot
    // of the vector-memory stream as every later tile has it: the tile's
    // layout rows and 32 stores that the hardware drops (a window of zero
    // bytes; distinct offsets, so that none is merged away); then stage 0's
    // A fragments 0..3 and B fragments.  (The wait below counts everything
    // issued after stage 0's loads; the scheduler barriers keep that issue
    // order.)
    __builtin_amdgcn_sched_barrier(0);
    dma_stage(rf, L.off, buf0, 0, wave);
    __builtin_amdgcn_sched_barrier(0);
    load_scales(rf, 0, int(p.rows), L.sa_off, sa[0], sbw[0], sbs[0]);
    dma_stage(rf, L.off, buf1, 1, wave);
    load_scales(rf, 1, int(p.rows), L.sa_off, sa[1], sbw[1], sbs[1]);
    __builtin_amdgcn_sched_barrier(0);
    {
        const __amdgpu_buffer_rsrc_t none = make_rsrc(p.d, 0);
        if (!MASKED) {
            const __amdgpu_buffer_rsrc_t mr_ = make_rsrc(p.meta + cur.row0, uint32_t(cur.lim) * 4u);
            lay[0] = __builtin_amdgcn_raw_buffer_load_b128(mr_, uint32_t(L.sa_off) * 4u, 0, 0);
            lay[1] = __builtin_amdgcn_raw_buffer_load_b128(mr_, uint32_t(L.sa_off + 64) * 4u, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 32; ++s)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, none, 0x80000000u + 16u * uint32_t(s), 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    GFG_WAITCNT(2 * SL + DMA_OPS + Epi<MASKED>::OPS, 15);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int y = 0; y < 4; ++y)
        af[y] = join(lds16(buf0, frag_off(L.a_lo_e, L.a_lo_o, y)), lds16(buf0, frag_off(L.a_hi_e, L.a_hi_o, y)));
#pragma unroll
    for (int x = 0; x < 8; ++x)
        bf0[x] = join(lds16(buf0, frag_off(L.b_lo_e, L.b_lo_o, x)), lds16(buf0, frag_off(L.b_hi_e, L.b_hi_o, x)));

    while (true) {
#pragma unroll
        for (int y = 0; y < 8; ++y)
#pragma unroll
            for (int x = 0; x < 8; ++x) acc[y][x] = v4f{};
        i = __builtin_amdgcn_readfirstlane(i);
        const unsigned i_next = i + order.slots;
        const bool have_next = i_next < order.x_count;
        // the next tile, decoded here (its divisions stay out of the K loop)
        TileInfo next = cur;
        if (have_next) {
            int mr2, nt2;
            order.item(i_next, gm, unsigned(NT), unsigned(n_work), &mr2, &nt2);
            next = tile_info<MASKED>(p, __builtin_amdgcn_readfirstlane(work[mr2]), nt2);
        }
        // The stage refilled by step k is k + 2 of this tile; from step KB - 2 on it is
        // the next tile's stage k + 2 - KB (KB is even, so it lands in the buffer
        // that stage expects), or, on the last tile, a dummy copy of the last stage.
        // The loop runs at least once (KB >= 2), which the compiler is told, so
        // its own waits at the tile boundary count the boundary's operations.
        // The tile's first pair of steps is peeled: its second-half wait also
        // counts the tile-boundary operations.  (A run-time choice of the wait
        // inside the step would put a branch between the halves, and the
        // compiler then moves the first half's MFMAs past the barrier.)
        int kb = 0;
        auto refills = [&](int k, int& r0, int& r1) {
            if (k + 2 == KB && have_next) rf = make_refill<MASKED>(p, next, L.wn);
            r0 = k + 2 < KB ? k + 2 : (have_next ? k + 2 - KB : KB - 1);
            r1 = k + 3 < KB ? k + 3 : (have_next ? k + 3 - KB : KB - 1);
        };
        {
            int kr0, kr1;
            refills(0, kr0, kr1);
            if constexpr (MASKED)
                k_step<0, SL + FIRST_HALF_DMA + Epi<MASKED>::OPS>(L, int(p.rows), buf0, buf0 + A_BYTES, buf1, kr0, rf, acc, af, bf0, bf1, sa, sbw, sbs);
            else
                k_step<0, SL + FIRST_HALF_DMA + Epi<MASKED>::OPS, MASKED, true>(L, int(p.rows), buf0, buf0 + A_BYTES, buf1, kr0, rf, acc, af, bf0, bf1,
                                                                sa, sbw, sbs, okm_lds, lay, cur.lim, cur.g);
            k_step<1, SL + FIRST_HALF_DMA>(L, int(p.rows), buf1, buf1 + A_BYTES, buf0, kr1, rf, acc, af, bf1, bf0, sa, sbw, sbs);
            kb = 2;
        }

        while (kb < KB) {
            int kr0, kr1;
            refills(kb, kr0, kr1);
            k_step<0, SL + FIRST_HALF_DMA>(L, int(p.rows), buf0, buf0 + A_BYTES, buf1, kr0, rf, acc, af, bf0, bf1, sa, sbw, sbs);
            k_step<1, SL + FIRST_HALF_DMA>(L, int(p.rows), buf1, buf1 + A_BYTES, buf0, kr1, rf, acc, af, bf1, bf0, sa, sbw, sbs);
            kb += 2;
        }

        // ---- epilogue.  Lane (l16, lq) holds, for each y, output row
        // 128 wm + 64 (y >> 2) + 4 l16 + (y & 3), and for each column half hx
        // the 16 columns 128 wn + 64 hx + 16 lq .. +15 (acc[y][4 hx + x][i] is
        // column 16 lq + 4 i + x): the 16-byte chunks 2 lq and 2 lq + 1 of that
        // row's 128-byte line.  Swapping lane bit 0 with the chunk (DPP
        // quad_perm 1,0,3,2) hands slot h of lane (l16, lq) chunk 2 lq + (l16 & 1)
        // of row 4 ((l16 & ~1) | h) + y, so every store instruction writes eight
        // whole lines; those go out non-temporal.
        // The next tile's layout words are loaded first: they complete before
        // the stores (completion follows issue order), so the next tile's
        // first step can use them without waiting for the stores.  After the
        // last tile the window is empty: the loads return zeros and touch no
        // memory, and no branch splits the stores.
        if (!MASKED) {
            const __amdgpu_buffer_rsrc_t mr_ =
                make_rsrc(p.meta + next.row0, have_next ? uint32_t(next.lim) * 4u : 0u);
            lay[0] = __builtin_amdgcn_raw_buffer_load_b128(mr_, uint32_t(L.sa_off) * 4u, 0, 0);
            lay[1] = __builtin_amdgcn_raw_buffer_load_b128(mr_, uint32_t(L.sa_off + 64) * 4u, 0, 0);
        }
        GFG_SB();
        const int64_t out_row0 = (MASKED ? int64_t(cur.g) * p.rows : 0) + cur.row0;
        const __amdgpu_buffer_rsrc_t dr = make_rsrc(reinterpret_cast<uint8_t*>(p.d) + (out_row0 * p.N + cur.n0) * 2,
                                                    uint32_t(BM) * uint32_t(p.N) * 2u);
        const int ln = lane_now();
        // bit y: the lane's own row for y may be written (the masked layout's
        // rows end at the tile's limit; the contiguous layout's also belong to
        // the tile's group)
        const int okm = MASKED ? row_mask<true>(L, lay, cur.lim, cur.g) : int(okm_lds[L.wave * 64 + ln]);
        // per slot h, the row bits of the pair lane whose rows the slot now holds
        const int okh[2] = {__builtin_amdgcn_update_dpp(0, okm, 0xA0, 0xF, 0xF, false),
                            __builtin_amdgcn_update_dpp(0, okm, 0xF5, 0xF, 0xF, false)};
        const bool odd = (ln & 1) != 0;
        const uint32_t rbase = uint32_t(L.wm * 128 + 4 * ((ln & 15) & ~1));
        const uint32_t colb = uint32_t((L.wn * 128 + 16 * (ln >> 4) + 8 * (ln & 1)) * 2);
#pragma unroll
        for (int y = 0; y < 8; ++y)
#pragma unroll
            for (int hx = 0; hx < 2; ++hx) {
                u32x4 P[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const v4f c0 = acc[y][4 * hx], c1 = acc[y][4 * hx + 1], c2 = acc[y][4 * hx + 2],
                              c3 = acc[y][4 * hx + 3];
                    const f8v v = {c0[2 * hh], c1[2 * hh], c2[2 * hh], c3[2 * hh],
                                   c0[2 * hh + 1], c1[2 * hh + 1], c2[2 * hh + 1], c3[2 * hh + 1]};
                    P[hh] = __builtin_bit_cast(u32x4, __builtin_convertvector(v, out8));
                }
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t a = P[0][d], b = P[1][d];
                    const uint32_t ax = uint32_t(__builtin_amdgcn_update_dpp(0, int(a), 0xB1, 0xF, 0xF, false));
                    const uint32_t bx = uint32_t(__builtin_amdgcn_update_dpp(0, int(b), 0xB1, 0xF, 0xF, false));
                    P[0][d] = odd ? bx : a;
                    P[1][d] = odd ? b : ax;
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint32_t row = rbase + uint32_t(4 * hh + 64 * (y >> 2) + (y & 3));
                    // a row that may not be written gets bit 31, past the
                    // window's end (the offset itself stays below 2^31)
                    const uint32_t voff = (row * uint32_t(p.N) * 2u + colb + uint32_t(128 * hx)) |
                                          ((~uint32_t(okh[hh]) >> y) << 31);
                    __builtin_amdgcn_raw_buffer_store_b128(P[hh], dr, voff, 0, 2 /* nt */);
                }
                GFG_SB();
            }
        if (!have_next) break;
        cur = next;
        i = i_next;
    }
    GFG_WAITCNT(0, 0);   // the dummy refills of the last steps land before the workgroup ends
}

}  // namespace

// Launch the 256 x 256 kernel.  The caller has checked: N a multiple of 256 and
// at most 2^22, K / 128 even, scale rows a multiple of 4 and scale_a 4-byte
// aligned, n_cand <= 4096 candidates of the layout's tile height (128-row for
// the contiguous layout, 256-row for the masked one).
int launch_gemm256(const Params& p, bool masked, unsigned n_cand, int out_dtype, hipStream_t s) {
    int cus = 0;
    if (int rc = device_cus(&cus)) return rc;
    const unsigned NT = unsigned(p.N / BN);
    const unsigned upper = n_cand * NT;
    unsigned grid = upper < unsigned(cus) ? upper : unsigned(cus);
    const int lim = grid_limit();
    if (lim > 0 && grid > unsigned(lim)) grid = unsigned(lim);
    const unsigned nx = unsigned(p.num_xcd);
    grid = (grid + nx - 1) / nx * nx;
    if (grid == 0) return GFG_OK;
    const bool bf16 = out_dtype == GFG_OUT_BF16;
    if (masked) {
        if (bf16)
            hipLaunchKernelGGL((grouped_fp8_gemm256_kernel<true, __bf16>), dim3(grid), dim3(NTHREADS), 0, s, p);
        else
            hipLaunchKernelGGL((grouped_fp8_gemm256_kernel<true, _Float16>), dim3(grid), dim3(NTHREADS), 0, s, p);
    } else {
        if (bf16)
            hipLaunchKernelGGL((grouped_fp8_gemm256_kernel<false, __bf16>), dim3(grid), dim3(NTHREADS), 0, s, p);
        else
            hipLaunchKernelGGL((grouped_fp8_gemm256_kernel<false, _Float16>), dim3(grid), dim3(NTHREADS), 0, s, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GFG_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GFG_OK;
}

}  // namespace gfg
