// Grouped FP8 (E4M3) block-scaled GEMM on 256 x 256 output tiles for gfx950
// (MI355X): the launches with enough 256 x 256 tiles to give every CU one.
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
//  * 8 wave64s, two per SIMD; wave w owns rows 128*(w >> 2) .. +127 and
//    columns 64*(w & 3) .. +63 of the tile, so each SIMD holds one wave of
//    each half of the rows;
//  * v_mfma_scale_f32_32x32x64_f8f6f4 with the E8M0 bytes as hardware scale
//    operands; a 128-K step is two 64-K halves, and the fragments of the next
//    half are read from LDS while the current half's eight MFMAs run.  The
//    four A fragments roll through four register slots (fragment y is
//    replaced as soon as its two MFMAs are issued), the two B fragments are
//    double-buffered: 128 accumulators plus 64 fragment registers;
//  * two 64 KB LDS stages filled by direct-to-LDS loads; the LDS rows are
//    stored fragment-major (row 32*y + p of a wave's A rows holds tile row
//    4p + y, so a lane's four output rows are adjacent and share one A-scale
//    dword), with 16-byte chunks XOR-swizzled by (row >> 1) & 7, which keeps
//    both the fragment reads and the DMA writes free of bank conflicts;
//  * a persistent grid over (M tile, N tile) work items in the shared
//    XCD-range / grouped-M order; the refills of a tile's last two steps load
//    the next tile's first two stages, and the tile's output stores are
//    issued after them, so neither the next tile's first loads nor the output
//    write stand between two tiles' MFMAs;
//  * the contiguous layout's M tiles follow each expert's run of 128-row
//    tiles in pairs (a run of odd length ends in a 128-row tile);
//  * output through buffer stores of whole 128-byte lines: a 4 x 4 DPP
//    transpose inside each lane quad turns the MFMA's (row, 16 columns) per
//    lane into eight complete lines per store instruction, sent non-temporal
//    (measured on the 32768 x 7168 x 2304 grouped case: partial-line stores
//    cost about a fifth of the kernel time, whole-line temporal stores half
//    of that, whole-line non-temporal ones a third of that again);
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
constexpr int NTHREADS = 512, WAVES = 8;
constexpr int A_BYTES = BM * BK;                 // 32 KB of A per stage
constexpr int STAGE = A_BYTES + BN * BK;         // + 32 KB of B
constexpr int A_DMA = A_BYTES / 1024 / WAVES;    // 1 KB DMA instructions per wave and stage
constexpr int B_DMA = BN * BK / 1024 / WAVES;
constexpr int CAND_MAX = 4096;                   // candidate M tiles (128-row contiguous, 256-row masked)
constexpr int FRAG_ROWS = 32 * BK;               // LDS bytes of one 32-row fragment

// Vector-memory operations a wave issues, in order: per stage A_DMA + B_DMA
// DMAs then one A-scale dword load; per tile boundary 16 output stores and,
// for the contiguous layout, one load of the next tile's grouped_layout rows.
constexpr int DMA_OPS = A_DMA + B_DMA;
constexpr int SL = 1;
template <bool MASKED>
struct Epi {
    static constexpr int OPS = 16 + (MASKED ? 0 : 1);
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
    r.sb_row = uniform_ptr(p.b_scale + (int64_t(t.g) * (p.N / 128) + (t.n0 + wn * 64) / 128) * KB);
    return r;
}

// Block-wide exclusive scan (sum, or max with identity -1) over the 512 threads.
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

// Issue one stage's loads: its A and B tiles by LDS DMA into `dst` and this
// lane's scales (A: the dword of its four rows; B: the wave's scale word).
// DMA chunk j of wave w fills LDS rows 8*(j*WAVES + w) .. +7 of A (then B);
// lane i writes physical chunk i % 8 of row +i/8 from the offsets in off_a /
// off_b (tile-invariant; the K step enters as the scalar offset).
struct LaneOffsets {
    uint32_t a[A_DMA];
    uint32_t b[B_DMA];
};

__device__ __forceinline__ void dma_stage(const Refill& r, const LaneOffsets& o, GFG_LDS uint8_t* dst, int kb,
                                          int wave) {
    const uint32_t ks = uint32_t(kb) * BK;
#pragma unroll
    for (int j = 0; j < A_DMA; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r.a_rsrc, (GFG_LDS void*)(dst + (j * WAVES + wave) * 1024), 16, o.a[j],
                                                 ks, 0, 0);
#pragma unroll
    for (int j = 0; j < B_DMA; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r.b_rsrc,
                                                 (GFG_LDS void*)(dst + A_BYTES + (j * WAVES + wave) * 1024), 16,
                                                 o.b[j], ks, 0, 0);
}

// (The K-block stride goes into the vector offset, which the hardware range
// check covers: rows past the region's end in the last K-block read zero
// instead of bytes past the tensor.)
__device__ __forceinline__ void load_scales(const Refill& r, int kb, int rows, int sa_off, int& sa, int& sbw,
                                            int& sbs) {
    sa = int(__builtin_amdgcn_raw_buffer_load_b32(r.sa_rsrc, uint32_t(sa_off) + uint32_t(kb) * uint32_t(rows), 0, 0));
    sbw = load_scale_word(r.sb_row, kb);
    sbs = 8 * int((reinterpret_cast<uintptr_t>(r.sb_row) + uintptr_t(kb)) & 3);
}

__device__ __forceinline__ v8i read_frag(const GFG_LDS uint8_t* __restrict__ src, int a0, int a1) {
    const u32x4 l = *reinterpret_cast<const GFG_LDS u32x4*>(src + a0);
    const u32x4 h = *reinterpret_cast<const GFG_LDS u32x4*>(src + a1);
    return __builtin_bit_cast(v8i, __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Instruction order of one half step for the scheduler: MFMA (y, 0), a B
// fragment read (two ds_read), [DMAs], MFMA (y, 1), A fragment y's two reads,
// [DMAs]; the scale loads last.
template <int Y, int NV>
__device__ __forceinline__ void sched_half() {
    if constexpr (Y < 4) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA (y, 0)
        if constexpr (Y < 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // B fragment read
        if constexpr (NV > 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // DMA
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA (y, 1)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                  // A fragment y
        if constexpr (NV > 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // DMA
        sched_half<Y + 1, NV>();
    }
}

template <int Y>
__device__ __forceinline__ void mfma_row(v16f (&acc)[4][2], const v8i (&bf)[2], const v8i& a, int sb, int sa) {
    acc[Y][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[0], a, acc[Y][0], 0, 0, 0, sb, Y, sa);
    acc[Y][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[1], a, acc[Y][1], 0, 0, 0, sb, Y, sa);
}

struct Lane {
    int a_addr[2][2];    // [K half][chunk] LDS offsets of this lane's A fragment reads (+ 4096 * y)
    int b_addr[2][2];    // B (+ 4096 * x), from the stage base
    LaneOffsets off;     // DMA source offsets
    int wave, wm, wn, sa_off;
};

// One 128-K step k: stage k in `cur`, stage k+1 in `nxt` (its DMA in flight
// until this step's second half).  On entry af / bf0 hold the fragments of
// (k, K half 0).  The first half runs their MFMAs and reads (k, half 1); the
// second half waits for stage k+1 and the other waves, refills `cur` with
// stage kr (k + 2 of this tile, or the next tile's stage, or a dummy copy of
// the last stage when nothing is left), runs (k, half 1) and reads
// (k+1, half 0) from `nxt`.  VMWAIT: vector-memory operations issued after
// stage k+1's DMAs (its A-scale load, plus the tile-boundary operations in the
// first step of a tile).  Both halves are straight-line code, so the
// scheduler keeps the MFMA / fragment-read / DMA interleave.
template <int PAR, int VMWAIT>
__device__ __forceinline__ void k_step(const Lane& L, int rows, GFG_LDS uint8_t* __restrict__ cur,
                                       GFG_LDS uint8_t* __restrict__ nxt, int kr, const Refill& rf,
                                       v16f (&acc)[4][2], v8i (&af)[4], v8i (&bf0)[2], v8i (&bf1)[2], int (&sa)[2],
                                       int (&sbw)[2], int (&sbs)[2]) {
    const int sa_k = sa[PAR];
    const int sb_k = (sbw[PAR] >> sbs[PAR]) & 0xff;
    // ---- K half 0
    __builtin_amdgcn_sched_barrier(0);
    GFG_WAITCNT(63, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_row<0>(acc, bf0, af[0], sb_k, sa_k);
    bf1[0] = read_frag(cur, L.b_addr[1][0], L.b_addr[1][1]);
    af[0] = read_frag(cur, L.a_addr[1][0], L.a_addr[1][1]);
    mfma_row<1>(acc, bf0, af[1], sb_k, sa_k);
    bf1[1] = read_frag(cur, L.b_addr[1][0] + FRAG_ROWS, L.b_addr[1][1] + FRAG_ROWS);
    af[1] = read_frag(cur, L.a_addr[1][0] + FRAG_ROWS, L.a_addr[1][1] + FRAG_ROWS);
    mfma_row<2>(acc, bf0, af[2], sb_k, sa_k);
    af[2] = read_frag(cur, L.a_addr[1][0] + 2 * FRAG_ROWS, L.a_addr[1][1] + 2 * FRAG_ROWS);
    mfma_row<3>(acc, bf0, af[3], sb_k, sa_k);
    af[3] = read_frag(cur, L.a_addr[1][0] + 3 * FRAG_ROWS, L.a_addr[1][1] + 3 * FRAG_ROWS);
    sched_half<0, 0>();
    // ---- K half 1
    __builtin_amdgcn_sched_barrier(0);
    GFG_WAITCNT(VMWAIT, 0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mfma_row<0>(acc, bf1, af[0], sb_k, sa_k);
    bf0[0] = read_frag(nxt, L.b_addr[0][0], L.b_addr[0][1]);
    dma_stage(rf, L.off, cur, kr, L.wave);
    af[0] = read_frag(nxt, L.a_addr[0][0], L.a_addr[0][1]);
    mfma_row<1>(acc, bf1, af[1], sb_k, sa_k);
    bf0[1] = read_frag(nxt, L.b_addr[0][0] + FRAG_ROWS, L.b_addr[0][1] + FRAG_ROWS);
    af[1] = read_frag(nxt, L.a_addr[0][0] + FRAG_ROWS, L.a_addr[0][1] + FRAG_ROWS);
    mfma_row<2>(acc, bf1, af[2], sb_k, sa_k);
    af[2] = read_frag(nxt, L.a_addr[0][0] + 2 * FRAG_ROWS, L.a_addr[0][1] + 2 * FRAG_ROWS);
    mfma_row<3>(acc, bf1, af[3], sb_k, sa_k);
    af[3] = read_frag(nxt, L.a_addr[0][0] + 3 * FRAG_ROWS, L.a_addr[0][1] + 3 * FRAG_ROWS);
    // stage kr's scales replace stage k's, whose last MFMAs are issued above
    load_scales(rf, kr, rows, L.sa_off, sa[PAR], sbw[PAR], sbs[PAR]);
    sched_half<0, DMA_OPS / 4>();
    __builtin_amdgcn_sched_group_barrier(0x020, DMA_OPS - 4 * (DMA_OPS / 4) + SL, 0);
    __builtin_amdgcn_sched_barrier(0);
}

template <bool MASKED, typename OutT>
__global__ __launch_bounds__(NTHREADS, 1) void grouped_fp8_gemm256_kernel(Params p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t smem1[STAGE];
    __shared__ uint32_t work[CAND_MAX];      // work tiles in M order

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    GFG_LDS uint8_t* const buf0 = (GFG_LDS uint8_t*)smem0;
    GFG_LDS uint8_t* const buf1 = (GFG_LDS uint8_t*)smem1;

    // ---- 1. work tiles (the list build uses stage buffer 0 before the first DMA)
    GFG_LDS int16_t* const expo = reinterpret_cast<GFG_LDS int16_t*>(buf0);   // [CAND_MAX]
    GFG_LDS int* const tmp = reinterpret_cast<GFG_LDS int*>(buf0 + 2 * CAND_MAX);
    const int c0 = tid * 8;       // this thread's 8 consecutive candidates
    unsigned wmask = 0;           // bit j: candidate c0 + j starts a work tile
    unsigned hmask = 0;           // contiguous: ... that has only 128 rows (its run ends with it)
    if (MASKED) {
        // candidate g * mt_per_group + j: rows [256 j, 256 j + 256) of group g
#pragma unroll
        for (int j = 0; j < 8; ++j) {
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
        for (int j = 0; j < 8; ++j) {
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
        for (int j = 0; j < 8; ++j) {
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
        for (int j = 0; j < 8; ++j) {
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
    for (int j = 0; j < 8; ++j)
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
    const unsigned gm = p.group_m > 0 ? unsigned(p.group_m) : 4u;
    unsigned i = order.slot;
    if (i >= order.x_count) return;

    Lane L;
    L.wave = wave;
    L.wm = wave >> 2;
    L.wn = wave & 3;
    const int pl = lane & 31, h = lane >> 5, key = (pl >> 1) & 7;
    L.sa_off = L.wm * 128 + 4 * pl;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = ((4 * kh + 2 * h + j) ^ key) << 4;
            L.a_addr[kh][j] = (L.wm * 128 + pl) * BK + c;
            L.b_addr[kh][j] = A_BYTES + (L.wn * 64 + pl) * BK + c;
        }
    // DMA sources.  LDS rows are 128 bytes; the physical chunk (lane & 7) of
    // row R holds logical chunk (lane & 7) ^ ((R >> 1) & 7).
    // A: row R holds tile row 128 (R >> 7) + 4 (R & 31) + ((R >> 5) & 3), so
    // that fragment y's lane row p is tile row 4p + y.
    // B: row R = 64 wn' + 32 x + i holds tile column 64 wn' + 32 x + 16 ((i >> 2) & 1) + 4 (i >> 3) + (i & 3),
    // so that the MFMA hands lane (p, h) columns 32 x + 16 h .. +15 of one output row.
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
        const int R = 8 * (j * WAVES + wave) + (lane >> 3);
        const int tr = (R >> 7) * 128 + 4 * (R & 31) + ((R >> 5) & 3);
        L.off.a[j] = uint32_t(tr) * uint32_t(p.K) + uint32_t(((lane & 7) ^ ((R >> 1) & 7)) << 4);
    }
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) {
        const int R = 8 * (j * WAVES + wave) + (lane >> 3);
        const int ii = R & 31;
        const int col = (R >> 5) * 32 + 16 * ((ii >> 2) & 1) + 4 * (ii >> 3) + (ii & 3);
        L.off.b[j] = uint32_t(col) * uint32_t(p.K) + uint32_t(((lane & 7) ^ ((R >> 1) & 7)) << 4);
    }

    const int KB = p.K / BK;   // even and >= 2 (checked on the host)
    __builtin_assume(KB >= 2);
    int mr, nt;
    order.item(i, gm, unsigned(NT), unsigned(n_work), &mr, &nt);
    TileInfo cur = tile_info<MASKED>(p, work[mr], nt);
    Refill rf = make_refill<MASKED>(p, cur, L.wn);

    v16f acc[4][2];
    v8i af[4], bf0[2], bf1[2];
    int sa[2], sbw[2], sbs[2];
    u32x4 lay = u32x4{0u, 0u, 0u, 0u};
    typedef OutT out8 __attribute__((ext_vector_type(8)));
    typedef float f8v __attribute__((ext_vector_type(8)));

    // ---- prologue: stages 0 and 1 of the first tile, then the tile-boundary
    // slot of the vector-memory stream: 16 stores that the hardware drops (a
    // window of zero bytes) and the layout rows of the tile
    // ---- the first tile's start: stages 0 and 1, then the tile-boundary slot
    // of the vector-memory stream as every later tile has it: 16 stores that
    // the hardware drops (a window of zero bytes; distinct offsets, so that
    // none is merged away) and the tile's layout rows; then stage 0's
    // fragments of K half 0
    // (The wait below counts everything issued after stage 0's loads; the
    // scheduler barriers keep that issue order.)
    __builtin_amdgcn_sched_barrier(0);
    dma_stage(rf, L.off, buf0, 0, wave);
    __builtin_amdgcn_sched_barrier(0);
    load_scales(rf, 0, int(p.rows), L.sa_off, sa[0], sbw[0], sbs[0]);
    dma_stage(rf, L.off, buf1, 1, wave);
    load_scales(rf, 1, int(p.rows), L.sa_off, sa[1], sbw[1], sbs[1]);
    __builtin_amdgcn_sched_barrier(0);
    {
        const __amdgpu_buffer_rsrc_t none = make_rsrc(p.d, 0);
#pragma unroll
        for (int s = 0; s < 16; ++s)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, none, 0x80000000u + 16u * uint32_t(s), 0, 0);
        if (!MASKED) {
            const __amdgpu_buffer_rsrc_t mr_ = make_rsrc(p.meta + cur.row0, uint32_t(cur.lim) * 4u);
            lay = __builtin_amdgcn_raw_buffer_load_b128(mr_, uint32_t(L.sa_off) * 4u, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    GFG_WAITCNT(2 * SL + DMA_OPS + Epi<MASKED>::OPS, 15);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int y = 0; y < 4; ++y)
        af[y] = read_frag(buf0, L.a_addr[0][0] + y * FRAG_ROWS, L.a_addr[0][1] + y * FRAG_ROWS);
#pragma unroll
    for (int x = 0; x < 2; ++x) bf0[x] = read_frag(buf0, L.b_addr[0][0] + x * FRAG_ROWS, L.b_addr[0][1] + x * FRAG_ROWS);

    while (true) {
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
            for (int x = 0; x < 2; ++x) acc[y][x] = v16f{};
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
        int kb = 0;
        do {
            if (kb + 2 == KB && have_next) rf = make_refill<MASKED>(p, next, L.wn);
            const int kr0 = kb + 2 < KB ? kb + 2 : (have_next ? kb + 2 - KB : KB - 1);
            const int kr1 = kb + 3 < KB ? kb + 3 : (have_next ? kb + 3 - KB : KB - 1);
            if (kb == 0)
                k_step<0, SL + Epi<MASKED>::OPS>(L, int(p.rows), buf0, buf1, kr0, rf, acc, af, bf0, bf1, sa, sbw, sbs);
            else
                k_step<0, SL>(L, int(p.rows), buf0, buf1, kr0, rf, acc, af, bf0, bf1, sa, sbw, sbs);
            k_step<1, SL>(L, int(p.rows), buf1, buf0, kr1, rf, acc, af, bf0, bf1, sa, sbw, sbs);
            kb += 2;
        } while (kb < KB);

        // ---- epilogue.  Lane (p, h) holds, for each y, output row 128 wm + 4p + y,
        // columns 64 wn + 32 x + 16 h .. +15 (acc[y][x]): the 16-byte chunks
        // 4x + 2h + jj (jj: which 8 columns) of that row's 128-byte line.  A 4 x 4
        // transpose inside each lane quad (slot s = 2x + jj against lane bits 0
        // and 1, by DPP) hands lane 4q + j, slot s, chunk 4 (j >> 1) + 2h + (j & 1)
        // of row 16q + 4s + y, so every store instruction writes eight whole
        // lines; those go out non-temporal.
        const int64_t out_row0 = (MASKED ? int64_t(cur.g) * p.rows : 0) + cur.row0;
        const __amdgpu_buffer_rsrc_t dr = make_rsrc(reinterpret_cast<uint8_t*>(p.d) + (out_row0 * p.N + cur.n0) * 2,
                                                    uint32_t(BM) * uint32_t(p.N) * 2u);
        // bit y: the lane's own row 128 wm + 4p + y may be written; then, per
        // slot s, the bits of quad lane s (whose rows that slot now holds)
        int okm = 0;
#pragma unroll
        for (int y = 0; y < 4; ++y)
            okm |= int(L.sa_off + y < cur.lim && (MASKED || int(lay[y]) == cur.g)) << y;
        const int okq[4] = {__builtin_amdgcn_update_dpp(0, okm, 0x00, 0xF, 0xF, false),
                            __builtin_amdgcn_update_dpp(0, okm, 0x55, 0xF, 0xF, false),
                            __builtin_amdgcn_update_dpp(0, okm, 0xAA, 0xF, 0xF, false),
                            __builtin_amdgcn_update_dpp(0, okm, 0xFF, 0xF, 0xF, false)};
        const bool j0 = (lane & 1) != 0, j1 = (lane & 2) != 0;
        const uint32_t qrow = uint32_t(L.wm * 128 + 16 * ((lane & 31) >> 2));
        const uint32_t colb = uint32_t(L.wn * 128 + 16 * (4 * ((lane >> 1) & 1) + 2 * h + (lane & 1)));
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            uint32_t P[4][4];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const v16f& a = acc[y][x];
                    const f8v v = {a[8 * jj + 0], a[8 * jj + 1], a[8 * jj + 2], a[8 * jj + 3],
                                   a[8 * jj + 4], a[8 * jj + 5], a[8 * jj + 6], a[8 * jj + 7]};
                    const u32x4 o = __builtin_bit_cast(u32x4, __builtin_convertvector(v, out8));
#pragma unroll
                    for (int d = 0; d < 4; ++d) P[2 * x + jj][d] = o[d];
                }
            // swap lane bit 0 with slot bit 0 (quad_perm 1,0,3,2), then lane bit 1
            // with slot bit 1 (quad_perm 2,3,0,1)
#pragma unroll
            for (int s1 = 0; s1 < 2; ++s1)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t a = P[2 * s1][d], b = P[2 * s1 + 1][d];
                    const uint32_t ax = uint32_t(__builtin_amdgcn_update_dpp(0, int(a), 0xB1, 0xF, 0xF, false));
                    const uint32_t bx = uint32_t(__builtin_amdgcn_update_dpp(0, int(b), 0xB1, 0xF, 0xF, false));
                    P[2 * s1][d] = j0 ? bx : a;
                    P[2 * s1 + 1][d] = j0 ? b : ax;
                }
#pragma unroll
            for (int s0 = 0; s0 < 2; ++s0)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t a = P[s0][d], b = P[2 + s0][d];
                    const uint32_t ax = uint32_t(__builtin_amdgcn_update_dpp(0, int(a), 0x4E, 0xF, 0xF, false));
                    const uint32_t bx = uint32_t(__builtin_amdgcn_update_dpp(0, int(b), 0x4E, 0xF, 0xF, false));
                    P[s0][d] = j1 ? bx : a;
                    P[2 + s0][d] = j1 ? b : ax;
                }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t row = qrow + uint32_t(4 * s + y);
                const uint32_t voff = ((okq[s] >> y) & 1) ? row * uint32_t(p.N) * 2u + colb : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{P[s][0], P[s][1], P[s][2], P[s][3]}, dr, voff, 0,
                                                       2 /* nt */);
            }
        }
        if (!have_next) break;
        cur = next;
        if (!MASKED) {
            const __amdgpu_buffer_rsrc_t mr_ = make_rsrc(p.meta + cur.row0, uint32_t(cur.lim) * 4u);
            lay = __builtin_amdgcn_raw_buffer_load_b128(mr_, uint32_t(L.sa_off) * 4u, 0, 0);
        }
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
