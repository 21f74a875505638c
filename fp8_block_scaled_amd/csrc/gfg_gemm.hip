// Grouped FP8 (E4M3) block-scaled GEMM kernels for gfx950 (MI355X).
//
// Computes D[rows of expert g] = A[rows] . B[g]^T (contiguous layout) and
// D[g, m<masked_m[g]] = A[g] . B[g]^T (masked layout) as defined on the first
// reference page, "Grouped and Batched GEMM kernels with blockscaling
// matching DeepGEMM API" (sections "Summary" and "DeepGEMM conformance
// details"): E4M3 operands, E8M0 scales per (1,128) block of A (stored
// transposed [K/128][M]) and per (128,128) block of B, applied by the
// hardware-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4.
//
// Design (gfx950-first):
//  * one persistent workgroup of 8 wave64s (two per SIMD) per CU; the grid
//    walks a device-built list of valid (expert, 128-row) tiles, so padding
//    tiles (contiguous) and masked-off tiles (masked) cost nothing;
//  * tile order: grouped-M traversal inside contiguous per-XCD ranges (the
//    hardware deals workgroups round-robin over the 8 XCDs, so workgroup w
//    sits on XCD w % 8 and each XCD's L2 sees neighbouring tiles);
//  * a 128 x BN x 128 block tile per K-step: exactly one scale block along
//    K, so each MFMA takes its A and B scale bytes straight from the
//    E8M0 tensors;
//  * three LDS stages per tile, filled by direct-to-LDS global loads
//    (global_load_lds, 16 B per lane) through a 16-byte-chunk XOR swizzle;
//    the loads for step k+3 are issued while step k computes, with explicit
//    vmcnt waits counted per step;
//  * waves laid out 2 (M) x 4 (N), 64 x BN/4 outputs each; fragments for
//    step k+1 are read from LDS while the MFMAs of step k run;
//  * the MFMA's first operand is the B tile (N rows) and its second the A
//    tile (M rows), so a lane's accumulators hold output columns of one row;
//    on the 256-column tile, B fragment x takes the wave's columns 4*l16 + x,
//    which hands each lane 16 consecutive columns of its row; one DPP swap
//    between neighbouring lanes then makes every 16-byte store instruction
//    write eight whole 128-byte lines, sent non-temporal (4 consecutive
//    columns and one 8-byte store per fragment on the 128-column tile and for
//    silu_mul).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <vector>

#include "gfg.h"
#include "gfg_device.h"
#include "gfg_internal.h"

namespace gfg {
namespace {

constexpr int BM = 128;          // rows of A per tile (= scale block edge)
constexpr int BK = 128;          // K per step (= one E8M0 block along K)
constexpr int NTHREADS = 512;    // 8 wave64s, two per SIMD
constexpr int MT_MAX = 4096;     // largest number of candidate 128-row tiles
// Byte offset of 16-byte chunk c (0..7) of row r inside a [rows][128 B] LDS tile.
// XORing the chunk with r & 7 makes both access patterns conflict-free on
// gfx950 (measured with SQ_LDS_BANK_CONFLICT): the MFMA fragment read (16
// consecutive rows, one 16-byte chunk per lane) and the staging write (8 lanes
// per row covering its 8 chunks).
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }

// The A tile is laid out differently: an A fragment takes rows 4 apart (row
// 4*l16 + f of the wave's 64, so that a lane's four rows have adjacent scale
// bytes).  Sixteen such rows all have the same row parity, and the parity
// picks the half of the 64 four-byte banks a 128-byte row falls in, so a plain
// layout reads them with two-way bank conflicts (measured: half the LDS read
// rate).  LDS row p therefore holds A row a_row(p) = p ^ ((p >> 2) & 1), which
// moves every other lane's rows to the other half, and the 16-byte chunks are
// XOR-swizzled with (p >> 2) & 7.  Measured conflict-free at the full rate.
__device__ __forceinline__ int a_row(int p) { return p ^ ((p >> 2) & 1); }   // an involution
__device__ __forceinline__ int swz_a(int p, int c) { return p * BK + ((c ^ ((p >> 2) & 7)) << 4); }

// Candidate 128-row tile c: is it computed, and its auxiliary value (the
// tile's expert for the contiguous layout, its valid rows for the masked one).
template <bool MASKED>
__device__ __forceinline__ bool cand_valid(const Params& p, int c, int* aux) {
    if (MASKED) {
        const int g = c / p.mt_per_group, j = c - g * p.mt_per_group;
        int mm = p.meta[g];
        mm = mm < 0 ? 0 : (mm > p.rows ? int(p.rows) : mm);
        *aux = min(BM, mm - j * BM);
        return *aux > 0;
    } else {
        const int g = p.meta[int64_t(c) * BM];
        *aux = g;
        return g >= 0 && g < p.G;
    }
}

// Per-tile, per-lane constants of the K loop.  SAW: the lane's four A-scale
// bytes (rows 4*l16 .. 4*l16+3 of its wave's 64) are read as one aligned dword
// (scale rows a multiple of 4 bytes apart); otherwise as four bytes.
template <int BN_, bool SAW_, bool SILU_ = false, bool MX_ = false, bool MX4_ = false>
struct TileCtx {
    static constexpr int BN = BN_;
    static constexpr bool SAW = SAW_;
    // MX operands: one E8M0 scale per 32 consecutive K elements of every row of
    // A and of B, both stored transposed ([K/32][rows]).  The scaled MFMA takes
    // a lane's 32 bytes as K [16lq, 16lq + 16) and [64 + 16lq, 80 + 16lq) of its
    // row (logical chunks lq and lq + 4, as loaded) and applies to K-block b
    // (K [32b, 32b + 32)) the scale of lane group b (measured on gfx950 with a
    // one-hot probe).  So lane group lq carries the scales of block 4*kb + lq:
    // one dword per lane and operand, bytes y (A) or x (B) picked by op_sel,
    // and B is staged like A (fragment rows 4*l16 + x) so that a lane's four B
    // rows are adjacent in the transposed scale layout.
    static constexpr bool MX = MX_ || MX4_;
    // MXFP4: E2M1 elements two per byte, so a 128-byte stage row holds 256 K
    // values and feeds two scaled MFMAs, on the lane's 16-byte chunks lq and
    // lq + 4, with a scale dword per half and operand: sa[0], sa[1] for A; sb
    // and sbu for B.  For E2M1 the MFMA takes a lane's 16 bytes as 32
    // consecutive K values, one scale block, and applies lane group b's scale
    // to K [32b, 32b + 32) (measured with a one-hot probe), so the plain
    // packing (element 2i in the low nibble of byte i) is its operand order.
    static constexpr bool MX4 = MX4_;
    // B staged like A (LDS row p holds B row a_row(p)) with fragment x on the
    // wave's columns 4*l16 + x: a lane's accumulators then cover 16
    // consecutive output columns.  Every 256-column tile except silu_mul, whose
    // tile interleaves gate and up rows.
    static constexpr bool BL = MX || (!SILU_ && BN_ == 256);
    // gemm1 with silu_mul: the B tile holds gate and up rows, and fragments
    // x < FN/2 (gate) take the gate block's scale, x >= FN/2 (up) the up block's.
    // (MXFP4: B is staged like A and every row carries its own scales, so
    // lanes with lq < 2 end up with gate values and lanes lq + 2 with the up
    // values of the same columns.)
    static constexpr bool SILU = SILU_;
    static constexpr int WAVES = NTHREADS / 64;
    static constexpr int WN = BN / 4;               // columns per wave (2 x 4 wave grid)
    static constexpr int FN = WN / 16;              // 16-column MFMA tiles per wave
    static constexpr int FM = 4;                    // 16-row MFMA tiles per wave (64 rows)
    static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, STAGE = A_BYTES + B_BYTES;
    static constexpr int A_DMA = A_BYTES / 1024 / WAVES;   // 1 KB LDS-DMA wave instructions per stage
    static constexpr int B_DMA = B_BYTES / 1024 / WAVES;
    // vector-memory loads one wave issues per stage: DMAs and the A scales (one
    // dword or FM bytes); the B-scale dword is a scalar load
    static constexpr int SA_LOADS = SAW ? 1 : FM;
    static constexpr int LOADS = A_DMA + B_DMA + SA_LOADS + (MX ? 1 : 0) + (MX4 ? 2 : 0);   // + B-scale dwords

    // Buffer resources (scalar registers): base + byte count.  The hardware
    // returns zero for any offset past the count instead of touching memory.
    const uint8_t* a_tile;            // A row m0, K 0 of the region
    const uint8_t* b_tile;            // B row n0 of expert g, K 0
    const uint8_t* sa_base;           // scale_a row m0 of K-block 0 (of the region)
    uint32_t sa_kbytes;               // bytes of one K step's scale_a rows from row m0 (sa_stride - m0)
    const uint8_t* sb_row;            // scale_b row (all K-blocks) of this wave's 128-column block
    const uint8_t* sbu_row;           // SILU: scale_b row of the up block (sb_row: the gate block)
    uint32_t sa_stride;        // scale_a bytes between 128-wide K steps
    __amdgpu_buffer_rsrc_t sb_rsrc;   // MX: scale_b of expert g from column n0 of block 0
    uint32_t sb_off, sb_stride;       // MX: this lane's B-scale dword offset, bytes per K step
    uint32_t sb_off1;                 // MX4: the second half's B-scale dword offset (sa_off[1]: A's)
    uint32_t a_off[A_DMA];     // per-lane source offsets of this wave's DMA chunks
    uint32_t b_off[B_DMA];
    uint32_t sa_off[4];        // A-scale byte offsets (SAW: [0] only, the dword)
    // LDS byte offsets of this lane's fragment rows, logical chunks lq (lo) and
    // lq + 4 (hi).  A fragment y sits at a_*_e + y*BK for even y and at
    // a_*_o + y*BK for odd y (the row-parity exchange of the A layout).
    // (BL: B rows as A's, at b_*_e / b_*_o.)
    int a_lo_e, a_lo_o, a_hi_e, a_hi_o, b_lo, b_hi;
    int b_lo_e, b_lo_o, b_hi_e, b_hi_o;
};

template <int BN>
struct Frags {
    v8i a[4];
    v8i b[BN / 64];
};

// The buffer resource of K step kb's scale_a rows from row m0: the range
// check covers the lane's whole offset, so rows past the region's end read
// zero in every K step instead of bytes past the tensor.
template <class C>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sa_rsrc(const C& c, int kb) {
    return make_rsrc(c.sa_base + uint64_t(uint32_t(kb)) * c.sa_stride, c.sa_kbytes);
}

// This lane's A-scale loads for stage kb (one dword, or FM bytes).
template <class C>
__device__ __forceinline__ void load_sa(const C& c, int kb, int (&sa)[4]) {
    const __amdgpu_buffer_rsrc_t rs = sa_rsrc(c, kb);
    if constexpr (C::SAW) {
        sa[0] = int(__builtin_amdgcn_raw_buffer_load_b32(rs, c.sa_off[0], 0, 0));
    } else {
#pragma unroll
        for (int f = 0; f < C::FM; ++f) sa[f] = __builtin_amdgcn_raw_buffer_load_b8(rs, c.sa_off[f], 0, 0);
    }
}

// The packed A-scale word of a stage: byte f = scale of fragment f's row.
template <class C>
__device__ __forceinline__ int sa_word(const int (&sa)[4]) {
    if constexpr (C::SAW) return sa[0];
    else return (sa[0] & 0xff) | ((sa[1] & 0xff) << 8) | ((sa[2] & 0xff) << 16) | (sa[3] << 24);
}

// Issue stage kb's loads: its A/B tiles by LDS DMA into buffer `dst` (A laid
// out with swz_a(), B with swz()) and this lane's scales into (sa, sb).
template <class C>
__device__ __forceinline__ void issue_stage(const C& c, GFG_LDS uint8_t* __restrict__ dst,
                                            int kb, int wave, int (&sa)[4], int& sb, int& sbu) {
    load_sa(c, kb, sa);
    if constexpr (C::MX)
        sb = int(__builtin_amdgcn_raw_buffer_load_b32(c.sb_rsrc, c.sb_off, uint32_t(kb) * c.sb_stride, 0));
    else
        sb = load_scale_word(c.sb_row, kb);
    if constexpr (C::SILU && !C::MX) sbu = load_scale_word(c.sbu_row, kb);
    if constexpr (C::MX4) {
        sa[1] = int(__builtin_amdgcn_raw_buffer_load_b32(sa_rsrc(c, kb), c.sa_off[1], 0, 0));
        sbu = int(__builtin_amdgcn_raw_buffer_load_b32(c.sb_rsrc, c.sb_off1, uint32_t(kb) * c.sb_stride, 0));
    }
    // K-block base pointers made opaque scalars, so each DMA address is a scalar
    // base plus this lane's 32-bit offset (no per-lane 64-bit induction variables)
    const uint8_t* ak = uniform_ptr(c.a_tile + int64_t(kb) * BK);
    const uint8_t* bk = uniform_ptr(c.b_tile + int64_t(kb) * BK);
#pragma unroll
    for (int j = 0; j < C::A_DMA; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(ak + c.a_off[j]),
                                         (GFG_LDS void*)(dst + (j * C::WAVES + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < C::B_DMA; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(bk + c.b_off[j]),
                                         (GFG_LDS void*)(dst + C::A_BYTES + (j * C::WAVES + wave) * 1024), 16, 0, 0);
}

// LDS offset (from the B tile) of B fragment x's chunk for this lane: row
// 16x + l16 of the wave's WN, or with BL row 4*l16 + x in the A-style layout.
template <class C>
__device__ __forceinline__ int b_frag(const C& c, int x, bool hi) {
    if constexpr (C::BL)
        return (hi ? ((x & 1) ? c.b_hi_o : c.b_hi_e) : ((x & 1) ? c.b_lo_o : c.b_lo_e)) + x * BK;
    else
        return (hi ? c.b_hi : c.b_lo) + x * 16 * BK;
}

// Read this lane's fragments of one stage from LDS.  A fragment (16 rows x 128 K):
// lane (l16, lq) holds one row's 16-byte chunks lq and lq + 4; A fragment y
// takes row 4*l16 + y of the wave's 64 rows, B fragment x the row b_frag() names.
template <class C>
__device__ __forceinline__ void read_frags(const C& c, const GFG_LDS uint8_t* __restrict__ src,
                                           Frags<C::BN>& f) {
#pragma unroll
    for (int y = 0; y < C::FM; ++y) {
        const u32x4 l = *reinterpret_cast<const GFG_LDS u32x4*>(src + ((y & 1) ? c.a_lo_o : c.a_lo_e) + y * BK);
        const u32x4 h = *reinterpret_cast<const GFG_LDS u32x4*>(src + ((y & 1) ? c.a_hi_o : c.a_hi_e) + y * BK);
        f.a[y] = __builtin_bit_cast(v8i, __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int x = 0; x < C::FN; ++x) {
        const u32x4 l = *reinterpret_cast<const GFG_LDS u32x4*>(src + C::A_BYTES + b_frag(c, x, false));
        const u32x4 h = *reinterpret_cast<const GFG_LDS u32x4*>(src + C::A_BYTES + b_frag(c, x, true));
        f.b[x] = __builtin_bit_cast(v8i, __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7));
    }
}

// MFMAs of A fragment Y against every B fragment: the A scale is byte Y of
// the packed word (op_sel picks it), the B scale the wave's byte.
// (MX: the B scale is byte X of the lane's dword, the scale of its row 4*l16 + X.)
// (MX4: two FP4 MFMAs per fragment pair, on the low and the high 16 bytes of
// the lane's fragments; saw/sb scale the first, saw1/sbu the second.)
template <class C, int Y, int X = 0>
__device__ __forceinline__ void mfma_row(const Frags<C::BN>& f, int saw, int sb, int sbu, int saw1,
                                         v4f (&acc)[C::FN][4]) {
    if constexpr (X < C::FN) {
        if constexpr (C::MX4) {
            acc[X][Y] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b[X], f.a[Y], acc[X][Y], 4, 4, X, sb, Y,
                                                                         saw);
            acc[X][Y] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                __builtin_shufflevector(f.b[X], f.b[X], 4, 5, 6, 7, -1, -1, -1, -1),
                __builtin_shufflevector(f.a[Y], f.a[Y], 4, 5, 6, 7, -1, -1, -1, -1), acc[X][Y], 4, 4, X, sbu, Y,
                saw1);
        } else {
            acc[X][Y] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                f.b[X], f.a[Y], acc[X][Y], 0, 0, C::MX ? X : 0, (C::SILU && X >= C::FN / 2) ? sbu : sb, Y, saw);
        }
        mfma_row<C, Y, X + 1>(f, saw, sb, sbu, saw1, acc);
    }
}

template <class C>
__device__ __forceinline__ void mfma_stage(const Frags<C::BN>& f, int saw, int sb, int sbu, int saw1,
                                           v4f (&acc)[C::FN][4]) {
    static_assert(C::FM == 4, "four A fragments per wave");
    mfma_row<C, 0>(f, saw, sb, sbu, saw1, acc);
    mfma_row<C, 1>(f, saw, sb, sbu, saw1, acc);
    mfma_row<C, 2>(f, saw, sb, sbu, saw1, acc);
    mfma_row<C, 3>(f, saw, sb, sbu, saw1, acc);
}

// One K-step k.  On entry: fragments of stage k are in `cur` (their LDS reads
// issued during step k-1), stage k+1's DMA was issued two steps ago.  The step
// waits for its own stage-(k+1) DMA and for `cur`, meets the other waves at
// the barrier (after which stage k+1 is visible and nobody reads stage k's
// buffer any more), refills that buffer with stage k+3, issues the reads of
// stage k+1's fragments, and runs stage k's MFMAs while those reads fly.
// VMWAIT = vector-memory loads this wave issued after stage k+1's DMA.
// Instruction order of one K-step for the scheduler: MFMA i is followed by
// DMA i (while i < NV) and fragment read i (while i < NR), so the loads of
// later stages are spread across this stage's MFMAs; the NS scale loads go last.
template <int I, int NM, int NV, int NR, int NS>
__device__ __forceinline__ void sched_pattern() {
    if constexpr (I < NM) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
        if constexpr (I < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read (DMA)
        if constexpr (I < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
        sched_pattern<I + 1, NM, NV, NR, NS>();
    } else if constexpr (NS > 0) {
        __builtin_amdgcn_sched_group_barrier(0x020, NS, 0);           // scale loads
    }
}

template <class C, bool ISSUE, bool READ, int VMWAIT>
__device__ __forceinline__ void k_step(const C& c, GFG_LDS uint8_t* __restrict__ refill,
                                       const GFG_LDS uint8_t* __restrict__ next, int kb_cur, int kb_refill,
                                       int wave,
                                       Frags<C::BN>& cur, Frags<C::BN>& nxt, int (&sa)[4], int& sb, int& sbu,
                                       v4f (&acc)[C::FN][4]) {
    __builtin_amdgcn_sched_barrier(0);
    GFG_WAITCNT(VMWAIT, 0);
    __builtin_amdgcn_s_barrier();
    // nothing that reads this step's scale registers may rise above the wait
    __builtin_amdgcn_sched_barrier(0);
    const int sa_use = sa_word<C>(sa);
    const int sb_use = C::MX ? sb : scale_byte(sb, c.sb_row, kb_cur);
    const int sbu_use = C::MX4 ? sbu : (C::SILU ? scale_byte(sbu, c.sbu_row, kb_cur) : sb_use);
    const int saw1 = C::MX4 ? sa[1] : 0;
    // The LDS DMA and the fragment reads are issued here, through this
    // function's restrict parameters, so the compiler knows the refilled
    // buffer and the buffer being read do not overlap and adds no wait for
    // the DMA before the reads.
    if (ISSUE) {
        const uint8_t* ak = uniform_ptr(c.a_tile + int64_t(kb_refill) * BK);
        const uint8_t* bk = uniform_ptr(c.b_tile + int64_t(kb_refill) * BK);
#pragma unroll
        for (int j = 0; j < C::A_DMA; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(ak + c.a_off[j]),
                                             (GFG_LDS void*)(refill + (j * C::WAVES + wave) * 1024), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < C::B_DMA; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(bk + c.b_off[j]),
                                             (GFG_LDS void*)(refill + C::A_BYTES + (j * C::WAVES + wave) * 1024),
                                             16, 0, 0);
    }
    if (READ) {
        // MX4: the lane's fragment offsets made opaque here, so that the
        // compiler adds the stage buffer's base per step instead of holding
        // one copy of every offset per buffer through the tile (the two
        // extra scale words per stage leave no registers for those copies)
        C o = c;
        if constexpr (C::MX4)
            asm volatile("" : "+v"(o.a_lo_e), "+v"(o.a_lo_o), "+v"(o.a_hi_e), "+v"(o.a_hi_o), "+v"(o.b_lo_e),
                         "+v"(o.b_lo_o), "+v"(o.b_hi_e), "+v"(o.b_hi_o));
#pragma unroll
        for (int y = 0; y < C::FM; ++y) {
            const u32x4 l = *reinterpret_cast<const GFG_LDS u32x4*>(next + ((y & 1) ? o.a_lo_o : o.a_lo_e) + y * BK);
            const u32x4 h = *reinterpret_cast<const GFG_LDS u32x4*>(next + ((y & 1) ? o.a_hi_o : o.a_hi_e) + y * BK);
            nxt.a[y] = __builtin_bit_cast(v8i, __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int x = 0; x < C::FN; ++x) {
            const u32x4 l = *reinterpret_cast<const GFG_LDS u32x4*>(next + C::A_BYTES + b_frag(o, x, false));
            const u32x4 h = *reinterpret_cast<const GFG_LDS u32x4*>(next + C::A_BYTES + b_frag(o, x, true));
            nxt.b[x] = __builtin_bit_cast(v8i, __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    }
    mfma_stage<C>(cur, sa_use, sb_use, sbu_use, saw1, acc);
    if (ISSUE) {   // after the MFMAs that read the old scale registers
        load_sa(c, kb_refill, sa);
        if constexpr (C::MX)
            sb = int(__builtin_amdgcn_raw_buffer_load_b32(c.sb_rsrc, c.sb_off, uint32_t(kb_refill) * c.sb_stride, 0));
        else
            sb = load_scale_word(c.sb_row, kb_refill);
        if constexpr (C::SILU && !C::MX) sbu = load_scale_word(c.sbu_row, kb_refill);
        if constexpr (C::MX4) {
            sa[1] = int(__builtin_amdgcn_raw_buffer_load_b32(sa_rsrc(c, kb_refill), c.sa_off[1], 0, 0));
            sbu = int(__builtin_amdgcn_raw_buffer_load_b32(c.sb_rsrc, c.sb_off1, uint32_t(kb_refill) * c.sb_stride,
                                                           0));
        }
    }
    sched_pattern<0, C::FN * C::FM * (C::MX4 ? 2 : 1), ISSUE ? C::A_DMA + C::B_DMA : 0,
                  READ ? 2 * (C::FM + C::FN) : 0, ISSUE ? C::LOADS - C::A_DMA - C::B_DMA : 0>();
    if (READ) cur = nxt;
    __builtin_amdgcn_sched_barrier(0);
}

// silu(g) * u on four fp32 values: silu(g) = g / (1 + e^-g), the exponential
// by the hardware base-2 exponential (e^-g = 2^(-g * log2 e)) and the division
// by the hardware reciprocal.  Large negative g gives 1 + e^-g = inf and
// silu = -0; large positive g gives e^-g = 0 and silu = g.
__device__ __forceinline__ v4f silu_mul4(v4f gv, v4f uv) {
    v4f r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(gv[i] * -1.44269504088896341f);
        r[i] = gv[i] * __builtin_amdgcn_rcpf(1.0f + e) * uv[i];
    }
    return r;
}

// SILU (gemm1 of the expert MLP): B[g] holds 2*I rows, gate rows [0, I) and
// up rows [I, 2*I); the output is [rows][I] = silu(gate) * up.  A tile covers
// 128 output columns o0.. and stages the 128 matching gate rows and 128 up rows
// as its 256 B rows, interleaved so that each wave's 64 columns are 32 gate
// and the same 32 up columns: fragments x and x + FN/2 of a lane then hold the
// gate and up values of the same four outputs.
// (MX4: p.K counts bytes of a row, half its E2M1 elements.)
template <int BN, bool MASKED, bool SAW, typename OutT, bool SILU, bool MX, bool MX4 = false>
__global__ __launch_bounds__(NTHREADS, 1) void grouped_fp8_gemm_kernel(Params p) {
    static_assert(!SILU || BN == 256, "the gate/up interleave assumes 64 B rows per wave");
    static_assert(!(MX || MX4) || (BN == 256 && SAW && (!SILU || MX4)),
                  "MX runs on the 256-column tile with packed scale words; silu_mul with MXFP4 only");
    using C = TileCtx<BN, SAW, SILU, MX, MX4>;
    constexpr int FN = C::FN, FM = C::FM, WN = C::WN;
    constexpr int L = C::LOADS;

    // three stage buffers as distinct LDS objects: the compiler gives each its
    // own alias scope, so a DMA into one buffer does not make reads of another
    // wait for it
    __shared__ __attribute__((aligned(1024))) uint8_t smem0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t smem1[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t smem2[C::STAGE];
    __shared__ uint16_t tile_list[MT_MAX];   // valid candidate 128-row tiles, ascending
    __shared__ uint16_t tile_aux[MT_MAX];    // contiguous: the tile's expert; masked: its valid rows

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers

    // ---- 1. compact the valid 128-row tiles (order preserved) --------------
    // (the scan's counters sit in stage buffer 0, unused until the first DMA)
    GFG_LDS int* const wave_count = reinterpret_cast<GFG_LDS int*>((GFG_LDS uint8_t*)smem0);
    GFG_LDS int* const s_total = wave_count + NTHREADS / 64;
    if (tid == 0) *s_total = 0;
    __syncthreads();
    for (int base = 0; base < p.n_cand; base += NTHREADS) {
        const int cnd = base + tid;
        int aux = 0;
        const bool v = cnd < p.n_cand && cand_valid<MASKED>(p, cnd, &aux);
        const uint64_t bal = __ballot(v);
        const int before = __popcll(bal & ((uint64_t(1) << lane) - 1));
        if (lane == 0) wave_count[wave] = __popcll(bal);
        __syncthreads();
        int off = *s_total;
        for (int w = 0; w < wave; ++w) off += wave_count[w];
        if (v) {
            tile_list[off + before] = uint16_t(cnd);
            tile_aux[off + before] = uint16_t(aux);
        }
        __syncthreads();
        if (tid == 0) {
            int sum = 0;
            for (int w = 0; w < NTHREADS / 64; ++w) sum += wave_count[w];
            *s_total += sum;
        }
        __syncthreads();
    }
    const int n_mtiles = __builtin_amdgcn_readfirstlane(*s_total);
    __syncthreads();   // every wave has read the counters before the DMA reuses their buffer
    const int NT = p.N / BN;
    const unsigned T = unsigned(n_mtiles) * unsigned(NT);

    // ---- 2. this workgroup's share: a contiguous range per XCD -------------
    TileOrder order;
    order.init(T, p.num_xcd);

    const int KB = p.K / BK;
    const int NB = p.N / 128;
    const int n_out = SILU ? p.N / 2 : p.N;   // output row length
    const int SKB = (MX4 ? 8 : MX ? 4 : 1) * KB;   // scale blocks along K (MX: 32 elements wide)
    const int wm = wave & 1, wn = wave >> 1;
    const int l16 = lane & 15, lq = lane >> 4;
    GFG_LDS uint8_t* const buf0 = (GFG_LDS uint8_t*)smem0;
    GFG_LDS uint8_t* const buf1 = (GFG_LDS uint8_t*)smem1;
    GFG_LDS uint8_t* const buf2 = (GFG_LDS uint8_t*)smem2;

    for (unsigned i = order.slot; i < order.x_count; i += order.slots) {
        // grouped-M order over (valid m-tile rank, n-tile).  When every
        // workgroup has at most two tiles, an XCD's 32 concurrent tiles span
        // 8 m-tiles x 4 n-tiles: on the 128 x 256 tile that streams 8*128 +
        // 4*256 rows of K bytes into its L2 per round instead of 4*128 + 8*256
        // (4 x 8), a fifth less.  Longer walks keep the narrower group_m.
        // (A caller-chosen group_m overrides both.)
        const unsigned gm = p.group_m > 0 ? unsigned(p.group_m) : (T <= 2u * gridDim.x ? 8u : 4u);
        int r_rank, nt;
        order.item(i, gm, unsigned(NT), unsigned(n_mtiles), &r_rank, &nt);

        const int cand = __builtin_amdgcn_readfirstlane(int(tile_list[r_rank]));
        const int aux = __builtin_amdgcn_readfirstlane(int(tile_aux[r_rank]));
        int g;
        int64_t m0;             // first row of the tile inside its region
        const uint8_t* a_reg;   // region base (rows x K)
        const uint8_t* sa_reg;  // region's scale base ([KB][rows])
        uint8_t* d_reg;
        int mlimit;             // rows that may be computed
        if (MASKED) {
            g = cand / p.mt_per_group;
            m0 = int64_t(cand - g * p.mt_per_group) * BM;
            a_reg = p.a + int64_t(g) * p.rows * p.K;
            sa_reg = p.a_scale + int64_t(g) * SKB * p.rows;
            d_reg = reinterpret_cast<uint8_t*>(p.d) + int64_t(g) * p.rows * n_out * int64_t(sizeof(OutT));
            mlimit = int(m0) + aux;
        } else {
            m0 = int64_t(cand) * BM;
            g = aux;
            a_reg = p.a;
            sa_reg = p.a_scale;
            d_reg = reinterpret_cast<uint8_t*>(p.d);
            mlimit = int(p.rows);
        }
        // first B row (GEMM; SILU: first gate row) and first output column
        const int n0 = nt * (SILU ? BN / 2 : BN);

        C c;
        c.a_tile = a_reg + m0 * p.K;
        c.b_tile = p.b + (int64_t(g) * p.N + n0) * p.K;
        c.sa_base = uniform_ptr(sa_reg + m0);
        if constexpr (C::MX) {
            // scale_b [G][K/32][N]: this lane's dword holds rows n0 + wn*WN +
            // 4*l16 .. +3 of block 4*kb + lq (MX4: 8*kb + lq, and 8*kb + 4 + lq)
            const int64_t sbe = int64_t(g) * SKB * p.N;
            c.sb_rsrc = make_rsrc(p.b_scale + sbe + n0, uint32_t(int64_t(SKB) * p.N - n0));
            // (SILU: the lane's four rows are gate rows 32*wn + 4*l16 .. for
            // l16 < 8 and up rows n_out + 32*wn + 4*(l16 - 8) .. otherwise)
            const int brow4 = !SILU ? wn * WN + 4 * l16 : (l16 < 8 ? 32 * wn + 4 * l16 : n_out + 32 * wn + 4 * (l16 - 8));
            c.sb_off = uint32_t(lq * p.N + brow4);
            c.sb_off1 = c.sb_off + uint32_t(4 * p.N);
            c.sb_stride = uint32_t((MX4 ? 8 : 4) * p.N);
        } else if constexpr (SILU) {
            c.sb_row = uniform_ptr(p.b_scale + (int64_t(g) * NB + n0 / 128) * KB);
            c.sbu_row = uniform_ptr(p.b_scale + (int64_t(g) * NB + (n_out + n0) / 128) * KB);
        } else {
            c.sb_row = uniform_ptr(p.b_scale + (int64_t(g) * NB + (n0 + wn * WN) / 128) * KB);
        }
        c.sa_stride = uint32_t((MX4 ? 8 : MX ? 4 : 1) * p.rows);
        c.sa_kbytes = c.sa_stride - uint32_t(m0);
        // DMA chunk j of this wave fills LDS rows 8*(j*WAVES + wave) .. +7; lane i
        // writes physical chunk i%8 of tile row R = +i/8, which holds logical
        // chunk (i%8) ^ key(R) of that row (A: key (R >> 2) & 7, B: R & 7).
        {
            const int rr = lane >> 3, pc = lane & 7;
#pragma unroll
            for (int j = 0; j < C::A_DMA; ++j) {
                const int pr = 8 * (j * C::WAVES + wave) + rr;    // LDS row
                const int lc = pc ^ ((pr >> 2) & 7);
                int64_t row = m0 + a_row(pr);
                row = row < mlimit ? row : mlimit - 1;           // clamp: never read outside
                c.a_off[j] = uint32_t(row - m0) * uint32_t(p.K) + uint32_t(lc * 16);
            }
#pragma unroll
            for (int j = 0; j < C::B_DMA; ++j) {
                const int R = 8 * (j * C::WAVES + wave) + rr;       // LDS row
                // SILU: LDS rows 64w .. 64w+31 hold gate rows o0 + 32w .., rows
                // 64w+32 .. 64w+63 the up rows I + o0 + 32w .. (B rows from n0)
                const int w = R >> 6, q = R & 63;
                if constexpr (C::BL) {   // staged like A: row a_row(R), key (R >> 2) & 7
                    const int ar = a_row(R), aw = ar >> 6, aq = ar & 63;   // a_row stays in R's 4-row group
                    const int brow = !SILU ? ar : (aq < 32 ? 32 * aw + aq : n_out + 32 * aw + (aq - 32));
                    c.b_off[j] = uint32_t(brow) * uint32_t(p.K) + uint32_t((pc ^ ((R >> 2) & 7)) * 16);
                } else {
                    const int brow = !SILU ? R : (q < 32 ? 32 * w + q : n_out + 32 * w + (q - 32));
                    c.b_off[j] = uint32_t(brow) * uint32_t(p.K) + uint32_t((pc ^ rr) * 16);
                }
            }
        }
        // A-scale offsets (from row m0 of K-block 0): the lane's rows are
        // wm*64 + 4*l16 + f.  The dword form needs no clamp: rows come in
        // aligned fours that are all valid or all past the region's end, where
        // the buffer read returns 0 (such rows are never stored).
        if constexpr (SAW) {
            // (MX: block 4*kb + lq of the lane's 32-wide K chunk)
            c.sa_off[0] = uint32_t((C::MX ? lq * int(p.rows) : 0) + wm * 64 + 4 * l16);
            if constexpr (MX4) c.sa_off[1] = c.sa_off[0] + uint32_t(4 * p.rows);
        } else {
#pragma unroll
            for (int f = 0; f < FM; ++f) {
                int64_t row = m0 + wm * 64 + 4 * l16 + f;
                row = row < mlimit ? row : mlimit - 1;
                c.sa_off[f] = uint32_t(row - m0);
            }
        }
        // fragment rows: A row wm*64 + 4*l16 + y lives in LDS row p0 + (y ^ odd)
        // with p0 = wm*64 + 4*l16 and odd = l16 & 1 (swizzle key l16 & 7 for
        // every y); B row wn*WN + x*16 + l16 (key l16 & 7).
        // (BL: B rows wn*WN + 4*l16 + x in LDS rows pb + (x ^ odd), as for A)
        {
            const int clo = lq, chi = lq + 4;
            const int p0 = wm * 64 + 4 * l16, odd = l16 & 1;
            c.a_lo_e = swz_a(p0, clo) + odd * BK;          // even y: row p0 + odd + y
            c.a_lo_o = swz_a(p0, clo) - odd * BK;          // odd y: row p0 - odd + y
            c.a_hi_e = swz_a(p0, chi) + odd * BK;
            c.a_hi_o = swz_a(p0, chi) - odd * BK;
            const int pb = wn * WN + 4 * l16;
            c.b_lo_e = swz_a(pb, clo) + odd * BK;
            c.b_lo_o = swz_a(pb, clo) - odd * BK;
            c.b_hi_e = swz_a(pb, chi) + odd * BK;
            c.b_hi_o = swz_a(pb, chi) - odd * BK;
        }
        c.b_lo = swz(wn * WN + l16, lq);
        c.b_hi = swz(wn * WN + l16, lq + 4);

        v4f acc[FN][FM];
#pragma unroll
        for (int x = 0; x < FN; ++x)
#pragma unroll
            for (int y = 0; y < FM; ++y) acc[x][y] = v4f{0.f, 0.f, 0.f, 0.f};

        Frags<BN> fa, fb;
        int sa0[4], sa1[4], sa2[4], sb0 = 0, sb1 = 0, sb2 = 0, su0 = 0, su1 = 0, su2 = 0;

        // Contiguous layout: the expert of each of this lane's four output rows
        // (4*l16 + y, consecutive grouped_layout entries), read now so that the
        // epilogue does not wait on a load.  The read goes through a buffer
        // resource over the tile's valid rows: entries past them read as 0,
        // and such rows fail the row < mlimit test anyway.
        u32x4 lay = u32x4{0u, 0u, 0u, 0u};
        if constexpr (!MASKED) {
            const int rv = int(min(int64_t(BM), p.rows - m0));
            const __amdgpu_buffer_rsrc_t mr = make_rsrc(p.meta + m0, uint32_t(rv) * 4u);
            lay = __builtin_amdgcn_raw_buffer_load_b128(mr, uint32_t(wm * 64 + 4 * l16) * 4u, 0, 0);
        }

        // prologue: stages 0..2 in flight (clamped to the last stage), stage 0's
        // fragments in `fa`.  The wait counts stage 1's and 2's operations as
        // the only ones younger than stage 0's, so the scheduler must not mix
        // the stages' loads (nor move the layout load among them): the
        // barriers pin the issue order.
        __builtin_amdgcn_sched_barrier(0);
        issue_stage(c, buf0, 0, wave, sa0, sb0, su0);
        __builtin_amdgcn_sched_barrier(0);
        issue_stage(c, buf1, min(1, KB - 1), wave, sa1, sb1, su1);
        __builtin_amdgcn_sched_barrier(0);
        issue_stage(c, buf2, min(2, KB - 1), wave, sa2, sb2, su2);
        __builtin_amdgcn_sched_barrier(0);
        GFG_WAITCNT(2 * L, 15);
        __builtin_amdgcn_s_barrier();
        read_frags(c, buf0, fa);

        // Every step has the same shape: it refills the buffer it frees with
        // stage k+3 (past the end: the last stage again, into a buffer nobody
        // reads any more) and reads stage k+1's fragments (past the end: unused).
        int kb = 0;
        for (; kb + 3 <= KB; kb += 3) {
            k_step<C, true, true, L>(c, buf0, buf1, kb, min(kb + 3, KB - 1), wave, fa, fb, sa0, sb0, su0, acc);
            k_step<C, true, true, L>(c, buf1, buf2, kb + 1, min(kb + 4, KB - 1), wave, fa, fb, sa1, sb1, su1, acc);
            k_step<C, true, true, L>(c, buf2, buf0, kb + 2, min(kb + 5, KB - 1), wave, fa, fb, sa2, sb2, su2, acc);
        }
        if (KB - kb >= 1) k_step<C, true, true, L>(c, buf0, buf1, kb, KB - 1, wave, fa, fb, sa0, sb0, su0, acc);
        if (KB - kb >= 2) k_step<C, true, true, L>(c, buf1, buf2, kb + 1, KB - 1, wave, fa, fb, sa1, sb1, su1, acc);
        // every wave is done with LDS before the next tile's prologue refills it
        GFG_WAITCNT(0, 0);
        __builtin_amdgcn_s_barrier();

        // ---- epilogue: lane owns row (4*l16 + y); columns 16lq .. +15 (BL) or
        // 16x + 4lq .. +3 of the wave's WN ----
        // (SILU: output columns o0 + 32*wn + 16x + 4lq .. +3 for x < FN/2, from
        // gate fragment x and up fragment x + FN/2)
        typedef OutT out4 __attribute__((ext_vector_type(4)));
        if constexpr (SILU && C::MX) {
            // lanes lq < 2 hold the gate values of wave columns 16lq + 4i + x,
            // lanes lq + 2 (32 lanes up) the up values of the same columns:
            // each lane reads its partner's accumulators through ds_bpermute
            const int partner = (lane ^ 32) * 4;
            v4f up[FN][FM];
#pragma unroll
            for (int x = 0; x < FN; ++x)
#pragma unroll
                for (int y = 0; y < FM; ++y)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // (the element goes through a scalar first: a bit_cast of
                        // a vector-element expression reads element 0 here)
                        const float e = acc[x][y][i];
                        up[x][y][i] = __builtin_bit_cast(
                            float, __builtin_amdgcn_ds_bpermute(partner, __builtin_bit_cast(int, e)));
                    }
            if (lq < 2) {
                typedef OutT out8 __attribute__((ext_vector_type(8)));
                typedef float f8v __attribute__((ext_vector_type(8)));
#pragma unroll
                for (int y = 0; y < FM; ++y) {
                    const int row = int(m0) + wm * 64 + 4 * l16 + y;
                    const bool ok = row < mlimit && (MASKED || int(lay[y]) == g);
                    if (!ok) continue;
                    const v4f c0 = silu_mul4(acc[0][y], up[0][y]), c1 = silu_mul4(acc[1][y], up[1][y]);
                    const v4f c2 = silu_mul4(acc[2][y], up[2][y]), c3 = silu_mul4(acc[3][y], up[3][y]);
                    OutT* drow = reinterpret_cast<OutT*>(d_reg) + int64_t(row) * n_out + n0 + wn * (WN / 2) + 16 * lq;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const f8v v = {c0[2 * h], c1[2 * h], c2[2 * h], c3[2 * h],
                                       c0[2 * h + 1], c1[2 * h + 1], c2[2 * h + 1], c3[2 * h + 1]};
                        *reinterpret_cast<out8*>(drow + 8 * h) = __builtin_convertvector(v, out8);
                    }
                }
            }
            continue;
        }
        if constexpr (C::BL && !SILU) {
            // Lane (l16, lq) holds 16-byte chunks 2lq + h (h = 0, 1) of the
            // 128-byte line of row 4*l16 + y.  Swapping lane bit 0 with h (DPP
            // quad_perm 1,0,3,2) hands slot h of the lane chunk 2lq + (l16 & 1)
            // of row 4*((l16 & ~1) | h) + y, so each store instruction writes
            // eight whole lines; those go out non-temporal.  The validity bits
            // of the rows a slot now holds come from the quad lane that owned them.
            typedef OutT out8 __attribute__((ext_vector_type(8)));
            typedef float f8v __attribute__((ext_vector_type(8)));
            int okm = 0;
#pragma unroll
            for (int y = 0; y < FM; ++y) {
                const int row = int(m0) + wm * 64 + 4 * l16 + y;
                okm |= int(row < mlimit && (MASKED || int(lay[y]) == g)) << y;
            }
            const int okh[2] = {__builtin_amdgcn_update_dpp(0, okm, 0xA0, 0xF, 0xF, false),
                                __builtin_amdgcn_update_dpp(0, okm, 0xF5, 0xF, 0xF, false)};
            const bool odd = (lane & 1) != 0;
            OutT* const dcol = reinterpret_cast<OutT*>(d_reg) + n0 + wn * WN + 16 * lq + 8 * (lane & 1);
#pragma unroll
            for (int y = 0; y < FM; ++y) {
                u32x4 P[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const v4f c0 = acc[0][y], c1 = acc[1][y], c2 = acc[2][y], c3 = acc[3][y];
                    const f8v v = {c0[2 * h], c1[2 * h], c2[2 * h], c3[2 * h],
                                   c0[2 * h + 1], c1[2 * h + 1], c2[2 * h + 1], c3[2 * h + 1]};
                    P[h] = __builtin_bit_cast(u32x4, __builtin_convertvector(v, out8));
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
                for (int h = 0; h < 2; ++h) {
                    if (!((okh[h] >> y) & 1)) continue;
                    const int row = int(m0) + wm * 64 + 4 * ((l16 & ~1) | h) + y;
                    __builtin_nontemporal_store(P[h], reinterpret_cast<u32x4*>(dcol + int64_t(row) * p.N));
                }
            }
            continue;
        }
#pragma unroll
        for (int y = 0; y < FM; ++y) {
            const int row = int(m0) + wm * 64 + 4 * l16 + y;   // rows of a region fit in 32 bits
            const bool ok = row < mlimit && (MASKED || int(lay[y]) == g);
            if (!ok) continue;
            if constexpr (C::BL) {
                // lane holds columns wn*WN + 16lq + 4i + x: value acc[x][y][i]
                typedef OutT out8 __attribute__((ext_vector_type(8)));
                OutT* drow = reinterpret_cast<OutT*>(d_reg) + int64_t(row) * p.N + n0 + wn * WN + 16 * lq;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const v4f c0 = acc[0][y], c1 = acc[1][y], c2 = acc[2][y], c3 = acc[3][y];
                    typedef float f8v __attribute__((ext_vector_type(8)));
                    const f8v v = {c0[2 * h], c1[2 * h], c2[2 * h], c3[2 * h],
                                   c0[2 * h + 1], c1[2 * h + 1], c2[2 * h + 1], c3[2 * h + 1]};
                    *reinterpret_cast<out8*>(drow + 8 * h) = __builtin_convertvector(v, out8);
                }
            } else if constexpr (SILU) {
                OutT* drow = reinterpret_cast<OutT*>(d_reg) + int64_t(row) * n_out + n0 + wn * (WN / 2) + 4 * lq;
#pragma unroll
                for (int x = 0; x < FN / 2; ++x)
                    *reinterpret_cast<out4*>(drow + x * 16) =
                        __builtin_convertvector(silu_mul4(acc[x][y], acc[x + FN / 2][y]), out4);
            } else {
                OutT* drow = reinterpret_cast<OutT*>(d_reg) + int64_t(row) * p.N + n0 + wn * WN + 4 * lq;
#pragma unroll
                for (int x = 0; x < FN; ++x)
                    *reinterpret_cast<out4*>(drow + x * 16) = __builtin_convertvector(acc[x][y], out4);
            }
        }
    }
}

// ---------------------------------------------------------------- launch layer
struct DeviceInfo {
    int cus = 0;
    bool ok = false;
};

int device_info(DeviceInfo* out) {
    static std::mutex mu;
    static std::vector<DeviceInfo> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(GFG_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(mu);
    if (int(cache.size()) <= dev) cache.resize(size_t(dev) + 1);
    if (!cache[size_t(dev)].ok) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return fail(GFG_EHIP, "hipDeviceGetAttribute(multiprocessor count) failed");
        cache[size_t(dev)].cus = cus;
        cache[size_t(dev)].ok = true;
    }
    *out = cache[size_t(dev)];
    return GFG_OK;
}

}  // namespace

int device_cus(int* cus) {
    DeviceInfo di;
    if (int rc = device_info(&di)) return rc;
    *cus = di.cus;
    return GFG_OK;
}

namespace {

template <int BN, bool MASKED, bool SAW, typename OutT, bool SILU = false, bool MX = false, bool MX4 = false>
int launch_t(const Params& p, unsigned n_cand_tiles, hipStream_t s) {
    DeviceInfo di;
    if (int rc = device_info(&di)) return rc;
    const unsigned NT = unsigned(p.N / BN);
    const unsigned upper = n_cand_tiles * NT;                 // valid tiles cannot exceed this
    unsigned grid = upper < unsigned(di.cus) ? upper : unsigned(di.cus);
    const int lim = grid_limit();
    if (lim > 0 && grid > unsigned(lim)) grid = unsigned(lim);
    const unsigned nx = unsigned(p.num_xcd);
    grid = (grid + nx - 1) / nx * nx;                         // whole slots on every XCD
    if (grid == 0) return GFG_OK;
    hipLaunchKernelGGL((grouped_fp8_gemm_kernel<BN, MASKED, SAW, OutT, SILU, MX, MX4>), dim3(grid), dim3(NTHREADS), 0,
                       s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GFG_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GFG_OK;
}

template <bool MASKED, bool SAW>
int dispatch_w(const Params& p, unsigned n_cand, int out_dtype, hipStream_t s) {
    const bool bf16 = out_dtype == GFG_OUT_BF16;
    if constexpr (SAW) {
        if (p.N % 256 == 0)
            return bf16 ? launch_t<256, MASKED, true, __bf16>(p, n_cand, s)
                        : launch_t<256, MASKED, true, _Float16>(p, n_cand, s);
    }
    // the byte-wise A-scale fallback keeps more registers live per stage and
    // stays on the 128-column tile, which has room for them
    return bf16 ? launch_t<128, MASKED, SAW, __bf16>(p, n_cand, s) : launch_t<128, MASKED, SAW, _Float16>(p, n_cand, s);
}

// The packed A-scale path needs every scale row (and so every aligned group of
// four rows) to start on a 4-byte boundary.
//
// Tile shape: the 256 x 256 kernel (gfg_gemm256.hip) moves a third fewer bytes
// per FLOP through the global -> LDS path than the 128 x 256 one, but has half
// as many tiles; it is chosen when it still gives every CU at least one tile
// (counted from the candidate M tiles, an upper bound for the masked layout)
// and its requirements hold: N a multiple of 256 and at most 2^22, K / 128
// even, packed A-scale words.
template <bool MASKED>
int dispatch(const Params& p, unsigned n_cand, int out_dtype, hipStream_t s) {
    const bool saw = p.rows % 4 == 0 && reinterpret_cast<uintptr_t>(p.a_scale) % 4 == 0;
    const int choice = tile_shape_choice();
    const bool fits256 = saw && p.N % 256 == 0 && p.N <= (1 << 22) && (p.K / 128) % 2 == 0;
    if (choice == GFG_TILE_256x256 && !fits256)
        return fail(GFG_EUNSUPPORTED,
                    "256 x 256 tiles need N a multiple of 256 (<= 2^22), K/128 even, scale rows a multiple of 4 "
                    "and scale_a 4-byte aligned");
    if (fits256 && choice != GFG_TILE_128x256) {
        Params q = p;
        unsigned nc = n_cand;
        if (MASKED) {
            q.mt_per_group = int((p.rows + 255) / 256);
            q.n_cand = q.mt_per_group * p.G;
            nc = unsigned(q.n_cand);
        }
        // Automatic choice (from timings of both shapes on 26 shapes): one
        // 256 x 256 tile takes about 1.6 times as long as one 128 x 256 tile
        // (1.5 to 1.9 measured), so the 256 x 256 kernel wins when its rounds
        // of tiles over the CUs, times 1.6, are at most the 128 x 256 one's
        // (two rounds against three is from 1% faster to 10% slower; one
        // against two, three against five and four against seven win by 4 to
        // 14%).  A single
        // round of it also needs a K loop of 32 steps or more, which hides
        // its fixed cost per tile (the first stages and the epilogue); the
        // masked layout, counted from the host-side upper bound M_max
        // (masked_m lives in device memory), needs two of its tiles per CU
        // by that count instead.  For the contiguous layout the experts'
        // runs must average at least two 128-row tiles, or most 256-row
        // tiles would be half tiles (the host sees only the total rows;
        // grouped_layout lives in device memory too).
        const uint64_t nt = unsigned(p.N / 256);
        const uint64_t t256 = uint64_t(MASKED ? nc : (n_cand + 1) / 2) * nt;
        const uint64_t t128 = uint64_t(n_cand) * nt;
        int cus = 0;
        if (int rc = device_cus(&cus)) return rc;
        const uint64_t r256 = (t256 + cus - 1) / cus, r128 = (t128 + cus - 1) / cus;
        const bool runs = MASKED || n_cand >= 2 * unsigned(p.G);
        const bool rounds = 8 * r256 <= 5 * r128;   // r256 * 1.6 <= r128
        const bool enough = MASKED ? t256 >= 2 * uint64_t(cus) : (r256 >= 2 || p.K / BK >= 32);
        if (choice == GFG_TILE_256x256 || (runs && rounds && enough))
            return launch_gemm256(q, MASKED, nc, out_dtype, s);
    }
    return saw ? dispatch_w<MASKED, true>(p, n_cand, out_dtype, s) : dispatch_w<MASKED, false>(p, n_cand, out_dtype, s);
}

int check_common(const char* fn, const void* a, const void* sa, const void* b, const void* sb,
                 const void* meta, const void* d, int64_t N, int64_t K, int32_t G, int32_t out_dtype) {
    if (!a || !sa || !b || !sb || !meta || !d) return fail(GFG_EINVAL, "%s: null pointer argument", fn);
    if (out_dtype != GFG_OUT_BF16 && out_dtype != GFG_OUT_F16)
        return fail(GFG_EINVAL, "%s: out_dtype %d is not GFG_OUT_BF16 or GFG_OUT_F16", fn, out_dtype);
    if (G <= 0 || G > 65535) return fail(GFG_EINVAL, "%s: G=%d outside [1, 65535]", fn, G);
    if (N <= 0 || K <= 0) return fail(GFG_EINVAL, "%s: N=%lld K=%lld must be positive", fn, (long long)N, (long long)K);
    if (N % 128 || K % 128)
        return fail(GFG_EUNSUPPORTED, "%s: N=%lld and K=%lld must be multiples of 128", fn, (long long)N, (long long)K);
    if (N > (int64_t(1) << 30) || K > (int64_t(1) << 23))   // 32-bit in-tile offsets
        return fail(GFG_EUNSUPPORTED, "%s: N=%lld or K=%lld too large (N <= 2^30, K <= 2^23)", fn,
                    (long long)N, (long long)K);
    // B rows are addressed from the tile's first row with 32-bit byte offsets
    // (the up rows of silu_mul lie up to N/2 + 255 rows further on), and the
    // MX B scales [K/32][N] of an expert with 32-bit buffer offsets
    if (N * K >= (int64_t(1) << 32))
        return fail(GFG_EUNSUPPORTED, "%s: N*K=%lld bytes of one expert's B must stay below 2^32", fn,
                    (long long)(N * K));
    return GFG_OK;
}

// The A-scale region [scale blocks along K][rows] is read with 32-bit buffer
// offsets.  sk = scale blocks per 128 bytes of a row: 1 for the (1,128) scales,
// 4 for MXFP8, 8 for MXFP4 (K counts bytes here).
int check_scale_extent(const char* fn, int64_t rows, int64_t K, int sk) {
    const int64_t extent = rows * (K / 128) * sk;
    if (extent >= (int64_t(1) << 32))
        return fail(GFG_EUNSUPPORTED, "%s: the A-scale region (%lld bytes) must stay below 2^32", fn,
                    (long long)extent);
    return GFG_OK;
}

// Parameters of a contiguous call: M rows of A mapped to experts by
// grouped_layout, B [G][N][K].  Returns GFG_OK with *n_cand set, or an error.
int contig_params(const char* fn, const void* a, const uint8_t* a_scale, const void* b, const uint8_t* b_scale,
                  const int32_t* grouped_layout, void* d, int64_t M, int64_t N, int64_t K, int32_t G,
                  int32_t out_dtype, int sk, Params* p, int64_t* n_cand) {
    if (M < 0) return fail(GFG_EINVAL, "%s: M=%lld is negative", fn, (long long)M);
    if (int rc = check_common(fn, a, a_scale, b, b_scale, grouped_layout, d, N, K, G, out_dtype)) return rc;
    if (int rc = check_scale_extent(fn, M, K, sk)) return rc;
    *n_cand = (M + BM - 1) / BM;
    if (*n_cand > MT_MAX)
        return fail(GFG_EUNSUPPORTED, "%s: M=%lld exceeds %d rows", fn, (long long)M, MT_MAX * BM);
    *p = Params{};
    p->a = static_cast<const uint8_t*>(a);
    p->a_scale = a_scale;
    p->b = static_cast<const uint8_t*>(b);
    p->b_scale = b_scale;
    p->meta = grouped_layout;
    p->d = d;
    p->rows = M;
    p->N = int(N);
    p->K = int(K);
    p->G = G;
    p->n_cand = int(*n_cand);
    p->mt_per_group = 0;
    p->group_m = locality_group_m();
    p->num_xcd = locality_num_xcd();
    return GFG_OK;
}

// Parameters of a masked call: A [G][M_max][K], rows m < masked_m[g] computed.
int masked_params(const char* fn, const void* a, const uint8_t* a_scale, const void* b, const uint8_t* b_scale,
                  const int32_t* masked_m, void* d, int32_t G, int64_t M_max, int64_t N, int64_t K,
                  int32_t out_dtype, int sk, Params* p, int64_t* n_cand) {
    if (M_max < 0) return fail(GFG_EINVAL, "%s: M_max=%lld is negative", fn, (long long)M_max);
    if (int rc = check_common(fn, a, a_scale, b, b_scale, masked_m, d, N, K, G, out_dtype)) return rc;
    if (int rc = check_scale_extent(fn, M_max, K, sk)) return rc;
    const int64_t per = (M_max + BM - 1) / BM;
    *n_cand = per * G;
    if (*n_cand > MT_MAX)
        return fail(GFG_EUNSUPPORTED, "%s: G*ceil(M_max/128)=%lld exceeds %d", fn, (long long)*n_cand, MT_MAX);
    *p = Params{};
    p->a = static_cast<const uint8_t*>(a);
    p->a_scale = a_scale;
    p->b = static_cast<const uint8_t*>(b);
    p->b_scale = b_scale;
    p->meta = masked_m;
    p->d = d;
    p->rows = M_max;
    p->N = int(N);
    p->K = int(K);
    p->G = G;
    p->n_cand = int(*n_cand);
    p->mt_per_group = int(per);
    p->group_m = locality_group_m();
    p->num_xcd = locality_num_xcd();
    return GFG_OK;
}

// gemm1 + silu_mul runs on the 256-row B tile with the packed A-scale words.
int check_silu(const char* fn, int64_t I, int64_t rows, const uint8_t* a_scale) {
    if (I <= 0) return fail(GFG_EINVAL, "%s: I=%lld must be positive", fn, (long long)I);
    if (I % 128) return fail(GFG_EUNSUPPORTED, "%s: I=%lld must be a multiple of 128", fn, (long long)I);
    if (rows % 4 || reinterpret_cast<uintptr_t>(a_scale) % 4)
        return fail(GFG_EUNSUPPORTED, "%s: needs scale_a rows (%lld) a multiple of 4 and scale_a 4-byte aligned", fn,
                    (long long)rows);
    return GFG_OK;
}

// The MX GEMM runs on the 256-column tile with one scale dword per lane and
// operand: N a multiple of 256, scale rows a multiple of 4, both scale
// tensors 4-byte aligned.
int check_mx(const char* fn, int64_t N, int64_t rows, const uint8_t* a_scale, const uint8_t* b_scale) {
    if (N % 256) return fail(GFG_EUNSUPPORTED, "%s: N=%lld must be a multiple of 256", fn, (long long)N);
    if (rows % 4 || reinterpret_cast<uintptr_t>(a_scale) % 4 || reinterpret_cast<uintptr_t>(b_scale) % 4)
        return fail(GFG_EUNSUPPORTED,
                    "%s: needs scale_a rows (%lld) a multiple of 4 and both scale tensors 4-byte aligned", fn,
                    (long long)rows);
    return GFG_OK;
}

template <bool MASKED, bool MX4 = false>
int dispatch_mx(const Params& p, unsigned n_cand, int out_dtype, hipStream_t s) {
    return out_dtype == GFG_OUT_BF16 ? launch_t<256, MASKED, true, __bf16, false, !MX4, MX4>(p, n_cand, s)
                                     : launch_t<256, MASKED, true, _Float16, false, !MX4, MX4>(p, n_cand, s);
}

template <bool MASKED>
int dispatch_mx4_silu(const Params& p, unsigned n_cand, int out_dtype, hipStream_t s) {
    return out_dtype == GFG_OUT_BF16 ? launch_t<256, MASKED, true, __bf16, true, false, true>(p, n_cand, s)
                                     : launch_t<256, MASKED, true, _Float16, true, false, true>(p, n_cand, s);
}

template <bool MASKED>
int dispatch_silu(const Params& p, unsigned n_cand, int out_dtype, hipStream_t s) {
    return out_dtype == GFG_OUT_BF16 ? launch_t<256, MASKED, true, __bf16, true>(p, n_cand, s)
                                     : launch_t<256, MASKED, true, _Float16, true>(p, n_cand, s);
}

}  // namespace
}  // namespace gfg

using namespace gfg;

extern "C" int grouped_fp8_gemm_contiguous(const void* a, const uint8_t* a_scale, const void* b,
                                           const uint8_t* b_scale, const int32_t* grouped_layout, void* d,
                                           int64_t M, int64_t N, int64_t K, int32_t G, int32_t out_dtype,
                                           void* stream) {
    clear_error();
    Params p;
    int64_t n_cand = 0;
    if (int rc = contig_params("grouped_fp8_gemm_contiguous", a, a_scale, b, b_scale, grouped_layout, d, M, N, K, G,
                               out_dtype, 1, &p, &n_cand))
        return rc;
    if (M == 0) return GFG_OK;
    return dispatch<false>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}

extern "C" int grouped_fp8_gemm_masked(const void* a, const uint8_t* a_scale, const void* b,
                                       const uint8_t* b_scale, const int32_t* masked_m, void* d, int32_t G,
                                       int64_t M_max, int64_t N, int64_t K, int32_t out_dtype, void* stream) {
    clear_error();
    Params p;
    int64_t n_cand = 0;
    if (int rc = masked_params("grouped_fp8_gemm_masked", a, a_scale, b, b_scale, masked_m, d, G, M_max, N, K,
                               out_dtype, 1, &p, &n_cand))
        return rc;
    if (M_max == 0) return GFG_OK;
    return dispatch<true>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}

extern "C" int grouped_fp8_gemm_silu_mul_contiguous(const void* a, const uint8_t* a_scale, const void* b,
                                                    const uint8_t* b_scale, const int32_t* grouped_layout, void* d,
                                                    int64_t M, int64_t I, int64_t K, int32_t G, int32_t out_dtype,
                                                    void* stream) {
    clear_error();
    const char* fn = "grouped_fp8_gemm_silu_mul_contiguous";
    if (int rc = check_silu(fn, I, M < 0 ? 0 : M, a_scale)) return rc;
    Params p;
    int64_t n_cand = 0;
    if (int rc = contig_params(fn, a, a_scale, b, b_scale, grouped_layout, d, M, 2 * I, K, G, out_dtype, 1, &p, &n_cand))
        return rc;
    if (M == 0) return GFG_OK;
    return dispatch_silu<false>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}

extern "C" int grouped_fp8_gemm_silu_mul_masked(const void* a, const uint8_t* a_scale, const void* b,
                                                const uint8_t* b_scale, const int32_t* masked_m, void* d, int32_t G,
                                                int64_t M_max, int64_t I, int64_t K, int32_t out_dtype,
                                                void* stream) {
    clear_error();
    const char* fn = "grouped_fp8_gemm_silu_mul_masked";
    if (int rc = check_silu(fn, I, M_max < 0 ? 0 : M_max, a_scale)) return rc;
    Params p;
    int64_t n_cand = 0;
    if (int rc = masked_params(fn, a, a_scale, b, b_scale, masked_m, d, G, M_max, 2 * I, K, out_dtype, 1, &p, &n_cand))
        return rc;
    if (M_max == 0) return GFG_OK;
    return dispatch_silu<true>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}

extern "C" int grouped_mxfp8_gemm_contiguous(const void* a, const uint8_t* a_scale, const void* b,
                                             const uint8_t* b_scale, const int32_t* grouped_layout, void* d,
                                             int64_t M, int64_t N, int64_t K, int32_t G, int32_t out_dtype,
                                             void* stream) {
    clear_error();
    const char* fn = "grouped_mxfp8_gemm_contiguous";
    Params p;
    int64_t n_cand = 0;
    if (int rc = contig_params(fn, a, a_scale, b, b_scale, grouped_layout, d, M, N, K, G, out_dtype, 4, &p, &n_cand))
        return rc;
    if (int rc = check_mx(fn, N, M, a_scale, b_scale)) return rc;
    if (M == 0) return GFG_OK;
    return dispatch_mx<false>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}

extern "C" int grouped_mxfp8_gemm_masked(const void* a, const uint8_t* a_scale, const void* b,
                                         const uint8_t* b_scale, const int32_t* masked_m, void* d, int32_t G,
                                         int64_t M_max, int64_t N, int64_t K, int32_t out_dtype, void* stream) {
    clear_error();
    const char* fn = "grouped_mxfp8_gemm_masked";
    Params p;
    int64_t n_cand = 0;
    if (int rc = masked_params(fn, a, a_scale, b, b_scale, masked_m, d, G, M_max, N, K, out_dtype, 4, &p, &n_cand))
        return rc;
    if (int rc = check_mx(fn, N, M_max, a_scale, b_scale)) return rc;
    if (M_max == 0) return GFG_OK;
    return dispatch_mx<true>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}

// MXFP4: K counts E2M1 elements; the rows of a and b are K/2 bytes.  K must be
// a multiple of 256 (one 128-byte stage), checked here before the byte sizes
// go to the common checks.
static int check_k4(const char* fn, int64_t K) {
    if (K <= 0) return fail(GFG_EINVAL, "%s: K=%lld must be positive", fn, (long long)K);
    if (K % 256) return fail(GFG_EUNSUPPORTED, "%s: K=%lld must be a multiple of 256", fn, (long long)K);
    return GFG_OK;
}

extern "C" int grouped_mxfp4_gemm_contiguous(const void* a, const uint8_t* a_scale, const void* b,
                                             const uint8_t* b_scale, const int32_t* grouped_layout, void* d,
                                             int64_t M, int64_t N, int64_t K, int32_t G, int32_t out_dtype,
                                             void* stream) {
    clear_error();
    const char* fn = "grouped_mxfp4_gemm_contiguous";
    if (int rc = check_k4(fn, K)) return rc;
    Params p;
    int64_t n_cand = 0;
    if (int rc = contig_params(fn, a, a_scale, b, b_scale, grouped_layout, d, M, N, K / 2, G, out_dtype, 8, &p, &n_cand))
        return rc;
    if (int rc = check_mx(fn, N, M, a_scale, b_scale)) return rc;
    if (M == 0) return GFG_OK;
    return dispatch_mx<false, true>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}

extern "C" int grouped_mxfp4_gemm_masked(const void* a, const uint8_t* a_scale, const void* b,
                                         const uint8_t* b_scale, const int32_t* masked_m, void* d, int32_t G,
                                         int64_t M_max, int64_t N, int64_t K, int32_t out_dtype, void* stream) {
    clear_error();
    const char* fn = "grouped_mxfp4_gemm_masked";
    if (int rc = check_k4(fn, K)) return rc;
    Params p;
    int64_t n_cand = 0;
    if (int rc = masked_params(fn, a, a_scale, b, b_scale, masked_m, d, G, M_max, N, K / 2, out_dtype, 8, &p, &n_cand))
        return rc;
    if (int rc = check_mx(fn, N, M_max, a_scale, b_scale)) return rc;
    if (M_max == 0) return GFG_OK;
    return dispatch_mx<true, true>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}

// a4w4 gemm1 with silu_mul: B [G][2I][K/2] E2M1 (gate rows, then up rows),
// output [rows][I].  K counts E2M1 elements (a multiple of 256), I a multiple
// of 128.
extern "C" int grouped_mxfp4_gemm_silu_mul_contiguous(const void* a, const uint8_t* a_scale, const void* b,
                                                      const uint8_t* b_scale, const int32_t* grouped_layout,
                                                      void* d, int64_t M, int64_t I, int64_t K, int32_t G,
                                                      int32_t out_dtype, void* stream) {
    clear_error();
    const char* fn = "grouped_mxfp4_gemm_silu_mul_contiguous";
    if (int rc = check_k4(fn, K)) return rc;
    if (int rc = check_silu(fn, I, M < 0 ? 0 : M, a_scale)) return rc;
    Params p;
    int64_t n_cand = 0;
    if (int rc = contig_params(fn, a, a_scale, b, b_scale, grouped_layout, d, M, 2 * I, K / 2, G, out_dtype, 8, &p,
                               &n_cand))
        return rc;
    if (int rc = check_mx(fn, 2 * I, M, a_scale, b_scale)) return rc;
    if (M == 0) return GFG_OK;
    return dispatch_mx4_silu<false>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}

extern "C" int grouped_mxfp4_gemm_silu_mul_masked(const void* a, const uint8_t* a_scale, const void* b,
                                                  const uint8_t* b_scale, const int32_t* masked_m, void* d,
                                                  int32_t G, int64_t M_max, int64_t I, int64_t K,
                                                  int32_t out_dtype, void* stream) {
    clear_error();
    const char* fn = "grouped_mxfp4_gemm_silu_mul_masked";
    if (int rc = check_k4(fn, K)) return rc;
    if (int rc = check_silu(fn, I, M_max < 0 ? 0 : M_max, a_scale)) return rc;
    Params p;
    int64_t n_cand = 0;
    if (int rc = masked_params(fn, a, a_scale, b, b_scale, masked_m, d, G, M_max, 2 * I, K / 2, out_dtype, 8, &p,
                               &n_cand))
        return rc;
    if (int rc = check_mx(fn, 2 * I, M_max, a_scale, b_scale)) return rc;
    if (M_max == 0) return GFG_OK;
    return dispatch_mx4_silu<true>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}
