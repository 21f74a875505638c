// Device-side pieces shared by the grouped GEMM kernels of libgfg (gfx950).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace gfg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Arguments of one grouped GEMM launch (either layout).
struct Params {
    const uint8_t* a;        // contiguous [M][K]; masked [G][Mmax][K]
    const uint8_t* a_scale;  // contiguous [KB][M]; masked [G][KB][Mmax]
    const uint8_t* b;        // [G][N][K]
    const uint8_t* b_scale;  // [G][NB][KB]
    const int32_t* meta;     // grouped_layout [M] or masked_m [G]
    void* d;                 // contiguous [M][N]; masked [G][Mmax][N]
    int64_t rows;            // contiguous: M; masked: Mmax
    int N, K, G;
    int n_cand;              // candidate M tiles of the kernel's tile height
    int mt_per_group;        // masked: candidate M tiles per group
    int group_m;             // grouped-M width in M tiles (0: the kernel's default)
    int num_xcd;             // XCDs the tile order is split over (1: one linear order)
};

#define GFG_LDS __attribute__((address_space(3)))

// s_waitcnt immediate (gfx9 encoding): wait until at most VM vector-memory
// operations and LG LDS/scalar operations of this wave are outstanding.
#define GFG_WAITCNT(VM, LG) \
    __builtin_amdgcn_s_waitcnt(((VM) & 15) | ((((VM) >> 4) & 3) << 14) | (7 << 4) | (((LG) & 15) << 8))

// Raw buffer resource over [base, base + bytes): stride 0, 32-bit data format.
// The hardware returns zero for loads, and drops stores, at offsets past `bytes`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}

// A wave-uniform pointer re-materialized from scalar registers.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    return reinterpret_cast<const uint8_t*>((uint64_t(hi) << 32) | lo);
}

// The 4-byte word holding scale byte kb of a wave's scale_b row, read through
// the scalar data cache into a scalar register (the byte is extracted where it
// is used).  A scalar load is counted by lgkmcnt, not by the vector-memory
// counter that the LDS DMA waits use.  An aligned word that contains a byte of
// an allocation lies in the same page as that byte.
typedef const __attribute__((address_space(4))) uint32_t sword_t;
__device__ __forceinline__ int load_scale_word(const uint8_t* row, int kb) {
    return int(*reinterpret_cast<sword_t*>(reinterpret_cast<uintptr_t>(row + kb) & ~uintptr_t(3)));
}
__device__ __forceinline__ int scale_byte(int word, const uint8_t* row, int kb) {
    return (word >> (8 * int((reinterpret_cast<uintptr_t>(row) + uintptr_t(kb)) & 3))) & 0xff;
}

// The tile order shared by the kernels: T = (M tiles) x (N tiles) work items
// are dealt to `num_xcd` XCDs as contiguous ranges (the hardware places
// workgroup w on XCD w % 8, so a range stays in one XCD's L2), and inside a
// range the items follow a grouped-M order gm M tiles wide, with a shortened
// final group.  Returns the M-tile rank and N tile of item i of this
// workgroup's share, or false past its end.
struct TileOrder {
    unsigned x_start, x_count, slot, slots;
    __device__ __forceinline__ void init(unsigned T, int num_xcd) {
        const unsigned nx = unsigned(num_xcd);
        const unsigned xcd = blockIdx.x % nx;
        slot = blockIdx.x / nx;
        slots = gridDim.x / nx;
        const unsigned per = T / nx, rem = T % nx;
        x_start = xcd * per + (xcd < rem ? xcd : rem);
        x_count = per + (xcd < rem ? 1u : 0u);
    }
    __device__ __forceinline__ void item(unsigned i, unsigned gm, unsigned NT, unsigned n_mtiles, int* mrank,
                                         int* nt) const {
        const unsigned t = x_start + i;
        const unsigned per_group = gm * NT;
        const unsigned grp = t / per_group;
        const unsigned first = grp * gm;
        const unsigned gsz = min(gm, n_mtiles - first);
        const unsigned in_grp = t - grp * per_group;
        *mrank = int(first + in_grp % gsz);
        *nt = int(in_grp / gsz);
    }
};

// The CU count of the current device (cached per device).
int device_cus(int* cus);

// The 256 x 256-tile kernel of the plain grouped GEMM (gfg_gemm256.hip).
// n_cand: candidate M tiles (contiguous: 128-row, masked: 256-row, with
// p.mt_per_group = ceil(M_max / 256)).
int launch_gemm256(const Params& p, bool masked, unsigned n_cand, int out_dtype, hipStream_t s);

}  // namespace gfg
