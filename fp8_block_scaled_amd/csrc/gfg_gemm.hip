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
//  * one persistent workgroup of 4 wave64s per CU slot; the grid walks a
//    device-built list of valid (expert, 128-row) tiles, so padding tiles
//    (contiguous) and masked-off tiles (masked) cost nothing;
//  * tile order: grouped-M traversal inside contiguous per-XCD ranges (the
//    hardware deals workgroups round-robin over the 8 XCDs, so workgroup w
//    sits on XCD w % 8 and each XCD's L2 sees neighbouring tiles);
//  * a 128 x BN x 128 block tile per K-step: exactly one scale block along
//    K, so each MFMA takes its A and B scale bytes straight from the
//    E8M0 tensors;
//  * A/B tiles double-buffered in LDS with a 16-byte-chunk XOR swizzle;
//    global loads for step k+1 are in flight while step k computes;
//  * the MFMA's first operand is the B tile (N rows) and its second the A
//    tile (M rows), so each lane ends up owning 4 consecutive output columns
//    of one row, written as one 8-byte store.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <vector>

#include "gfg.h"
#include "gfg_internal.h"

namespace gfg {
namespace {

constexpr int BM = 128;          // rows of A per tile (= scale block edge)
constexpr int BK = 128;          // K per step (= one E8M0 block along K)
constexpr int NTHREADS = 256;    // 4 wave64s, one per SIMD
constexpr int MT_MAX = 4096;     // largest number of candidate 128-row tiles
constexpr int NUM_XCD = 8;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct Params {
    const uint8_t* a;        // contiguous [M][K]; masked [G][Mmax][K]
    const uint8_t* a_scale;  // contiguous [KB][M]; masked [G][KB][Mmax]
    const uint8_t* b;        // [G][N][K]
    const uint8_t* b_scale;  // [G][NB][KB]
    const int32_t* meta;     // grouped_layout [M] or masked_m [G]
    void* d;                 // contiguous [M][N]; masked [G][Mmax][N]
    int64_t rows;            // contiguous: M; masked: Mmax
    int N, K, G;
    int n_cand;              // candidate 128-row tiles: ceil(M/128) or G*ceil(Mmax/128)
    int mt_per_group;        // masked: ceil(Mmax/128)
    int group_m;             // grouped-M width (in 128-row tiles)
};

// Byte offset of 16-byte chunk c (0..7) of row r inside a [rows][128 B] LDS tile.
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }

template <bool MASKED>
__device__ __forceinline__ bool cand_valid(const Params& p, int c, int* g_out) {
    if (MASKED) {
        const int g = c / p.mt_per_group, j = c - g * p.mt_per_group;
        int mm = p.meta[g];
        mm = mm < 0 ? 0 : (mm > p.rows ? int(p.rows) : mm);
        *g_out = g;
        return j * BM < mm;
    } else {
        const int g = p.meta[int64_t(c) * BM];
        *g_out = g;
        return g >= 0 && g < p.G;
    }
}

template <int BN, bool MASKED, typename OutT>
__global__ __launch_bounds__(NTHREADS, 1) void grouped_fp8_gemm_kernel(Params p) {
    constexpr int WN = BN / 2;          // columns per wave (2 x 2 wave grid)
    constexpr int FN = WN / 16;         // 16-column MFMA tiles per wave
    constexpr int FM = 4;               // 16-row MFMA tiles per wave (64 rows)
    constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
    constexpr int A_LD = A_BYTES / (16 * NTHREADS);   // 16-byte loads per thread per step
    constexpr int B_LD = B_BYTES / (16 * NTHREADS);

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (A_BYTES + B_BYTES)];
    __shared__ int tile_list[MT_MAX];   // valid candidates, ascending: cand | group << 13
    __shared__ int wave_count[NTHREADS / 64];
    __shared__ int s_total;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // ---- 1. compact the valid 128-row tiles (order preserved) --------------
    if (tid == 0) s_total = 0;
    __syncthreads();
    for (int base = 0; base < p.n_cand; base += NTHREADS) {
        const int c = base + tid;
        int g = -1;
        const bool v = c < p.n_cand && cand_valid<MASKED>(p, c, &g);
        const uint64_t bal = __ballot(v);
        const int before = __popcll(bal & ((uint64_t(1) << lane) - 1));
        if (lane == 0) wave_count[wave] = __popcll(bal);
        __syncthreads();
        int off = s_total;
        for (int w = 0; w < wave; ++w) off += wave_count[w];
        if (v) tile_list[off + before] = c | (g << 13);
        __syncthreads();
        if (tid == 0) s_total += wave_count[0] + wave_count[1] + wave_count[2] + wave_count[3];
        __syncthreads();
    }
    const int n_mtiles = s_total;
    const int NT = p.N / BN;
    const unsigned T = unsigned(n_mtiles) * unsigned(NT);

    // ---- 2. this workgroup's share: a contiguous range per XCD -------------
    const unsigned xcd = blockIdx.x % NUM_XCD, slot = blockIdx.x / NUM_XCD;
    const unsigned slots = gridDim.x / NUM_XCD;
    const unsigned per = T / NUM_XCD, rem = T % NUM_XCD;
    const unsigned x_start = xcd * per + (xcd < rem ? xcd : rem);
    const unsigned x_count = per + (xcd < rem ? 1u : 0u);

    const int KB = p.K / BK;
    const int NB = p.N / 128;
    const int wm = wave & 1, wn = wave >> 1;
    const int l16 = lane & 15, lq = lane >> 4;

    for (unsigned i = slot; i < x_count; i += slots) {
        // grouped-M order over (valid m-tile rank, n-tile)
        const unsigned t = x_start + i;
        const unsigned gm = unsigned(p.group_m);
        const unsigned per_group = gm * unsigned(NT);
        const unsigned grp = t / per_group;
        const unsigned first = grp * gm;
        const unsigned gsz = min(gm, unsigned(n_mtiles) - first);   // shortened final group
        const unsigned in_grp = t - grp * per_group;
        const int r_rank = int(first + in_grp % gsz);
        const int nt = int(in_grp / gsz);

        const int packed = tile_list[r_rank];
        const int cand = packed & 8191, g = packed >> 13;
        int64_t m0;             // first row of the tile inside its region
        const uint8_t* a_reg;   // region base (rows x K)
        const uint8_t* sa_reg;  // region's scale base ([KB][rows])
        uint8_t* d_reg;
        int mlimit;             // rows that may be computed
        if (MASKED) {
            m0 = int64_t(cand - g * p.mt_per_group) * BM;
            a_reg = p.a + int64_t(g) * p.rows * p.K;
            sa_reg = p.a_scale + int64_t(g) * KB * p.rows;
            d_reg = reinterpret_cast<uint8_t*>(p.d) + int64_t(g) * p.rows * p.N * int64_t(sizeof(OutT));
            int mm = p.meta[g];
            mlimit = mm < 0 ? 0 : (mm > p.rows ? int(p.rows) : mm);
        } else {
            m0 = int64_t(cand) * BM;
            a_reg = p.a;
            sa_reg = p.a_scale;
            d_reg = reinterpret_cast<uint8_t*>(p.d);
            mlimit = int(p.rows);
        }
        const int n0 = nt * BN;
        const uint8_t* b_reg = p.b + (int64_t(g) * p.N + n0) * p.K;

        // global source pointers for this thread's staging chunks
        const uint8_t* pa[A_LD];
        int a_lds[A_LD];
#pragma unroll
        for (int j = 0; j < A_LD; ++j) {
            const int q = j * NTHREADS + tid, r = q >> 3, c = q & 7;
            int64_t row = m0 + r;
            row = row < mlimit ? row : (mlimit > 0 ? mlimit - 1 : 0);   // clamp: never read outside
            pa[j] = a_reg + row * p.K + c * 16;
            a_lds[j] = swz(r, c);
        }
        // B rows are all in bounds: chunk j of this thread is row j*32 + tid/8
        const uint8_t* pb = b_reg + int64_t(tid >> 3) * p.K + (tid & 7) * 16;
        const int64_t b_step = int64_t(NTHREADS / 8) * p.K;
        int b_lds[B_LD];
#pragma unroll
        for (int j = 0; j < B_LD; ++j) {
            const int q = j * NTHREADS + tid, r = q >> 3, c = q & 7;
            b_lds[j] = swz(r, c);
        }
        // scale sources: this lane's 4 A rows, and the wave's B block row
        const uint8_t* psa[FM];
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            int64_t row = m0 + wm * 64 + f * 16 + l16;
            row = row < mlimit ? row : (mlimit > 0 ? mlimit - 1 : 0);
            psa[f] = sa_reg + row;
        }
        const uint8_t* psb = p.b_scale + (int64_t(g) * NB + (n0 + wn * WN) / 128) * KB;

        v4f acc[FN][FM];
#pragma unroll
        for (int x = 0; x < FN; ++x)
#pragma unroll
            for (int y = 0; y < FM; ++y) acc[x][y] = v4f{0.f, 0.f, 0.f, 0.f};

        u32x4 ra[A_LD], rb[B_LD];
        int sa_cur[FM], sa_nxt[FM], sb_cur, sb_nxt;

#define GFG_LOAD_STAGE(KBI)                                                                      \
        {                                                                                        \
            const int64_t ko_ = int64_t(KBI) * BK;                                               \
            _Pragma("unroll") for (int j = 0; j < A_LD; ++j)                                     \
                ra[j] = *reinterpret_cast<const u32x4*>(pa[j] + ko_);                  \
            _Pragma("unroll") for (int j = 0; j < B_LD; ++j)                                     \
                rb[j] = *reinterpret_cast<const u32x4*>(pb + j * b_step + ko_);                  \
        }
#define GFG_LOAD_SCALES(KBI, SA, SB)                                                             \
        {                                                                                        \
            _Pragma("unroll") for (int f = 0; f < FM; ++f) SA[f] = psa[f][int64_t(KBI) * p.rows]; \
            SB = psb[KBI];                                                                       \
        }
#define GFG_STORE_STAGE(BUF)                                                                     \
        {                                                                                        \
            uint8_t* sA_ = smem + (BUF) * (A_BYTES + B_BYTES);                                   \
            uint8_t* sB_ = sA_ + A_BYTES;                                                        \
            _Pragma("unroll") for (int j = 0; j < A_LD; ++j)                                     \
                *reinterpret_cast<u32x4*>(sA_ + a_lds[j]) = ra[j];                               \
            _Pragma("unroll") for (int j = 0; j < B_LD; ++j)                                     \
                *reinterpret_cast<u32x4*>(sB_ + b_lds[j]) = rb[j];                               \
        }

        GFG_LOAD_STAGE(0)
        GFG_LOAD_SCALES(0, sa_cur, sb_cur)
        GFG_STORE_STAGE(0)
        __syncthreads();

        for (int kb = 0; kb < KB; ++kb) {
            const int buf = kb & 1;
            const bool more = kb + 1 < KB;
            if (more) {
                GFG_LOAD_STAGE(kb + 1)
                GFG_LOAD_SCALES(kb + 1, sa_nxt, sb_nxt)
            }
            const uint8_t* sA = smem + buf * (A_BYTES + B_BYTES);
            const uint8_t* sB = sA + A_BYTES;
            // A fragments: lane (l16, lq) holds row l16 of the 16-row tile, chunks lq and lq+4
            v8i af[FM];
#pragma unroll
            for (int f = 0; f < FM; ++f) {
                const int r = wm * 64 + f * 16 + l16;
                const u32x4 lo = *reinterpret_cast<const u32x4*>(sA + swz(r, lq));
                const u32x4 hi = *reinterpret_cast<const u32x4*>(sA + swz(r, lq + 4));
                af[f] = __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int x = 0; x < FN; ++x) {
                const int r = wn * WN + x * 16 + l16;
                const u32x4 lo = *reinterpret_cast<const u32x4*>(sB + swz(r, lq));
                const u32x4 hi = *reinterpret_cast<const u32x4*>(sB + swz(r, lq + 4));
                const v8i bf = __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int y = 0; y < FM; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        bf, af[y], acc[x][y], 0, 0, 0, sb_cur, 0, sa_cur[y]);
            }
            if (more) GFG_STORE_STAGE(buf ^ 1)
            __syncthreads();
            if (more) {
#pragma unroll
                for (int f = 0; f < FM; ++f) sa_cur[f] = sa_nxt[f];
                sb_cur = sb_nxt;
            }
        }
#undef GFG_LOAD_STAGE
#undef GFG_LOAD_SCALES
#undef GFG_STORE_STAGE

        // ---- epilogue: lane owns row (16y + l16), columns 16x + 4lq .. +3 -----
#pragma unroll
        for (int y = 0; y < FM; ++y) {
            const int64_t row = m0 + wm * 64 + y * 16 + l16;
            bool ok = row < mlimit;
            if (!MASKED && ok) ok = p.meta[row] == g;
            if (!ok) continue;
            OutT* drow = reinterpret_cast<OutT*>(d_reg) + row * p.N + n0 + wn * WN + 4 * lq;
#pragma unroll
            for (int x = 0; x < FN; ++x) {
                typedef OutT out4 __attribute__((ext_vector_type(4)));
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

template <int BN, bool MASKED, typename OutT>
int launch_t(const Params& p, unsigned n_cand_tiles, hipStream_t s) {
    DeviceInfo di;
    if (int rc = device_info(&di)) return rc;
    const unsigned NT = unsigned(p.N / BN);
    const unsigned upper = n_cand_tiles * NT;                 // valid tiles cannot exceed this
    unsigned grid = upper < unsigned(di.cus) ? upper : unsigned(di.cus);
    grid = (grid + NUM_XCD - 1) / NUM_XCD * NUM_XCD;          // whole slots on every XCD
    if (grid == 0) return GFG_OK;
    hipLaunchKernelGGL((grouped_fp8_gemm_kernel<BN, MASKED, OutT>), dim3(grid), dim3(NTHREADS), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GFG_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GFG_OK;
}

template <bool MASKED>
int dispatch(const Params& p, unsigned n_cand, int out_dtype, hipStream_t s) {
    const bool wide = p.N % 256 == 0;
    if (out_dtype == GFG_OUT_BF16)
        return wide ? launch_t<256, MASKED, __bf16>(p, n_cand, s) : launch_t<128, MASKED, __bf16>(p, n_cand, s);
    return wide ? launch_t<256, MASKED, _Float16>(p, n_cand, s) : launch_t<128, MASKED, _Float16>(p, n_cand, s);
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
    if (N > (int64_t(1) << 30) || K > (int64_t(1) << 30))
        return fail(GFG_EUNSUPPORTED, "%s: N or K too large", fn);
    return GFG_OK;
}

int group_m_default() { return 4; }

}  // namespace
}  // namespace gfg

using namespace gfg;

extern "C" int grouped_fp8_gemm_contiguous(const void* a, const uint8_t* a_scale, const void* b,
                                           const uint8_t* b_scale, const int32_t* grouped_layout, void* d,
                                           int64_t M, int64_t N, int64_t K, int32_t G, int32_t out_dtype,
                                           void* stream) {
    clear_error();
    const char* fn = "grouped_fp8_gemm_contiguous";
    if (M < 0) return fail(GFG_EINVAL, "%s: M=%lld is negative", fn, (long long)M);
    if (int rc = check_common(fn, a, a_scale, b, b_scale, grouped_layout, d, N, K, G, out_dtype)) return rc;
    if (M == 0) return GFG_OK;
    const int64_t n_cand = (M + BM - 1) / BM;
    if (n_cand > MT_MAX)
        return fail(GFG_EUNSUPPORTED, "%s: M=%lld exceeds %d rows", fn, (long long)M, MT_MAX * BM);
    Params p{};
    p.a = static_cast<const uint8_t*>(a);
    p.a_scale = a_scale;
    p.b = static_cast<const uint8_t*>(b);
    p.b_scale = b_scale;
    p.meta = grouped_layout;
    p.d = d;
    p.rows = M;
    p.N = int(N);
    p.K = int(K);
    p.G = G;
    p.n_cand = int(n_cand);
    p.mt_per_group = 0;
    p.group_m = group_m_default();
    return dispatch<false>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}

extern "C" int grouped_fp8_gemm_masked(const void* a, const uint8_t* a_scale, const void* b,
                                       const uint8_t* b_scale, const int32_t* masked_m, void* d, int32_t G,
                                       int64_t M_max, int64_t N, int64_t K, int32_t out_dtype, void* stream) {
    clear_error();
    const char* fn = "grouped_fp8_gemm_masked";
    if (M_max < 0) return fail(GFG_EINVAL, "%s: M_max=%lld is negative", fn, (long long)M_max);
    if (int rc = check_common(fn, a, a_scale, b, b_scale, masked_m, d, N, K, G, out_dtype)) return rc;
    if (M_max == 0) return GFG_OK;
    const int64_t per = (M_max + BM - 1) / BM;
    const int64_t n_cand = per * G;
    if (n_cand > MT_MAX)
        return fail(GFG_EUNSUPPORTED, "%s: G*ceil(M_max/128)=%lld exceeds %d", fn, (long long)n_cand, MT_MAX);
    Params p{};
    p.a = static_cast<const uint8_t*>(a);
    p.a_scale = a_scale;
    p.b = static_cast<const uint8_t*>(b);
    p.b_scale = b_scale;
    p.meta = masked_m;
    p.d = d;
    p.rows = M_max;
    p.N = int(N);
    p.K = int(K);
    p.G = G;
    p.n_cand = int(n_cand);
    p.mt_per_group = int(per);
    p.group_m = group_m_default();
    return dispatch<true>(p, unsigned(n_cand), out_dtype, static_cast<hipStream_t>(stream));
}
