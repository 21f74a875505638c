// Device-side per-token activation quantizer for gfx950 (MI355X).
//
// Produces the GEMM's A operand on the GPU: for every (1,128) block of a row
// (one token, 128 channels), the E8M0 scale 2^t with t the smallest integer
// such that 448 * 2^t >= max|x| over the block (rounded up, so |x / 2^t| never
// exceeds the E4M3 maximum 448), stored transposed as scale_t[K/128][M], and
// q = E4M3(x / 2^t) rounded to nearest, ties to even.  This is the operand
// preparation of the first reference page, "Grouped and Batched GEMM kernels
// with blockscaling matching DeepGEMM API" (sections "Summary" and "DeepGEMM
// conformance details"), done on the device instead of the host.
//
// Design: HBM-bound streaming.  A tile is 32 rows x 8 K-blocks (1024
// channels); a grid sized to what the device holds at once walks the tiles
// (grid stride), so no half-empty last round.  Sixteen lanes share one (1,128) block, eight
// consecutive channels per lane: one 16-byte (bf16) or two 16-byte (f32)
// loads per lane, eight blocks' loads in flight before the first is used, the
// block maximum by a 16-lane butterfly over the magnitude bits, the E4M3
// encoding by gfx950's packed FP8 conversion (round to nearest even; exact
// against the CPU definition on every E4M3 midpoint and subnormal), eight
// E4M3 bytes stored as one 8-byte store per lane (128 contiguous bytes per
// block).  The kernel moves little data per instruction, so the instruction
// count per element, not only the bytes, sets its speed.  The
// tile's scale bytes are collected in LDS and written as 32-byte runs along
// M, the fastest axis of the transposed scale tensor.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gfg.h"
#include "gfg_internal.h"

namespace gfg {
namespace {

constexpr int QT = 256;        // threads per workgroup
constexpr int QROWS = 32;      // rows per tile
constexpr int QKB = 8;         // K-blocks per tile
constexpr int QBLK = 128;      // channels per scale block
constexpr int QU = 8;          // blocks in flight per lane group

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Smallest integer t with 448 * 2^t >= a, for finite a > 0.  a = 1.f * 2^e and
// 448 = 1.75 * 2^8, so t = e - 8 when 1.f <= 1.75 (mantissa field <= 0x600000)
// and e - 7 otherwise; a subnormal a is normalized first.
__device__ __forceinline__ int ceil_e8m0_exp(float a) {
    uint32_t u = __float_as_uint(a);
    int e = int(u >> 23) - 127;
    uint32_t mant = u & 0x7FFFFFu;
    if (e == -127) {                                  // subnormal: a = mant * 2^-149
        // the leading one sits lz places below the implicit-bit position 23
        const int lz = __builtin_clz(mant) - 8;
        mant = (mant << lz) & 0x7FFFFFu;
        e = -126 - lz;
    }
    return mant <= 0x600000u ? e - 8 : e - 7;
}

template <typename InT>
__device__ __forceinline__ void load8(const InT* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
    v[0] = __uint_as_float(a[0]); v[1] = __uint_as_float(a[1]);
    v[2] = __uint_as_float(a[2]); v[3] = __uint_as_float(a[3]);
    v[4] = __uint_as_float(b[0]); v[5] = __uint_as_float(b[1]);
    v[6] = __uint_as_float(b[2]); v[7] = __uint_as_float(b[3]);
}

template <>
__device__ __forceinline__ void load8<__bf16>(const __bf16* p, float (&v)[8]) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);   // bf16 -> f32 is a 16-bit shift, exact
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(a[i] << 16);
        v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
}

// x [G][M][K] -> q [G][M][K] e4m3 bytes, scale_t [G][K/128][M] E8M0 bytes.
// Tiles: ceil(M/32) x ceil(KB/8) per group, G groups; any 1-D grid.
template <typename InT>
__global__ __launch_bounds__(QT) void quant_act_1x128_kernel(const InT* __restrict__ x, uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ scale_t, int M, int K, int G) {
    __shared__ uint8_t s_lds[QKB][QROWS];
    const int KB = K / QBLK;
    const int tm = (M + QROWS - 1) / QROWS, tk = (KB + QKB - 1) / QKB;
    const int64_t n_tiles = int64_t(tm) * tk * G;
    const int tid = threadIdx.x, lane16 = tid & 15, grp = tid >> 4;   // 16 blocks in flight per pass
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int g = int(tile / (int64_t(tm) * tk));
    const int rest = int(tile - int64_t(g) * tm * tk);
    const int m0 = (rest % tm) * QROWS, kb0 = (rest / tm) * QKB;
    const int64_t gofs = int64_t(g) * M * K;
    const int nkb = min(QKB, KB - kb0), nrows = min(QROWS, M - m0);

    // QU blocks per lane group per pass, all loads issued before any is used:
    // HBM latency is hidden by the loads in flight, not by occupancy alone
    for (int j0 = grp; j0 < QROWS * QKB; j0 += QU * (QT / 16)) {
        float v[QU][8];
        bool live[QU];
        int64_t off[QU];
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            const int j = j0 + u * (QT / 16);
            const int r = j % QROWS, kbc = j / QROWS;     // consecutive groups walk down the rows
            live[u] = j < QROWS * QKB && r < nrows && kbc < nkb;   // uniform across the 16 lanes
            // a block past the edge loads the workgroup's first block instead (always
            // present), so every load is issued unconditionally; only stores are predicated
            off[u] = gofs + (live[u] ? int64_t(m0 + r) * K + int64_t(kb0 + kbc) * QBLK
                                     : int64_t(m0) * K + int64_t(kb0) * QBLK) + lane16 * 8;
            load8<InT>(x + off[u], v[u]);
        }
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            const int j = j0 + u * (QT / 16);
            const int r = j % QROWS, kbc = j / QROWS;
            // max |x| as the integer max of the magnitude bits: for finite floats the
            // orders agree, and NaN / infinity (exponent field all ones) land above
            // every finite value, which flags the block
            uint32_t ab = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) ab = max(ab, __float_as_uint(v[u][i]) & 0x7FFFFFFFu);
#pragma unroll
            for (int w = 8; w >= 1; w >>= 1) ab = max(ab, uint32_t(__shfl_xor(int(ab), w, 16)));
            const bool bad = ab >= 0x7F800000u;
            // t = 0 for an all-zero block; t below the E8M0 range is raised to
            // -127, which still keeps |x / 2^t| <= 448
            int t = ab ? ceil_e8m0_exp(__uint_as_float(ab)) : 0;
            t = t < -127 ? -127 : t;
            uint32_t lo, hi;
            uint8_t sbyte;
            if (bad) {                                // no valid scale: E8M0 NaN, E4M3 NaN codes
                lo = hi = 0x7F7F7F7Fu;
                sbyte = 0xFF;
            } else {
                // x * 2^-t is exact (a power of two; results below the fp32
                // normal range are far below the smallest E4M3 step and encode
                // as zero); the hardware conversion rounds to nearest even
                const float inv = __builtin_ldexpf(1.0f, -t);
                float y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = v[u][i] * inv;
                lo = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false));
                lo = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], int(lo), true));
                hi = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false));
                hi = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], int(hi), true));
                sbyte = uint8_t(t + 127);
            }
            if (live[u]) {
                *reinterpret_cast<u32x2*>(q + off[u]) = u32x2{lo, hi};
                if (lane16 == 0) s_lds[kbc][r] = sbyte;
            }
        }
    }
    __syncthreads();
    // scale bytes: K-block kbc of rows m0.. is a run of nrows bytes along M
    uint8_t* sg = scale_t + int64_t(g) * KB * M;
    for (int i = tid; i < QROWS * QKB; i += QT) {
        const int r = i % QROWS, kbc = i / QROWS;
        if (r < nrows && kbc < nkb) sg[int64_t(kb0 + kbc) * M + m0 + r] = s_lds[kbc][r];
    }
    __syncthreads();   // the next tile reuses s_lds
  }
}

}  // namespace
}  // namespace gfg

using namespace gfg;

extern "C" int fp8_quantize_act_1x128_device(const void* x, int32_t in_dtype, int32_t G, int64_t M, int64_t K,
                                              uint8_t* q, uint8_t* scale_t, void* stream) {
    clear_error();
    const char* fn = "fp8_quantize_act_1x128_device";
    if (in_dtype != GFG_IN_F32 && in_dtype != GFG_IN_BF16)
        return fail(GFG_EINVAL, "%s: in_dtype %d is not GFG_IN_F32 or GFG_IN_BF16", fn, in_dtype);
    if (G <= 0 || G > 65535) return fail(GFG_EINVAL, "%s: G=%d outside [1, 65535]", fn, G);
    if (M < 0 || K < 0) return fail(GFG_EINVAL, "%s: M=%lld K=%lld must be >= 0", fn, (long long)M, (long long)K);
    if (M == 0 || K == 0) return GFG_OK;
    if (!x || !q || !scale_t) return fail(GFG_EINVAL, "%s: null pointer argument", fn);
    if (K % QBLK) return fail(GFG_EUNSUPPORTED, "%s: K=%lld must be a multiple of 128", fn, (long long)K);
    if (M > (int64_t(1) << 30) || K > (int64_t(1) << 30))
        return fail(GFG_EUNSUPPORTED, "%s: M=%lld or K=%lld above 2^30", fn, (long long)M, (long long)K);
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(q)) % 16)
        return fail(GFG_EINVAL, "%s: x and q must be 16-byte aligned", fn);
    const int64_t KB = K / QBLK;
    const int64_t tiles = (M + QROWS - 1) / QROWS * ((KB + QKB - 1) / QKB) * G;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(GFG_EHIP, "%s: device query failed", fn);
    // four resident 256-thread workgroups per CU (the kernel's occupancy)
    const unsigned grid = unsigned(tiles < int64_t(cus) * 4 ? tiles : int64_t(cus) * 4);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (in_dtype == GFG_IN_F32)
        hipLaunchKernelGGL(quant_act_1x128_kernel<float>, dim3(grid), dim3(QT), 0, s, static_cast<const float*>(x), q,
                           scale_t, int(M), int(K), int(G));
    else
        hipLaunchKernelGGL(quant_act_1x128_kernel<__bf16>, dim3(grid), dim3(QT), 0, s, static_cast<const __bf16*>(x), q,
                           scale_t, int(M), int(K), int(G));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GFG_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
    return GFG_OK;
}
