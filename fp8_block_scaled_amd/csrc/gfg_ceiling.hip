// Measured ceilings for the benchmark (gfx950): the rates of the GEMM kernels'
// two scaled MFMAs with nothing else running, and the rates of a plain HBM copy and of a
// plain HBM read.  They are not part of the GEMM; the benchmark reports its
// kernels' fractions against these next to the published peaks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gfg.h"
#include "gfg_ceiling.h"
#include "gfg_device.h"
#include "gfg_internal.h"

namespace gfg {
namespace {

constexpr int CEIL_THREADS = 512;   // 8 wave64s per CU, as in the 128-row GEMM kernel
constexpr int CEIL_FRAGS = 12;      // fragments per wave: 8 A (two K halves), 4 B

// Each wave keeps twelve 32-byte-per-lane operand fragments loaded from
// `ops` (real E4M3 data, so the matrix pipes switch as in the GEMM) and issues
// a 128 x 64 wave tile's MFMA pattern of one 128-K step, 16
// v_mfma_scale_f32_32x32x64_f8f6f4 on eight accumulators, `iters` times.
// Scales are 127 (2^0).  Each thread writes one float (the sum of its
// accumulators) to `sink`, so that nothing is optimized away.
__global__ __launch_bounds__(CEIL_THREADS, 1) void mfma_ceiling_kernel(const uint8_t* __restrict__ ops, int iters,
                                                                       float* __restrict__ sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const v8i* src = reinterpret_cast<const v8i*>(ops) + size_t(wave) * CEIL_FRAGS * 64 + lane;
    v8i f[CEIL_FRAGS];
#pragma unroll
    for (int j = 0; j < CEIL_FRAGS; ++j) f[j] = src[j * 64];
    v16f acc[4][2];
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int x = 0; x < 2; ++x) acc[y][x] = v16f{};
    const int sc = 0x7f7f7f7f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int y = 0; y < 4; ++y)
#pragma unroll
                for (int x = 0; x < 2; ++x)
                    acc[y][x] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f[8 + 2 * h + x], f[4 * h + y],
                                                                                acc[y][x], 0, 0, 0, sc, 0, sc);
    }
    float s = 0.f;
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int i = 0; i < 16; ++i) s += acc[y][x][i];
    sink[size_t(blockIdx.x) * CEIL_THREADS + threadIdx.x] = s;
}

// The same operands, FLOPs and waves with v_mfma_scale_f32_16x16x128_f8f6f4
// (the instruction of both GEMM kernels): per iteration each wave issues 32 of
// them, A fragments 0..3 against B fragments 4..11, on 32 four-register
// accumulators.
__global__ __launch_bounds__(CEIL_THREADS, 1) void mfma16_ceiling_kernel(const uint8_t* __restrict__ ops, int iters,
                                                                         float* __restrict__ sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const v8i* src = reinterpret_cast<const v8i*>(ops) + size_t(wave) * CEIL_FRAGS * 64 + lane;
    v8i f[CEIL_FRAGS];
#pragma unroll
    for (int j = 0; j < CEIL_FRAGS; ++j) f[j] = src[j * 64];
    v4f acc[4][8];
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[y][x] = v4f{};
    const int sc = 0x7f7f7f7f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
            for (int x = 0; x < 8; ++x)
                acc[y][x] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f[4 + x], f[y], acc[y][x], 0, 0, 0, sc, 0,
                                                                             sc);
    }
    float s = 0.f;
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int x = 0; x < 8; ++x)
#pragma unroll
            for (int i = 0; i < 4; ++i) s += acc[y][x][i];
    sink[size_t(blockIdx.x) * CEIL_THREADS + threadIdx.x] = s;
}

// Grid-stride copy of n 16-byte words.
__global__ __launch_bounds__(256) void copy_ceiling_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                           int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// Grid-stride read of n 16-byte words, four loads in flight per thread; each
// wave writes the XOR of everything it read to sink[4 * block + wave].
__global__ __launch_bounds__(256) void read_ceiling_kernel(const u32x4* __restrict__ src, int64_t n,
                                                           uint32_t* __restrict__ sink) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        x ^= a ^ b ^ c ^ d;
    }
    for (; i < n; i += stride) x ^= __builtin_nontemporal_load(src + i);
    uint32_t v = x[0] ^ x[1] ^ x[2] ^ x[3];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) v ^= uint32_t(__shfl_xor(int(v), d, 64));
    if ((threadIdx.x & 63) == 0) sink[int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)] = v;
}

}  // namespace
}  // namespace gfg

using namespace gfg;

extern "C" {

GFG_API int gfg_device_peak(double* fp8_tflops, int32_t* cus, int32_t* max_sclk_mhz) {
    clear_error();
    if (!fp8_tflops || !cus || !max_sclk_mhz) return fail(GFG_EINVAL, "gfg_device_peak: null pointer argument");
    int dev = 0, n = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(GFG_EHIP, "gfg_device_peak: hipGetDevice failed");
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, dev) != hipSuccess || n <= 0 || khz <= 0)
        return fail(GFG_EHIP, "gfg_device_peak: hipDeviceGetAttribute failed");
    *cus = n;
    *max_sclk_mhz = khz / 1000;
    // dense FP8 MFMA: per CU and clock, 4 SIMDs x 2048 FLOP (one 16x16x128 FP8
    // MFMA, 65,536 FLOP, every 32 cycles per SIMD)
    *fp8_tflops = double(n) * 8192.0 * double(khz) * 1e3 / 1e12;
    return GFG_OK;
}

GFG_API int64_t gfg_ceiling_mfma_operand_bytes(void) {
    return int64_t(CEIL_THREADS / 64) * CEIL_FRAGS * 64 * 32;
}

GFG_API int gfg_ceiling_mfma(const uint8_t* operands, int64_t operand_bytes, int32_t iters, float* sink,
                             int64_t sink_floats, double* flops, void* stream) {
    clear_error();
    if (!operands || !sink || !flops) return fail(GFG_EINVAL, "gfg_ceiling_mfma: null pointer argument");
    if (operand_bytes < gfg_ceiling_mfma_operand_bytes())
        return fail(GFG_EINVAL, "gfg_ceiling_mfma: operands hold %lld bytes, need %lld", (long long)operand_bytes,
                    (long long)gfg_ceiling_mfma_operand_bytes());
    if (reinterpret_cast<uintptr_t>(operands) & 31)
        return fail(GFG_EINVAL, "gfg_ceiling_mfma: operands must be 32-byte aligned");
    if (iters < 1) return fail(GFG_EINVAL, "gfg_ceiling_mfma: iters=%d must be positive", iters);
    int cus = 0;
    if (int rc = device_cus(&cus)) return rc;
    if (sink_floats < int64_t(cus) * CEIL_THREADS)
        return fail(GFG_EINVAL, "gfg_ceiling_mfma: sink holds %lld floats, need %lld", (long long)sink_floats,
                    (long long)(int64_t(cus) * CEIL_THREADS));
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(cus), dim3(CEIL_THREADS), 0, static_cast<hipStream_t>(stream),
                       operands, int(iters), sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GFG_EHIP, "gfg_ceiling_mfma: launch failed: %s", hipGetErrorString(e));
    *flops = double(cus) * (CEIL_THREADS / 64) * double(iters) * 16.0 * (32.0 * 32.0 * 64.0 * 2.0);
    return GFG_OK;
}

GFG_API int gfg_ceiling_mfma_16x16x128(const uint8_t* operands, int64_t operand_bytes, int32_t iters, float* sink,
                                        int64_t sink_floats, double* flops, void* stream) {
    clear_error();
    if (!operands || !sink || !flops) return fail(GFG_EINVAL, "gfg_ceiling_mfma_16x16x128: null pointer argument");
    if (operand_bytes < gfg_ceiling_mfma_operand_bytes())
        return fail(GFG_EINVAL, "gfg_ceiling_mfma_16x16x128: operands hold %lld bytes, need %lld",
                    (long long)operand_bytes, (long long)gfg_ceiling_mfma_operand_bytes());
    if (reinterpret_cast<uintptr_t>(operands) & 31)
        return fail(GFG_EINVAL, "gfg_ceiling_mfma_16x16x128: operands must be 32-byte aligned");
    if (iters < 1) return fail(GFG_EINVAL, "gfg_ceiling_mfma_16x16x128: iters=%d must be positive", iters);
    int cus = 0;
    if (int rc = device_cus(&cus)) return rc;
    if (sink_floats < int64_t(cus) * CEIL_THREADS)
        return fail(GFG_EINVAL, "gfg_ceiling_mfma_16x16x128: sink holds %lld floats, need %lld",
                    (long long)sink_floats, (long long)(int64_t(cus) * CEIL_THREADS));
    hipLaunchKernelGGL(mfma16_ceiling_kernel, dim3(cus), dim3(CEIL_THREADS), 0, static_cast<hipStream_t>(stream),
                       operands, int(iters), sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(GFG_EHIP, "gfg_ceiling_mfma_16x16x128: launch failed: %s", hipGetErrorString(e));
    *flops = double(cus) * (CEIL_THREADS / 64) * double(iters) * 32.0 * (16.0 * 16.0 * 128.0 * 2.0);
    return GFG_OK;
}

GFG_API int gfg_ceiling_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    clear_error();
    if (!src || !dst) return fail(GFG_EINVAL, "gfg_ceiling_copy: null pointer argument");
    if (bytes <= 0 || bytes % 16 != 0)
        return fail(GFG_EINVAL, "gfg_ceiling_copy: bytes=%lld must be a positive multiple of 16", (long long)bytes);
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15)
        return fail(GFG_EINVAL, "gfg_ceiling_copy: src and dst must be 16-byte aligned");
    int cus = 0;
    if (int rc = device_cus(&cus)) return rc;
    hipLaunchKernelGGL(copy_ceiling_kernel, dim3(cus * 16), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GFG_EHIP, "gfg_ceiling_copy: launch failed: %s", hipGetErrorString(e));
    return GFG_OK;
}

GFG_API int gfg_ceiling_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words, void* stream) {
    clear_error();
    if (!src || !sink) return fail(GFG_EINVAL, "gfg_ceiling_read: null pointer argument");
    if (bytes <= 0 || bytes % 16 != 0)
        return fail(GFG_EINVAL, "gfg_ceiling_read: bytes=%lld must be a positive multiple of 16", (long long)bytes);
    if (reinterpret_cast<uintptr_t>(src) & 15) return fail(GFG_EINVAL, "gfg_ceiling_read: src must be 16-byte aligned");
    int cus = 0;
    if (int rc = device_cus(&cus)) return rc;
    if (sink_words < int64_t(cus) * 64)
        return fail(GFG_EINVAL, "gfg_ceiling_read: sink holds %lld words, need %lld", (long long)sink_words,
                    (long long)(int64_t(cus) * 64));
    hipLaunchKernelGGL(read_ceiling_kernel, dim3(cus * 16), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), bytes / 16, sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GFG_EHIP, "gfg_ceiling_read: launch failed: %s", hipGetErrorString(e));
    return GFG_OK;
}

}  // extern "C"
