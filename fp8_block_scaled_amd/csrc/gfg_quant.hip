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
// Design: HBM-bound streaming, register-pipelined.  Sixteen lanes share one
// (1,128) block, eight consecutive channels per lane (one 16-byte bf16 or two
// 16-byte f32 loads), the block maximum by a 16-lane butterfly over the
// magnitude bits, the E4M3 encoding by gfx950's packed FP8 conversion (round
// to nearest even; exact against the CPU definition on every E4M3 midpoint and
// subnormal), eight code bytes per lane in one 8-byte store (128 contiguous
// bytes per block).  The blocks are walked as (group, 32-row stripe, K-block)
// "triples" of 32 blocks down the rows; a workgroup item is QU/2 consecutive
// triples, and a workgroup loads its next item into a second register set
// before it encodes the current one, so the next loads are in flight during
// the encoding and the stores.  Every load and store goes through a buffer
// descriptor that spans exactly the triple's valid rows: lanes of rows past
// the end of M fall outside the descriptor, where the hardware returns zeros
// for loads and drops stores.  With no predicated branches around the memory
// operations, the compiler's counter waits stay exact (wait for the item being
// encoded, not for the one in flight).  The input loads are non-temporal.  The scale byte goes straight to the
// transposed scale tensor from lane 0 of each group: the 32 rows of a triple
// are 32 consecutive bytes along M, written by one workgroup.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gfg.h"
#include "gfg_internal.h"

namespace gfg {
namespace {

constexpr int QT = 256;        // threads per workgroup: 16 lane groups
constexpr int QBLK = 128;      // channels per scale block
constexpr int QROWS = 32;      // rows per triple

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

// Raw buffer descriptor over [base, base + bytes); every field is wave-uniform
// and read-first-laned so the descriptor lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, uint32_t bytes) {
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    void* p = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, int(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000);
}

// Elements from a triple's first block to the end of its last valid row's
// block: the span its live lanes touch.  A row past the last valid one starts
// at or beyond the span (K >= 128), so its lanes fall outside the descriptor.
__device__ __forceinline__ uint32_t triple_span(uint32_t rows, uint32_t K) {
    return rows ? (rows - 1) * K + uint32_t(QBLK) : 0u;
}

// Cache-policy operand of the input loads: nt (bit 1 on gfx950).  The codes
// and scales are stored with the default policy, since the GEMM reads them next.
constexpr int kLoadNT = 2;

template <typename InT> struct InWords;      // 16-byte loads per lane per block
template <> struct InWords<__bf16> { static constexpr int n = 1; };
template <> struct InWords<float> { static constexpr int n = 2; };

// Position (g, st, kb) of a triple: group, 32-row stripe, K-block.
struct Cursor { int g, st, kb; };

template <int QU>
struct Item {
    int64_t base[QU / 2];    // element offset of (g, row st*32, block kb)
    int64_t sbase[QU / 2];   // scale byte offset of (g, kb, row st*32)
    uint32_t rows[QU / 2];   // valid rows of the triple; 0 past the last group
};

// The QU/2 triples from c on; past the last group, rows 0 (no access).
template <int QU>
__device__ __forceinline__ void locate(Item<QU>& it, Cursor c, int M, int K, int G, int KB, int tm) {
#pragma unroll
    for (int d = 0; d < QU / 2; ++d) {
        const bool ok = c.g < G;
        it.base[d] = ok ? (int64_t(c.g) * M + c.st * QROWS) * K + int64_t(c.kb) * QBLK : 0;
        it.sbase[d] = ok ? (int64_t(c.g) * KB + c.kb) * M + c.st * QROWS : 0;
        it.rows[d] = ok ? uint32_t(min(QROWS, M - c.st * QROWS)) : 0u;
        if (++c.kb == KB) { c.kb = 0; if (++c.st == tm) { c.st = 0; ++c.g; } }
    }
}

// c += delta, both in the (g, st, kb) mixed radix (delta.kb < KB, delta.st < tm).
__device__ __forceinline__ void advance(Cursor& c, const Cursor& delta, int KB, int tm) {
    c.kb += delta.kb;
    int carry = c.kb >= KB;
    if (carry) c.kb -= KB;
    c.st += delta.st + carry;
    carry = c.st >= tm;
    if (carry) c.st -= tm;
    c.g += delta.g + carry;
}

// Load an item: lane group grp takes row grp of each triple's first half
// (u even) and row 16 + grp of its second half (u odd).
template <typename InT, int QU>
__device__ __forceinline__ void fetch(u32x4 (&raw)[QU][InWords<InT>::n], const InT* x, const Item<QU>& it,
                                      uint32_t xo0, uint32_t xo1, uint32_t K) {
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int d = u >> 1;
        const auto r = uniform_rsrc(x + it.base[d], triple_span(it.rows[d], K) * uint32_t(sizeof(InT)));
        // non-temporal (cache policy nt): every input byte is read exactly once
#pragma unroll
        for (int w = 0; w < InWords<InT>::n; ++w)
            raw[u][w] = __builtin_amdgcn_raw_buffer_load_b128(r, ((u & 1) ? xo1 : xo0) + 16u * w, 0, kLoadNT);
    }
}

// Encode and store an item.
template <typename InT, int QU>
__device__ __forceinline__ void emit(const u32x4 (&raw)[QU][InWords<InT>::n], uint8_t* q, uint8_t* scale_t,
                                     const Item<QU>& it, uint32_t qo0, uint32_t qo1, uint32_t so0, uint32_t so1,
                                     uint32_t K) {
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int d = u >> 1;
        float v[8];
        if constexpr (InWords<InT>::n == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {                 // bf16 -> f32 is a 16-bit shift, exact
                v[2 * i] = __uint_as_float(raw[u][0][i] << 16);
                v[2 * i + 1] = __uint_as_float(raw[u][0][i] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = __uint_as_float(raw[u][0][i]);
                v[4 + i] = __uint_as_float(raw[u][1][i]);
            }
        }
        // max |x| as the integer max of the magnitude bits: for finite floats the
        // orders agree, and NaN / infinity (exponent field all ones) land above
        // every finite value, which flags the block
        uint32_t ab = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) ab = max(ab, __float_as_uint(v[i]) & 0x7FFFFFFFu);
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1) ab = max(ab, uint32_t(__shfl_xor(int(ab), w, 16)));
        const bool bad = ab >= 0x7F800000u;
        // t = 0 for an all-zero block; t below the E8M0 range is raised to
        // -127, which still keeps |x / 2^t| <= 448
        int t = ab ? ceil_e8m0_exp(__uint_as_float(ab)) : 0;
        t = t < -127 ? -127 : t;
        uint32_t lo, hi;
        uint8_t sbyte;
        if (bad) {                                    // no valid scale: E8M0 NaN, E4M3 NaN codes
            lo = hi = 0x7F7F7F7Fu;
            sbyte = 0xFF;
        } else {
            // x * 2^-t is exact (a power of two; results below the fp32
            // normal range are far below the smallest E4M3 step and encode
            // as zero); the hardware conversion rounds to nearest even
            const float inv = __builtin_ldexpf(1.0f, -t);
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = v[i] * inv;
            lo = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false));
            lo = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], int(lo), true));
            hi = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false));
            hi = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], int(hi), true));
            sbyte = uint8_t(t + 127);
        }
        const auto rq = uniform_rsrc(q + it.base[d], triple_span(it.rows[d], K));
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, rq, (u & 1) ? qo1 : qo0, 0, 0);
        const auto rs = uniform_rsrc(scale_t + it.sbase[d], it.rows[d]);
        __builtin_amdgcn_raw_buffer_store_b8(sbyte, rs, (u & 1) ? so1 : so0, 0, 0);
    }
}

// x [G][M][K] -> q [G][M][K] e4m3 bytes, scale_t [G][K/128][M] E8M0 bytes.
// Needs K <= 2^24 and G * ceil(M/32) * K/128 < 2^31; any 1-D grid of QT threads.
template <typename InT, int QU>
__global__ __launch_bounds__(QT) void quant_act_1x128_kernel(const InT* __restrict__ x, uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ scale_t, int M, int K, int G) {
    const int KB = K / QBLK;
    const int tm = (M + QROWS - 1) / QROWS;
    const int lane16 = threadIdx.x & 15, grp = threadIdx.x >> 4;
    // lane offsets inside a triple (element / code byte / scale byte); only
    // lane 0 of a group writes the scale byte, the others aim outside the span
    const uint32_t qo0 = uint32_t(grp) * uint32_t(K) + uint32_t(lane16 * 8), qo1 = qo0 + 16u * uint32_t(K);
    const uint32_t xo0 = qo0 * uint32_t(sizeof(InT)), xo1 = qo1 * uint32_t(sizeof(InT));
    const uint32_t so0 = lane16 == 0 ? uint32_t(grp) : 0x40000000u;
    const uint32_t so1 = lane16 == 0 ? uint32_t(grp + 16) : 0x40000000u;
    // first triple of this workgroup and the per-item step, as (g, st, kb)
    const int s0 = int(blockIdx.x) * (QU / 2), ds = int(gridDim.x) * (QU / 2);
    Cursor c{s0 / KB / tm, (s0 / KB) % tm, s0 % KB};
    const Cursor delta{ds / KB / tm, (ds / KB) % tm, ds % KB};
    u32x4 ra[QU][InWords<InT>::n], rb[QU][InWords<InT>::n];
    Item<QU> ia, ib;
    locate(ia, c, M, K, G, KB, tm);
    fetch<InT, QU>(ra, x, ia, xo0, xo1, uint32_t(K));
    // two register sets in turn: the next item's loads go out before the
    // current one is encoded; the walk ends once the cursor passes group G
    while (true) {
        advance(c, delta, KB, tm);
        locate(ib, c, M, K, G, KB, tm);
        fetch<InT, QU>(rb, x, ib, xo0, xo1, uint32_t(K));
        emit<InT, QU>(ra, q, scale_t, ia, qo0, qo1, so0, so1, uint32_t(K));
        if (c.g >= G) break;
        advance(c, delta, KB, tm);
        locate(ia, c, M, K, G, KB, tm);
        fetch<InT, QU>(ra, x, ia, xo0, xo1, uint32_t(K));
        emit<InT, QU>(rb, q, scale_t, ib, qo0, qo1, so0, so1, uint32_t(K));
        if (c.g >= G) break;
    }
}

// blocks per lane group per item: 8 (bf16) or 4 (f32), 128 bytes of input per lane
template <typename InT> constexpr int kQU = sizeof(InT) == 2 ? 8 : 4;

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
    if (M > (int64_t(1) << 30) || K > (int64_t(1) << 24))
        return fail(GFG_EUNSUPPORTED, "%s: M=%lld above 2^30 or K=%lld above 2^24", fn, (long long)M, (long long)K);
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(q)) % 16)
        return fail(GFG_EINVAL, "%s: x and q must be 16-byte aligned", fn);
    const int64_t KB = K / QBLK;
    const int64_t triples = (M + QROWS - 1) / QROWS * KB * G;
    if (triples >= (int64_t(1) << 31) - 64)
        return fail(GFG_EUNSUPPORTED, "%s: G * ceil(M/32) * K/128 = %lld is 2^31 or more", fn, (long long)triples);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(GFG_EHIP, "%s: device query failed", fn);
    // eight workgroups per CU, or one per item when there are fewer items
    const int qu = in_dtype == GFG_IN_F32 ? kQU<float> : kQU<__bf16>;
    const int64_t items = (triples + qu / 2 - 1) / (qu / 2);
    const unsigned grid = unsigned(items < int64_t(cus) * 8 ? items : int64_t(cus) * 8);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (in_dtype == GFG_IN_F32)
        hipLaunchKernelGGL((quant_act_1x128_kernel<float, kQU<float>>), dim3(grid), dim3(QT), 0, s,
                           static_cast<const float*>(x), q, scale_t, int(M), int(K), int(G));
    else
        hipLaunchKernelGGL((quant_act_1x128_kernel<__bf16, kQU<__bf16>>), dim3(grid), dim3(QT), 0, s,
                           static_cast<const __bf16*>(x), q, scale_t, int(M), int(K), int(G));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GFG_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
    return GFG_OK;
}
