// Host side of libgfg: error reporting and the CPU quantizers.
//
// The quantizers produce the operands the GEMM consumes, as the first
// reference page ("Grouped and Batched GEMM kernels with blockscaling
// matching DeepGEMM API", section "DeepGEMM conformance details") describes:
// E8M0 block scales rounded up to a power of two so that |x / scale| <= 448,
// extracted on the host as plain bytes.  Per-token (1,128) blocks for
// activations, stored transposed [ceil(K/128)][M]; (128,128) blocks for
// weights.  E4M3 values are rounded to nearest, ties to even.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "gfg.h"
#include "gfg_internal.h"

namespace gfg {

static thread_local std::string t_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    t_last_error = buf;
    return code;
}

void clear_error() { t_last_error.clear(); }

static std::atomic<int> g_num_xcd{8};
static std::atomic<int> g_group_m{0};
static std::atomic<int> g_tile_shape{0};
static std::atomic<int> g_grid_limit{0};
int locality_num_xcd() { return g_num_xcd.load(std::memory_order_relaxed); }
int locality_group_m() { return g_group_m.load(std::memory_order_relaxed); }
int tile_shape_choice() { return g_tile_shape.load(std::memory_order_relaxed); }
int grid_limit() { return g_grid_limit.load(std::memory_order_relaxed); }

namespace {

inline uint32_t f2u(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

// Smallest integer t with 448 * 2^t >= amax, read off the float's bit fields.
// amax = 1.f * 2^e; 448 = 1.75 * 2^8, so t = e - 8 when 1.f <= 1.75 (mantissa
// field <= 0x600000) and e - 7 otherwise.  Subnormal amax go through frexp.
// Returns false when t is outside the E8M0 range or amax is not finite.
bool ceil_e8m0(float amax, int* t) {
    if (!(amax >= 0.0f) || std::isinf(amax)) return false;
    if (amax == 0.0f) { *t = 0; return true; }
    uint32_t u = f2u(amax);
    int e = int(u >> 23) - 127;
    uint32_t mant = u & 0x7FFFFFu;
    if (e == -127) {                       // subnormal: normalize by hand
        int p;
        float f = std::frexp(amax, &p);    // amax = f * 2^p, f in [0.5, 1)
        uint32_t uf = f2u(f * 2.0f);       // 1.x in [1, 2)
        e = p - 1;
        mant = uf & 0x7FFFFFu;
    }
    int tt = (mant <= 0x600000u) ? e - 8 : e - 7;
    if (tt < -127 || tt > 127) return false;
    *t = tt;
    return true;
}

// MX scale exponent under the "Even" rounding of the third reference page
// ("flydsl mxfp4 a4w4 MoE: bring gemm1/gemm2 to parity with the HIP backend",
// section "Notes"): amax is first rounded to the element format's precision
// (mbits fraction bits: 3 for E4M3, 1 for E2M1; nearest, ties to even), then
// t = floor(log2(rounded amax)) - emax, emax being the exponent of the
// format's largest power of two (8 for E4M3, 2 for E2M1).
//
// Read off the float's bit fields: amax = 1.f * 2^e.  Rounding 1.f to mbits
// fraction bits reaches 2 exactly when the kept bits are all ones and the
// dropped part is at least half a step (a tie rounds up there, since all ones
// is odd), i.e. when the 23-bit fraction field is >= 2^23 - 2^(22 - mbits).
// That carry adds one to the exponent.  Subnormal amax are normalized first
// (their t lies far below the E8M0 range anyway).
bool mx_even_e8m0(float amax, int mbits, int emax, int* t) {
    if (!(amax >= 0.0f) || std::isinf(amax)) return false;
    if (amax == 0.0f) { *t = 0; return true; }
    uint32_t u = f2u(amax);
    int e = int(u >> 23) - 127;
    uint32_t mant = u & 0x7FFFFFu;
    if (e == -127) {                       // subnormal: normalize by hand
        int p;
        const float f = std::frexp(amax, &p);   // amax = f * 2^p, f in [0.5, 1)
        e = p - 1;
        mant = f2u(f * 2.0f) & 0x7FFFFFu;
    }
    const uint32_t carry_from = 0x800000u - (0x400000u >> mbits);
    const int tt = e + (mant >= carry_from ? 1 : 0) - emax;
    if (tt < -127 || tt > 127) return false;
    *t = tt;
    return true;
}

// Nearest E2M1 code of v (|v| <= 6): magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 are
// codes 0..7; a value on a midpoint takes the code with an even mantissa bit
// (so 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0,
// 5 -> 4.0).  Bit 3 is the sign, kept for zero.
inline uint8_t e2m1_rne(float v) {
    const float a = std::fabs(v);
    uint8_t c;
    if (a <= 0.25f) c = 0;
    else if (a < 0.75f) c = 1;
    else if (a <= 1.25f) c = 2;
    else if (a < 1.75f) c = 3;
    else if (a <= 2.5f) c = 4;
    else if (a < 3.5f) c = 5;
    else if (a <= 5.0f) c = 6;
    else c = 7;
    return uint8_t(c | (std::signbit(v) ? 8 : 0));
}

// Nearest E4M3FN code of v (|v| <= 448), ties to the even mantissa.
inline uint8_t e4m3_rne(float v) {
    uint32_t u = f2u(v);
    uint8_t sign = uint8_t((u >> 24) & 0x80u);
    u &= 0x7FFFFFFFu;
    float a;
    std::memcpy(&a, &u, 4);
    if (a < 0.015625f) {                   // below 2^-6: subnormal step 2^-9
        int m = int(std::nearbyint(a * 512.0f));   // exact scaling; RNE
        return uint8_t(sign | m);          // m == 8 is the smallest normal, code 0x08
    }
    int e = int(u >> 23) - 127;            // -6 .. 8
    uint32_t mant = u & 0x7FFFFFu;
    uint32_t r = mant >> 20, rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    if (r == 8) { r = 0; ++e; }
    return uint8_t(sign | uint8_t(((e + 7) << 3) | int(r)));
}

template <class F>
void parallel_for(int64_t n, F&& f) {
    unsigned hw = std::thread::hardware_concurrency();
    int64_t nt = std::min<int64_t>({int64_t(hw ? hw : 1), int64_t(16), n});
    if (nt <= 1) { for (int64_t i = 0; i < n; ++i) f(i); return; }
    std::vector<std::thread> th;
    for (int64_t w = 0; w < nt; ++w)
        th.emplace_back([&, w] { for (int64_t i = w; i < n; i += nt) f(i); });
    for (auto& t : th) t.join();
}

}  // namespace
}  // namespace gfg

using namespace gfg;

extern "C" const char* grouped_fp8_last_error(void) { return t_last_error.c_str(); }

extern "C" const char* gfg_version(void) { return "gfg 0.2 gfx950"; }

extern "C" int grouped_fp8_set_tile_order(int32_t num_xcd, int32_t group_m) {
    clear_error();
    if (num_xcd < 1 || num_xcd > 8)
        return fail(GFG_EINVAL, "grouped_fp8_set_tile_order: num_xcd=%d outside [1, 8]", num_xcd);
    if (group_m < 0 || group_m > 64)
        return fail(GFG_EINVAL, "grouped_fp8_set_tile_order: group_m=%d outside [0, 64]", group_m);
    g_num_xcd.store(num_xcd, std::memory_order_relaxed);
    g_group_m.store(group_m, std::memory_order_relaxed);
    return GFG_OK;
}

extern "C" int grouped_fp8_set_grid_limit(int32_t max_workgroups) {
    clear_error();
    if (max_workgroups < 0)
        return fail(GFG_EINVAL, "grouped_fp8_set_grid_limit: max_workgroups=%d is negative", max_workgroups);
    g_grid_limit.store(max_workgroups, std::memory_order_relaxed);
    return GFG_OK;
}

extern "C" int grouped_fp8_set_tile_shape(int32_t shape) {
    clear_error();
    if (shape < GFG_TILE_AUTO || shape > GFG_TILE_256x256)
        return fail(GFG_EINVAL, "grouped_fp8_set_tile_shape: shape=%d is not a GFG_TILE_* value", shape);
    g_tile_shape.store(shape, std::memory_order_relaxed);
    return GFG_OK;
}

extern "C" int fp8_quantize_act_1x128(const float* x, int64_t M, int64_t K,
                                      uint8_t* q, uint8_t* scale_t) {
    clear_error();
    if (M < 0 || K <= 0) return fail(GFG_EINVAL, "fp8_quantize_act_1x128: bad sizes M=%lld K=%lld",
                                    (long long)M, (long long)K);
    if (M == 0) return GFG_OK;
    if (!x || !q || !scale_t) return fail(GFG_EINVAL, "fp8_quantize_act_1x128: null pointer");
    const int64_t KB = (K + 127) / 128;
    std::vector<int> bad(size_t(M), 0);
    parallel_for(M, [&](int64_t m) {
        const float* row = x + m * K;
        for (int64_t kb = 0; kb < KB; ++kb) {
            const int64_t k0 = kb * 128, k1 = std::min(K, k0 + 128);
            float amax = 0.0f;
            bool nan = false;
            for (int64_t k = k0; k < k1; ++k) {
                amax = std::max(amax, std::fabs(row[k]));
                nan |= row[k] != row[k];
            }
            int t;
            if (nan || !ceil_e8m0(amax, &t)) { bad[size_t(m)] = 1; return; }
            scale_t[kb * M + m] = uint8_t(t + 127);
            for (int64_t k = k0; k < k1; ++k) q[m * K + k] = e4m3_rne(std::ldexp(row[k], -t));
        }
    });
    for (int64_t m = 0; m < M; ++m)
        if (bad[size_t(m)])
            return fail(GFG_ERANGE, "fp8_quantize_act_1x128: row %lld has a block outside the E8M0 range "
                        "or a non-finite value", (long long)m);
    return GFG_OK;
}

extern "C" int fp8_quantize_weight_128x128(const float* w, int32_t G, int64_t N, int64_t K,
                                           uint8_t* q, uint8_t* scale) {
    clear_error();
    if (G <= 0 || N <= 0 || K <= 0)
        return fail(GFG_EINVAL, "fp8_quantize_weight_128x128: bad sizes G=%d N=%lld K=%lld",
                    G, (long long)N, (long long)K);
    if (!w || !q || !scale) return fail(GFG_EINVAL, "fp8_quantize_weight_128x128: null pointer");
    const int64_t NB = (N + 127) / 128, KB = (K + 127) / 128;
    std::vector<int> bad(size_t(G * NB), 0);
    parallel_for(int64_t(G) * NB, [&](int64_t gn) {
        const int64_t g = gn / NB, nb = gn % NB;
        const int64_t n0 = nb * 128, n1 = std::min(N, n0 + 128);
        const float* wg = w + g * N * K;
        uint8_t* qg = q + g * N * K;
        for (int64_t kb = 0; kb < KB; ++kb) {
            const int64_t k0 = kb * 128, k1 = std::min(K, k0 + 128);
            float amax = 0.0f;
            bool nan = false;
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t k = k0; k < k1; ++k) {
                    amax = std::max(amax, std::fabs(wg[n * K + k]));
                    nan |= wg[n * K + k] != wg[n * K + k];
                }
            int t;
            if (nan || !ceil_e8m0(amax, &t)) { bad[size_t(gn)] = 1; return; }
            scale[(g * NB + nb) * KB + kb] = uint8_t(t + 127);
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t k = k0; k < k1; ++k) qg[n * K + k] = e4m3_rne(std::ldexp(wg[n * K + k], -t));
        }
    });
    for (int64_t i = 0; i < int64_t(G) * NB; ++i)
        if (bad[size_t(i)])
            return fail(GFG_ERANGE, "fp8_quantize_weight_128x128: block row %lld has a block outside the "
                        "E8M0 range or a non-finite value", (long long)i);
    return GFG_OK;
}

extern "C" int fp8_quantize_mx_1x32(const float* x, int32_t G, int64_t R, int64_t K, uint8_t* q,
                                    uint8_t* scale_t) {
    clear_error();
    const char* fn = "fp8_quantize_mx_1x32";
    if (G <= 0 || R < 0 || K <= 0)
        return fail(GFG_EINVAL, "%s: bad sizes G=%d R=%lld K=%lld", fn, G, (long long)R, (long long)K);
    if (K % 32) return fail(GFG_EUNSUPPORTED, "%s: K=%lld must be a multiple of 32", fn, (long long)K);
    if (R == 0) return GFG_OK;
    if (!x || !q || !scale_t) return fail(GFG_EINVAL, "%s: null pointer", fn);
    const int64_t KB = K / 32;
    std::vector<int> bad(size_t(G * R), 0);
    parallel_for(int64_t(G) * R, [&](int64_t gr) {
        const int64_t g = gr / R, r = gr % R;
        const float* row = x + gr * K;
        for (int64_t j = 0; j < KB; ++j) {
            float amax = 0.0f;
            bool nan = false;
            for (int64_t k = 32 * j; k < 32 * j + 32; ++k) {
                amax = std::max(amax, std::fabs(row[k]));
                nan |= row[k] != row[k];
            }
            int t;
            if (nan || !mx_even_e8m0(amax, 3, 8, &t)) { bad[size_t(gr)] = 1; return; }
            scale_t[(g * KB + j) * R + r] = uint8_t(t + 127);
            for (int64_t k = 32 * j; k < 32 * j + 32; ++k) {
                const float v = std::ldexp(row[k], -t);
                q[gr * K + k] = e4m3_rne(std::min(448.0f, std::max(-448.0f, v)));
            }
        }
    });
    for (int64_t i = 0; i < int64_t(G) * R; ++i)
        if (bad[size_t(i)])
            return fail(GFG_ERANGE, "%s: row %lld has a block outside the E8M0 range or a non-finite value", fn,
                        (long long)i);
    return GFG_OK;
}

extern "C" int fp4_quantize_mx_1x32(const float* x, int32_t G, int64_t R, int64_t K, uint8_t* q,
                                    uint8_t* scale_t) {
    clear_error();
    const char* fn = "fp4_quantize_mx_1x32";
    if (G <= 0 || R < 0 || K <= 0)
        return fail(GFG_EINVAL, "%s: bad sizes G=%d R=%lld K=%lld", fn, G, (long long)R, (long long)K);
    if (K % 128) return fail(GFG_EUNSUPPORTED, "%s: K=%lld must be a multiple of 128", fn, (long long)K);
    if (R == 0) return GFG_OK;
    if (!x || !q || !scale_t) return fail(GFG_EINVAL, "%s: null pointer", fn);
    const int64_t KB = K / 32;
    std::vector<int> bad(size_t(G * R), 0);
    parallel_for(int64_t(G) * R, [&](int64_t gr) {
        const int64_t g = gr / R, r = gr % R;
        const float* row = x + gr * K;
        uint8_t codes[128];
        for (int64_t q0 = 0; q0 < K; q0 += 128) {          // one 128-element group, 64 bytes out
            for (int j = 0; j < 4; ++j) {
                const int64_t k0 = q0 + 32 * j;
                float amax = 0.0f;
                bool nan = false;
                for (int i = 0; i < 32; ++i) {
                    amax = std::max(amax, std::fabs(row[k0 + i]));
                    nan |= row[k0 + i] != row[k0 + i];
                }
                int t;
                if (nan || !mx_even_e8m0(amax, 1, 2, &t)) { bad[size_t(gr)] = 1; return; }
                scale_t[(g * KB + k0 / 32) * R + r] = uint8_t(t + 127);
                for (int i = 0; i < 32; ++i) {
                    const float v = std::ldexp(row[k0 + i], -t);
                    codes[32 * j + i] = e2m1_rne(std::min(6.0f, std::max(-6.0f, v)));
                }
            }
            // two elements per byte, the lower index in the low nibble
            uint8_t* out = q + gr * (K / 2) + q0 / 2;
            for (int j = 0; j < 64; ++j) out[j] = uint8_t(codes[2 * j] | (codes[2 * j + 1] << 4));
        }
    });
    for (int64_t i = 0; i < int64_t(G) * R; ++i)
        if (bad[size_t(i)])
            return fail(GFG_ERANGE, "%s: row %lld has a block outside the E8M0 range or a non-finite value", fn,
                        (long long)i);
    return GFG_OK;
}
