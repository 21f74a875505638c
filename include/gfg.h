/*
 * gfg.h — grouped FP8 (E4M3) block-scaled GEMM for MI355X (gfx950).
 *
 * C ABI of libgfg.so.  The operations are those of the first reference page,
 * "Grouped and Batched GEMM kernels with blockscaling matching DeepGEMM API"
 * (sections "Summary" and "DeepGEMM conformance details"):
 *
 *   D[rows of expert g] = A[rows] . B[g]^T          (contiguous layout)
 *   D[g, m, :]          = A[g, m, :] . B[g]^T       (masked layout, m < masked_m[g])
 *
 * with FP8 E4M3FN operands, one E8M0 scale per (1,128) block of A (per token,
 * per 128 channels, stored transposed as [ceil(K/128), M]) and one per
 * (128,128) block of B.  An E8M0 byte b means the scale 2^(b-127); b = 255
 * is NaN.  The product is exactly the product of the dequantized operands up
 * to fp32 summation order; D is rounded once to bf16 or f16 (nearest even).
 *
 * Conventions for every entry point:
 *  - Tensors are dense, row-major, contiguous, with the last named axis
 *    fastest.  "K-contiguous" ("nt"): A rows and B rows both run along K.
 *  - GEMM tensor pointers are DEVICE pointers owned by the caller.  The
 *    library never allocates, frees or synchronizes inside a GEMM call; the
 *    call is asynchronous on `stream` (a hipStream_t, NULL = null stream).
 *  - Quantizer pointers are HOST pointers owned by the caller; the quantizers
 *    are synchronous CPU functions.
 *  - Return value: GFG_OK (0) or an error code; no exceptions cross the ABI.
 *    grouped_fp8_last_error() returns a thread-local message for the last failure on
 *    the calling thread (valid until that thread's next call).
 *  - Argument checks (null pointers, sizes, enum values) happen on the host
 *    before anything is launched.  Device-resident metadata cannot be
 *    checked without a sync, so the kernels treat a grouped_layout entry
 *    outside [0, G) as padding and clamp masked_m[g] into [0, M_max].
 */
#ifndef GFG_H
#define GFG_H

#include <stdint.h>

#if defined(__GNUC__)
#define GFG_API __attribute__((visibility("default")))
#else
#define GFG_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum gfg_status {
    GFG_OK = 0,
    GFG_EINVAL = 1,       /* bad pointer, size or enum value                      */
    GFG_EUNSUPPORTED = 2, /* valid for the method, outside what the kernels tile  */
    GFG_EHIP = 3,         /* a HIP runtime call or kernel launch failed           */
    GFG_ERANGE = 4        /* quantizer: a block scale falls outside E8M0's range  */
};

enum gfg_out_dtype { GFG_OUT_BF16 = 0, GFG_OUT_F16 = 1 };
enum gfg_in_dtype { GFG_IN_F32 = 0, GFG_IN_BF16 = 1 };

/*
 * Contiguous grouped GEMM (the DeepGEMM-style m_grouped ... contiguous op).
 *
 *   a              [M][K]               e4m3 bytes
 *   a_scale        [ceil(K/128)][M]     E8M0 bytes, per token per 128-K block (transposed)
 *   b              [G][N][K]            e4m3 bytes
 *   b_scale        [G][ceil(N/128)][ceil(K/128)]  E8M0 bytes, K-block fastest
 *   grouped_layout [M]                  int32 expert id per row, -1 = padding
 *   d              [M][N]               bf16 or f16, written for rows whose
 *                                       grouped_layout is in [0, G); padding rows
 *                                       are left untouched
 *
 * Layout precondition: each expert's rows form runs that start on a multiple
 * of 128, padded with -1 up to the next multiple of 128, so every aligned
 * 128-row tile belongs to one expert (the expert of its first row; a tile
 * whose first row is padding is skipped).  A row whose entry differs from its
 * tile's expert is left untouched.
 *
 * Sizes: M >= 0 (M = 0 is a no-op), N > 0 and K > 0 multiples of 128 with
 * N <= 2^30 and K <= 2^23 (else GFG_EUNSUPPORTED), 1 <= G <= 65535, ceil(M/128) <= 4096 (else
 * GFG_EUNSUPPORTED).  The kernels address one expert's B and the A-scale
 * tensor with 32-bit byte offsets: N*K (bytes of one expert's B) and the
 * scale tensor's bytes (here ceil(K/128)*M; for the MX GEMMs below, one
 * byte per 32 K elements of every row) must stay below 2^32, else
 * GFG_EUNSUPPORTED.  These bounds hold for every entry point below.
 */
GFG_API int grouped_fp8_gemm_contiguous(const void* a, const uint8_t* a_scale,
                                const void* b, const uint8_t* b_scale,
                                const int32_t* grouped_layout, void* d,
                                int64_t M, int64_t N, int64_t K, int32_t G,
                                int32_t out_dtype, void* stream);

/*
 * Masked grouped GEMM (the DeepGEMM-style m_grouped ... masked op).
 *
 *   a         [G][M_max][K]               e4m3 bytes
 *   a_scale   [G][ceil(K/128)][M_max]     E8M0 bytes (the transposed layout, per group)
 *   b         [G][N][K]                   e4m3 bytes
 *   b_scale   [G][ceil(N/128)][ceil(K/128)]
 *   masked_m  [G]                         int32, DEVICE memory: rows computed per group
 *   d         [G][M_max][N]               rows m < masked_m[g] written, others untouched
 *
 * Sizes: M_max >= 0, N and K positive multiples of 128 (N <= 2^30, K <= 2^23),
 * 1 <= G <= 65535,
 * G * ceil(M_max/128) <= 4096 (else GFG_EUNSUPPORTED).
 */
GFG_API int grouped_fp8_gemm_masked(const void* a, const uint8_t* a_scale,
                            const void* b, const uint8_t* b_scale,
                            const int32_t* masked_m, void* d,
                            int32_t G, int64_t M_max, int64_t N, int64_t K,
                            int32_t out_dtype, void* stream);

/*
 * gemm1 of the expert MLP with its silu_mul epilogue (third reference page,
 * the pull request "flydsl mxfp4 a4w4 MoE: bring gemm1/gemm2 to parity with
 * the HIP backend", section "Changes", item gemm1), on the FP8 block-scaled
 * operands above.  Each expert's B holds 2*I rows: rows [0, I) are the gate
 * projection, rows [I, 2*I) the up projection.  For every computed row m:
 *
 *   h = A[m] . B[g]^T  (length 2*I, fp32),   out[m, j] = silu(h[j]) * h[I + j]
 *
 * with silu(x) = x / (1 + e^-x), e^-x taken by the hardware base-2
 * exponential and the division by the hardware reciprocal, then one rounding
 * to bf16 or f16.  Rows are chosen exactly as in the GEMMs above.
 *
 *   b        [G][2*I][K]                     e4m3 bytes (gate rows, then up rows)
 *   b_scale  [G][2*I/128][ceil(K/128)]       E8M0 bytes
 *   d        contiguous [M][I], masked [G][M_max][I]   bf16 or f16
 *   (a, a_scale, grouped_layout, masked_m as in the GEMMs)
 *
 * Sizes: as the GEMM with N = 2*I, and I a positive multiple of 128
 * (else GFG_EUNSUPPORTED; I <= 0 is GFG_EINVAL).  These entry points also
 * need M (M_max) a multiple of 4 and a_scale 4-byte aligned
 * (else GFG_EUNSUPPORTED).
 */
GFG_API int grouped_fp8_gemm_silu_mul_contiguous(const void* a, const uint8_t* a_scale,
                                         const void* b, const uint8_t* b_scale,
                                         const int32_t* grouped_layout, void* d,
                                         int64_t M, int64_t I, int64_t K, int32_t G,
                                         int32_t out_dtype, void* stream);
GFG_API int grouped_fp8_gemm_silu_mul_masked(const void* a, const uint8_t* a_scale,
                                     const void* b, const uint8_t* b_scale,
                                     const int32_t* masked_m, void* d,
                                     int32_t G, int64_t M_max, int64_t I, int64_t K,
                                     int32_t out_dtype, void* stream);

/*
 * MXFP8 grouped GEMM: the same two layouts on MX operands (third reference
 * page, "flydsl mxfp4 a4w4 MoE: bring gemm1/gemm2 to parity with the HIP
 * backend", section "Notes": MX kernels with E8M0 scales; here with E4M3
 * elements).  Every row of A and of B carries one E8M0 scale per 32
 * consecutive K elements; the hardware applies each one to its 32 products
 * inside the scaled MFMA.
 *
 *   a, b, grouped_layout / masked_m, d   as in the GEMMs above
 *   a_scale   contiguous [K/32][M], masked [G][K/32][M_max]   (transposed, per 32-wide K block)
 *   b_scale   [G][K/32][N]
 *
 * Sizes: as the GEMMs above, and N a multiple of 256, M (M_max) a multiple
 * of 4, a_scale and b_scale 4-byte aligned (else GFG_EUNSUPPORTED).
 */
GFG_API int grouped_mxfp8_gemm_contiguous(const void* a, const uint8_t* a_scale,
                                  const void* b, const uint8_t* b_scale,
                                  const int32_t* grouped_layout, void* d,
                                  int64_t M, int64_t N, int64_t K, int32_t G,
                                  int32_t out_dtype, void* stream);
GFG_API int grouped_mxfp8_gemm_masked(const void* a, const uint8_t* a_scale,
                              const void* b, const uint8_t* b_scale,
                              const int32_t* masked_m, void* d,
                              int32_t G, int64_t M_max, int64_t N, int64_t K,
                              int32_t out_dtype, void* stream);

/*
 * MX quantizer (CPU, synchronous) for the MXFP8 GEMM's operands:
 *   x [G][R][K] float -> q [G][R][K] e4m3, scale_t [G][K/32][R] E8M0
 * (A: G = 1, R = M; masked A: G groups of R = M_max; B: G experts of R = N).
 * Per row and 32-wide K block, the "Even" scale rounding of the third
 * reference page ("flydsl mxfp4 a4w4 MoE: bring gemm1/gemm2 to parity with
 * the HIP backend", section "Notes"): amax = max|x| is rounded to 3 fraction
 * bits (nearest, ties to even), t = floor(log2(rounded amax)) - 8 (t = 0 for
 * an all-zero block), scale byte t + 127, q = E4M3(clamp(x / 2^t, -448, 448))
 * nearest-even.  K must be a multiple of 32 (else GFG_EUNSUPPORTED);
 * GFG_ERANGE if t falls outside [-127, 127] or a value is not finite.
 */
GFG_API int fp8_quantize_mx_1x32(const float* x, int32_t G, int64_t R, int64_t K,
                         uint8_t* q, uint8_t* scale_t);

/*
 * MXFP4 grouped GEMM: the two layouts on E2M1 operands (the "mxfp4 (a4w4)"
 * element type of the third reference page, "flydsl mxfp4 a4w4 MoE: bring
 * gemm1/gemm2 to parity with the HIP backend", section "Summary"), one E8M0
 * scale per 32 K elements of every row, as in the MXFP8 GEMM.  K counts E2M1
 * elements; each row of a and b is K/2 bytes, two elements per byte with
 * the lower K index in the low nibble (as fp4_quantize_mx_1x32 writes).
 *
 *   a         contiguous [M][K/2], masked [G][M_max][K/2]      E2M1, two per byte
 *   b         [G][N][K/2]
 *   a_scale   contiguous [K/32][M], masked [G][K/32][M_max]
 *   b_scale   [G][K/32][N]
 *
 * Sizes: as the MXFP8 GEMM, with K a multiple of 256 (else GFG_EUNSUPPORTED).
 */
GFG_API int grouped_mxfp4_gemm_contiguous(const void* a, const uint8_t* a_scale,
                                  const void* b, const uint8_t* b_scale,
                                  const int32_t* grouped_layout, void* d,
                                  int64_t M, int64_t N, int64_t K, int32_t G,
                                  int32_t out_dtype, void* stream);
GFG_API int grouped_mxfp4_gemm_masked(const void* a, const uint8_t* a_scale,
                              const void* b, const uint8_t* b_scale,
                              const int32_t* masked_m, void* d,
                              int32_t G, int64_t M_max, int64_t N, int64_t K,
                              int32_t out_dtype, void* stream);

/*
 * a4w4 gemm1 with silu_mul: the gemm1 of the third reference page as the
 * page runs it ("mxfp4 (a4w4)" operands, section "Summary"; the silu_mul
 * epilogue, section "Changes", item gemm1).  The operands are those of the
 * MXFP4 GEMM above; the epilogue is that of grouped_fp8_gemm_silu_mul_*:
 * each expert's B holds 2*I rows, gate rows [0, I) then up rows [I, 2*I),
 * and for every computed row m
 *
 *   h = A[m] . B[g]^T  (length 2*I, fp32),   out[m, j] = silu(h[j]) * h[I + j]
 *
 *   a         contiguous [M][K/2], masked [G][M_max][K/2]      E2M1, two per byte
 *   b         [G][2*I][K/2]                                    (gate rows, then up rows)
 *   a_scale   contiguous [K/32][M], masked [G][K/32][M_max]    E8M0 bytes
 *   b_scale   [G][K/32][2*I]
 *   d         contiguous [M][I], masked [G][M_max][I]          bf16 or f16
 *   (grouped_layout, masked_m, out_dtype, stream as in the GEMMs)
 *
 * Sizes: K (E2M1 elements) a multiple of 256, I a positive multiple of 128,
 * M (M_max) a multiple of 4, both scale tensors 4-byte aligned (else
 * GFG_EUNSUPPORTED; I <= 0 or K <= 0 is GFG_EINVAL).  Rows are chosen as in
 * the GEMMs; other rows of d are left untouched.
 */
GFG_API int grouped_mxfp4_gemm_silu_mul_contiguous(const void* a, const uint8_t* a_scale,
                                           const void* b, const uint8_t* b_scale,
                                           const int32_t* grouped_layout, void* d,
                                           int64_t M, int64_t I, int64_t K, int32_t G,
                                           int32_t out_dtype, void* stream);
GFG_API int grouped_mxfp4_gemm_silu_mul_masked(const void* a, const uint8_t* a_scale,
                                       const void* b, const uint8_t* b_scale,
                                       const int32_t* masked_m, void* d,
                                       int32_t G, int64_t M_max, int64_t I, int64_t K,
                                       int32_t out_dtype, void* stream);

/*
 * MXFP4 quantizer (CPU, synchronous):
 *   x [G][R][K] float -> q [G][R][K/2] (two E2M1 codes per byte), scale_t [G][K/32][R] E8M0.
 * Per row and 32-wide K block, the "Even" scale rounding at E2M1's precision:
 * amax = max|x| rounded to 1 fraction bit (nearest, ties to even),
 * t = floor(log2(rounded amax)) - 2 (t = 0 for an all-zero block), scale
 * byte t + 127, code = E2M1(clamp(x / 2^t, -6, 6))
 * nearest-even (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 the sign).
 * Byte i of a row holds elements 2i (low nibble) and 2i + 1.  K must be a
 * multiple of 128 (else GFG_EUNSUPPORTED); GFG_ERANGE as fp8_quantize_mx_1x32.
 */
GFG_API int fp4_quantize_mx_1x32(const float* x, int32_t G, int64_t R, int64_t K,
                         uint8_t* q, uint8_t* scale_t);

/*
 * Host quantizers (CPU, synchronous), ceil-E8M0 scales and nearest-even E4M3:
 * for each block, t = the smallest integer with 448 * 2^t >= amax (t = 0 for
 * an all-zero block), scale byte = t + 127, q = E4M3(x / 2^t).  The rounding
 * up of the scale is what keeps |x / scale| <= 448 (first reference page,
 * section "DeepGEMM conformance details").  Ragged K (and N) are allowed:
 * a partial block uses only its elements.  Returns GFG_ERANGE if a block
 * needs t outside [-127, 127] or holds a non-finite value.
 *
 * fp8_quantize_act_1x128:    x [M][K] float -> q [M][K] e4m3, scale_t [ceil(K/128)][M]
 * fp8_quantize_weight_128x128: w [G][N][K] float -> q [G][N][K], scale [G][ceil(N/128)][ceil(K/128)]
 */
GFG_API int fp8_quantize_act_1x128(const float* x, int64_t M, int64_t K,
                           uint8_t* q, uint8_t* scale_t);
GFG_API int fp8_quantize_weight_128x128(const float* w, int32_t G, int64_t N, int64_t K,
                                uint8_t* q, uint8_t* scale);

/*
 * Device quantizer (GPU, asynchronous on `stream`): the activation quantizer
 * above, run on the device, producing the A operand of either GEMM layout.
 *
 *   x        [G][M][K]            float32 (in_dtype GFG_IN_F32) or bfloat16
 *                                 (GFG_IN_BF16), DEVICE memory, 16-byte aligned
 *   q        [G][M][K]            e4m3 bytes, DEVICE memory, 16-byte aligned
 *   scale_t  [G][K/128][M]        E8M0 bytes, DEVICE memory (the transposed
 *                                 per-token layout, per group)
 *
 * G = 1 gives the contiguous layout's a / a_scale; G groups of M = M_max rows
 * give the masked layout's.  Per (1,128) block: t = the smallest integer with
 * 448 * 2^t >= max|x| (t = 0 for an all-zero block), scale byte t + 127,
 * q = E4M3(x / 2^t) nearest-even, as in the host quantizer (first reference
 * page, sections "Summary" and "DeepGEMM conformance details").  Where the
 * host quantizer returns GFG_ERANGE the device one cannot stop; instead a
 * block with a NaN or infinity gets scale byte 255 (E8M0 NaN) and q = 0x7F
 * (E4M3 NaN) for all its elements, and a block so small that t < -127 gets
 * t = -127 (which still keeps |x / 2^t| <= 448).
 *
 * Sizes: G in [1, 65535]; M, K >= 0 (either 0 is a no-op); K a multiple of
 * 128, M <= 2^30, K <= 2^24 and G * ceil(M/32) * K/128 < 2^31 - 64 (else
 * GFG_EUNSUPPORTED).  The library allocates and synchronizes nothing.
 */
GFG_API int fp8_quantize_act_1x128_device(const void* x, int32_t in_dtype, int32_t G, int64_t M, int64_t K,
                                          uint8_t* q, uint8_t* scale_t, void* stream);

/*
 * Launch settings (process-wide, read at every GEMM call; not synchronized
 * with calls in flight on other threads).
 *
 * grouped_fp8_set_tile_order: the order in which a launch walks its
 * (M tile, N tile) work items.  The items are split into num_xcd contiguous
 * ranges, one per XCD (the hardware deals workgroup w to XCD w % 8, so with
 * num_xcd = 8 each range stays in one XCD's L2), and inside a range they
 * follow a grouped-M order group_m M tiles wide.  This is the locality mapping
 * of the second reference page ("[Kernel][MI350] Add cache-aware 8-wave
 * BF16/FP16 GEMM", section "Changes": XCD remap and grouped-M traversal with
 * a shortened final group, composed), made a run-time choice for its ablation
 * (section "Performance", second table).  Defaults: num_xcd = 8, group_m = 0
 * (each kernel's own width).  Every setting gives the same bytes: only the
 * order of the tiles changes.  num_xcd in [1, 8], group_m in [0, 64], else
 * GFG_EINVAL.
 *
 * grouped_fp8_set_tile_shape: the output tile of the plain FP8 GEMM calls
 * (grouped_fp8_gemm_contiguous / _masked).  GFG_TILE_AUTO picks 256 x 256
 * (where its requirements hold) when R256 * 1.6 <= R128, R being the rounds
 * of each shape's tiles over the CUs (ceil(tiles / CUs)), and either
 * R256 >= 2 or K >= 4096 (contiguous layout) or at least two 256 x 256 tiles
 * per CU (masked layout, counted from M_max: masked_m is device memory); for
 * the contiguous layout the rows must also average at least two 128-row tiles
 * per expert; else 128 x 256.  GFG_TILE_256x256 needs N a multiple of 256 and
 * at most 2^22, K/128 even, scale rows a multiple of 4 and scale_a 4-byte
 * aligned; a call that misses them then returns GFG_EUNSUPPORTED.  Other
 * values: GFG_EINVAL.  Results of the two tiles agree to the parity
 * tolerance; they are not promised to agree bit for bit.
 *
 * grouped_fp8_set_grid_limit: at most max_workgroups workgroups per GEMM
 * launch (0, the default: one per CU, fewer when there are fewer tiles).  The
 * grid is then rounded up to a multiple of num_xcd.  Each workgroup walks
 * more tiles; the results do not change.  Negative: GFG_EINVAL.
 */
enum gfg_tile_shape { GFG_TILE_AUTO = 0, GFG_TILE_128x256 = 1, GFG_TILE_256x256 = 2 };
GFG_API int grouped_fp8_set_tile_order(int32_t num_xcd, int32_t group_m);
GFG_API int grouped_fp8_set_tile_shape(int32_t shape);
GFG_API int grouped_fp8_set_grid_limit(int32_t max_workgroups);

/* Thread-local message describing the calling thread's last failure ("" if none). */
GFG_API const char* grouped_fp8_last_error(void);

/* Library version string. */
GFG_API const char* gfg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GFG_H */
