/*
 * gfg_ceiling.h — measured ceilings of libgfg's benchmark (gfx950, MI355X).
 *
 * Not part of the grouped GEMM.  The benchmark times these kernels on the
 * same GPU, in the same process, and reports its GEMM's fraction of each next
 * to the published peaks (FP8 dense MFMA 5.0 PFLOP/s, HBM 8 TB/s).  The second
 * reference page ("[Kernel][MI350] Add cache-aware 8-wave BF16/FP16 GEMM",
 * section "Performance") quotes its throughputs against a socket power limit,
 * which is why a ceiling measured on the box at hand is reported too.
 *
 * All functions return GFG_OK (0) or a GFG_E* code from gfg.h, with the message
 * in grouped_fp8_last_error().  Launches are asynchronous on `stream` (a
 * hipStream_t; NULL is the default stream); nothing is allocated.
 */
#ifndef GFG_CEILING_H
#define GFG_CEILING_H

#include <stdint.h>

#include "gfg.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The dense FP8 MFMA peak derived from the current device's own CU count and
 * maximum shader clock (hipDeviceAttributeClockRate): CUs x 8192 FLOP per
 * clock (4 SIMDs, each one 16x16x128 FP8 MFMA of 65,536 FLOP per 32 cycles).
 * All outputs are host pointers; null: GFG_EINVAL; a HIP query failing:
 * GFG_EHIP.
 */
GFG_API int gfg_device_peak(double* fp8_tflops, int32_t* cus, int32_t* max_sclk_mhz);

/* Bytes of operand data gfg_ceiling_mfma reads (device memory, 32-byte aligned). */
GFG_API int64_t gfg_ceiling_mfma_operand_bytes(void);

/*
 * The scaled-MFMA ceiling: one workgroup of 8 wave64s per CU, each wave
 * issuing the MFMA pattern of a 128 x 64 wave tile's 128-K step
 * (16 v_mfma_scale_f32_32x32x64_f8f6f4 on 8 accumulators) `iters` times, on
 * register operands loaded once from `operands` (E4M3 bytes; pass real
 * quantized data, as the matrix pipes' power, and so the clock, depends on
 * it), with every scale 127 (2^0).  No memory traffic inside the loop.
 *   operands      device, gfg_ceiling_mfma_operand_bytes() bytes (operand_bytes
 *                 states the buffer's size; less: GFG_EINVAL)
 *   sink          device float[sink_floats], at least CUs * 512; one float per
 *                 thread is written (so the MFMAs are not optimized away)
 *   flops         host; receives the FLOPs one launch performs
 *                 (CUs * 8 * iters * 16 * 2 * 32 * 32 * 64)
 * iters < 1 or a null pointer: GFG_EINVAL.
 */
GFG_API int gfg_ceiling_mfma(const uint8_t* operands, int64_t operand_bytes, int32_t iters, float* sink,
                             int64_t sink_floats, double* flops, void* stream);

/*
 * The same measurement with v_mfma_scale_f32_16x16x128_f8f6f4, the
 * instruction of both GEMM kernels: the same operands (gfg_ceiling_mfma_operand_bytes()),
 * waves and FLOPs per iteration (each wave issues 32 of them on 32
 * four-register accumulators), the same sink and argument rules.  On the same
 * bytes this shape runs faster than 32x32x64 (measured on MI355X: about 4720
 * against 4150-4340 TFLOP/s on random E4M3 bytes).
 *   flops         host; receives CUs * 8 * iters * 32 * 2 * 16 * 16 * 128
 */
GFG_API int gfg_ceiling_mfma_16x16x128(const uint8_t* operands, int64_t operand_bytes, int32_t iters, float* sink,
                                        int64_t sink_floats, double* flops, void* stream);

/*
 * The HBM copy ceiling: dst[0, bytes) = src[0, bytes) with 16-byte loads and
 * stores (16 workgroups of 256 threads per CU, grid-stride).  Device pointers,
 * 16-byte aligned, not overlapping; bytes a positive multiple of 16, else
 * GFG_EINVAL.  A launch moves 2 * bytes through HBM when the buffers exceed the
 * caches.
 */
GFG_API int gfg_ceiling_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * The HBM read ceiling: reads src[0, bytes) with 16-byte non-temporal loads
 * (16 workgroups of 256 threads per CU, grid-stride, four loads in flight per
 * thread) and writes, per wave, the XOR of the 32-bit words it read to
 * sink[4 * workgroup + wave], so sink's XOR is the XOR of all of src's words.
 * src: device, 16-byte aligned; bytes a positive multiple of 16; sink: device
 * uint32_t[sink_words], at least CUs * 64 words; else GFG_EINVAL.  A launch
 * reads `bytes` from HBM when src exceeds the caches.  The ceiling for the
 * read-dominated launches (weights streamed once), where the copy's equal
 * mix of reads and writes is the wrong yardstick.
 */
GFG_API int gfg_ceiling_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GFG_CEILING_H */
