"""Grouped FP8 (E4M3) block-scaled GEMM for MI355X (gfx950).

A thin ctypes binding over ``libgfg.so`` (declared in ``include/gfg.h``):
argument marshalling only.  Every step of the GEMM and of the device
quantizer runs in the library's HIP kernels; the host quantizers run in the
library's C++ host code.  There is no fallback: if the library is missing or
fails to load, every call raises.

The operations are the two DeepGEMM-style grouped ops described on the first
reference page, "Grouped and Batched GEMM kernels with blockscaling matching
DeepGEMM API": a contiguous layout (``grouped_layout`` maps rows to experts,
-1 marks padding) and a masked layout (``[G, M_max, K]`` with ``masked_m``),
FP8 E4M3 operands with (1,128) activation and (128,128) weight E8M0 scales.
Both layouts also come as gemm1 of the expert MLP with its silu_mul epilogue
(third reference page, the MoE gemm1/gemm2 pull request, section "Changes"):
``out = silu(gate) * up`` with gate and up the two halves of ``A . B[g]^T``,
and as an MXFP8 GEMM (one E8M0 scale per 32 K elements of every row of A and B).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "GfgError", "load_library", "grouped_fp8_gemm_contiguous", "grouped_fp8_gemm_masked",
    "fp8_quantize_act_1x128", "fp8_quantize_weight_128x128", "fp8_quantize_act_masked",
    "fp8_quantize_act_1x128_device", "raw_contiguous", "raw_masked", "raw_quantize_act_device",
    "grouped_fp8_gemm_silu_mul_contiguous", "grouped_fp8_gemm_silu_mul_masked",
    "raw_silu_mul_contiguous", "raw_silu_mul_masked",
    "grouped_mxfp8_gemm_contiguous", "grouped_mxfp8_gemm_masked", "fp8_quantize_mx_1x32",
    "raw_mx_contiguous", "raw_mx_masked",
    "grouped_mxfp4_gemm_contiguous", "grouped_mxfp4_gemm_masked", "fp4_quantize_mx_1x32",
    "raw_mx4_contiguous", "raw_mx4_masked",
    "OUT_BF16", "OUT_F16", "IN_F32", "IN_BF16",
    "set_tile_order", "set_tile_shape", "set_grid_limit", "TILE_AUTO", "TILE_128x256", "TILE_256x256",
]

# GFG_LIBRARY names another build of the library to load (the host-sanitizer
# build of the CPU tests); by default the in-tree libgfg.so.
_LIB_PATH = os.environ.get("GFG_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgfg.so")
OUT_BF16, OUT_F16 = 0, 1
IN_F32, IN_BF16 = 0, 1
_STATUS = {0: "GFG_OK", 1: "GFG_EINVAL", 2: "GFG_EUNSUPPORTED", 3: "GFG_EHIP", 4: "GFG_ERANGE"}
_lib = None


class GfgError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{_STATUS.get(code, code)}: {message}")
        self.code = code


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libgfg.so (once).  Raises if it is missing: there is no fallback path."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing; build it with `python -m fp8_block_scaled_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i64, i32, u8p = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.grouped_fp8_gemm_contiguous.argtypes = [vp, u8p, vp, u8p, vp, vp, i64, i64, i64, i32, i32, vp]
    lib.grouped_fp8_gemm_contiguous.restype = ctypes.c_int
    lib.grouped_fp8_gemm_masked.argtypes = [vp, u8p, vp, u8p, vp, vp, i32, i64, i64, i64, i32, vp]
    lib.grouped_fp8_gemm_masked.restype = ctypes.c_int
    lib.grouped_fp8_gemm_silu_mul_contiguous.argtypes = [vp, u8p, vp, u8p, vp, vp, i64, i64, i64, i32, i32, vp]
    lib.grouped_fp8_gemm_silu_mul_contiguous.restype = ctypes.c_int
    lib.grouped_fp8_gemm_silu_mul_masked.argtypes = [vp, u8p, vp, u8p, vp, vp, i32, i64, i64, i64, i32, vp]
    lib.grouped_fp8_gemm_silu_mul_masked.restype = ctypes.c_int
    lib.grouped_mxfp8_gemm_contiguous.argtypes = [vp, u8p, vp, u8p, vp, vp, i64, i64, i64, i32, i32, vp]
    lib.grouped_mxfp8_gemm_contiguous.restype = ctypes.c_int
    lib.grouped_mxfp8_gemm_masked.argtypes = [vp, u8p, vp, u8p, vp, vp, i32, i64, i64, i64, i32, vp]
    lib.grouped_mxfp8_gemm_masked.restype = ctypes.c_int
    lib.fp8_quantize_mx_1x32.argtypes = [vp, i32, i64, i64, vp, vp]
    lib.grouped_mxfp4_gemm_contiguous.argtypes = [vp, u8p, vp, u8p, vp, vp, i64, i64, i64, i32, i32, vp]
    lib.grouped_mxfp4_gemm_contiguous.restype = ctypes.c_int
    lib.grouped_mxfp4_gemm_masked.argtypes = [vp, u8p, vp, u8p, vp, vp, i32, i64, i64, i64, i32, vp]
    lib.grouped_mxfp4_gemm_masked.restype = ctypes.c_int
    lib.fp4_quantize_mx_1x32.argtypes = [vp, i32, i64, i64, vp, vp]
    lib.grouped_mxfp4_gemm_silu_mul_contiguous.argtypes = [vp, u8p, vp, u8p, vp, vp, i64, i64, i64, i32, i32, vp]
    lib.grouped_mxfp4_gemm_silu_mul_contiguous.restype = ctypes.c_int
    lib.grouped_mxfp4_gemm_silu_mul_masked.argtypes = [vp, u8p, vp, u8p, vp, vp, i32, i64, i64, i64, i32, vp]
    lib.grouped_mxfp4_gemm_silu_mul_masked.restype = ctypes.c_int
    lib.fp4_quantize_mx_1x32.restype = ctypes.c_int
    lib.fp8_quantize_mx_1x32.restype = ctypes.c_int
    lib.fp8_quantize_act_1x128.argtypes = [vp, i64, i64, vp, vp]
    lib.fp8_quantize_act_1x128.restype = ctypes.c_int
    lib.fp8_quantize_weight_128x128.argtypes = [vp, i32, i64, i64, vp, vp]
    lib.fp8_quantize_weight_128x128.restype = ctypes.c_int
    lib.fp8_quantize_act_1x128_device.argtypes = [vp, i32, i32, i64, i64, vp, vp, vp]
    lib.fp8_quantize_act_1x128_device.restype = ctypes.c_int
    lib.grouped_fp8_last_error.argtypes = []
    lib.grouped_fp8_last_error.restype = ctypes.c_char_p
    lib.grouped_fp8_set_tile_order.argtypes = [i32, i32]
    lib.grouped_fp8_set_tile_order.restype = ctypes.c_int
    lib.grouped_fp8_set_tile_shape.argtypes = [i32]
    lib.grouped_fp8_set_tile_shape.restype = ctypes.c_int
    lib.grouped_fp8_set_grid_limit.argtypes = [i32]
    lib.grouped_fp8_set_grid_limit.restype = ctypes.c_int
    lib.gfg_device_peak.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32),
                                    ctypes.POINTER(ctypes.c_int32)]
    lib.gfg_device_peak.restype = ctypes.c_int
    lib.gfg_ceiling_mfma_operand_bytes.argtypes = []
    lib.gfg_ceiling_mfma_operand_bytes.restype = i64
    lib.gfg_ceiling_mfma.argtypes = [vp, i64, i32, vp, i64, ctypes.POINTER(ctypes.c_double), vp]
    lib.gfg_ceiling_mfma.restype = ctypes.c_int
    lib.gfg_ceiling_mfma_16x16x128.argtypes = [vp, i64, i32, vp, i64, ctypes.POINTER(ctypes.c_double), vp]
    lib.gfg_ceiling_mfma_16x16x128.restype = ctypes.c_int
    lib.gfg_ceiling_copy.argtypes = [vp, vp, i64, vp]
    lib.gfg_ceiling_copy.restype = ctypes.c_int
    lib.gfg_ceiling_read.argtypes = [vp, i64, vp, i64, vp]
    lib.gfg_ceiling_read.restype = ctypes.c_int
    lib.gfg_version.argtypes = []
    lib.gfg_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise GfgError(rc, load_library().grouped_fp8_last_error().decode())


# ------------------------------------------------------------------ launch settings
TILE_AUTO, TILE_128x256, TILE_256x256 = 0, 1, 2


def set_tile_order(num_xcd: int = 8, group_m: int = 0) -> None:
    """XCD split and grouped-M width of the tile order (process-wide)."""
    _check(load_library().grouped_fp8_set_tile_order(num_xcd, group_m))


def set_tile_shape(shape: int = TILE_AUTO) -> None:
    """Output tile of the plain FP8 GEMM calls: TILE_AUTO, TILE_128x256 or TILE_256x256."""
    _check(load_library().grouped_fp8_set_tile_shape(shape))


def set_grid_limit(max_workgroups: int = 0) -> None:
    """Cap the workgroups of a GEMM launch (0: one per CU)."""
    _check(load_library().grouped_fp8_set_grid_limit(max_workgroups))


# ------------------------------------------------------------------ measured ceilings
def device_peak() -> dict:
    """The dense FP8 MFMA peak from the device's CU count and maximum clock."""
    tf, cus, mhz = ctypes.c_double(0.0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load_library().gfg_device_peak(ctypes.byref(tf), ctypes.byref(cus), ctypes.byref(mhz)))
    return {"fp8_tflops": tf.value, "cus": cus.value, "max_sclk_mhz": mhz.value}


def ceiling_mfma_operand_bytes() -> int:
    return int(load_library().gfg_ceiling_mfma_operand_bytes())


def ceiling_mfma(operands, operand_bytes, iters, sink, sink_floats, stream=0) -> float:
    """Launch the scaled-MFMA ceiling kernel (device addresses); returns the
    FLOPs of the launch."""
    flops = ctypes.c_double(0.0)
    _check(load_library().gfg_ceiling_mfma(operands, operand_bytes, iters, sink, sink_floats,
                                           ctypes.byref(flops), stream))
    return flops.value


def ceiling_mfma_16x16x128(operands, operand_bytes, iters, sink, sink_floats, stream=0) -> float:
    """Launch the 16x16x128 scaled-MFMA ceiling kernel (device addresses);
    returns the FLOPs of the launch."""
    flops = ctypes.c_double(0.0)
    _check(load_library().gfg_ceiling_mfma_16x16x128(operands, operand_bytes, iters, sink, sink_floats,
                                                     ctypes.byref(flops), stream))
    return flops.value


def ceiling_copy(src, dst, nbytes, stream=0) -> None:
    """Launch the HBM copy ceiling kernel (device addresses)."""
    _check(load_library().gfg_ceiling_copy(src, dst, nbytes, stream))


def ceiling_read(src, nbytes, sink, sink_words, stream=0) -> None:
    """Launch the HBM read ceiling kernel (device addresses; sink: uint32 words,
    at least CUs * 64)."""
    _check(load_library().gfg_ceiling_read(src, nbytes, sink, sink_words, stream))


# ------------------------------------------------------------------ raw pointer calls
def raw_contiguous(a, a_scale, b, b_scale, grouped_layout, d, M, N, K, G, out_dtype, stream=0) -> int:
    """Call the C entry point with integer addresses; returns the status code."""
    return load_library().grouped_fp8_gemm_contiguous(a, a_scale, b, b_scale, grouped_layout, d,
                                                      M, N, K, G, out_dtype, stream)


def raw_masked(a, a_scale, b, b_scale, masked_m, d, G, M_max, N, K, out_dtype, stream=0) -> int:
    return load_library().grouped_fp8_gemm_masked(a, a_scale, b, b_scale, masked_m, d,
                                                  G, M_max, N, K, out_dtype, stream)


def raw_silu_mul_contiguous(a, a_scale, b, b_scale, grouped_layout, d, M, I, K, G, out_dtype, stream=0) -> int:
    return load_library().grouped_fp8_gemm_silu_mul_contiguous(a, a_scale, b, b_scale, grouped_layout, d,
                                                               M, I, K, G, out_dtype, stream)


def raw_silu_mul_masked(a, a_scale, b, b_scale, masked_m, d, G, M_max, I, K, out_dtype, stream=0) -> int:
    return load_library().grouped_fp8_gemm_silu_mul_masked(a, a_scale, b, b_scale, masked_m, d,
                                                           G, M_max, I, K, out_dtype, stream)


def raw_mx_contiguous(a, a_scale, b, b_scale, grouped_layout, d, M, N, K, G, out_dtype, stream=0) -> int:
    return load_library().grouped_mxfp8_gemm_contiguous(a, a_scale, b, b_scale, grouped_layout, d,
                                                        M, N, K, G, out_dtype, stream)


def raw_mx_masked(a, a_scale, b, b_scale, masked_m, d, G, M_max, N, K, out_dtype, stream=0) -> int:
    return load_library().grouped_mxfp8_gemm_masked(a, a_scale, b, b_scale, masked_m, d,
                                                    G, M_max, N, K, out_dtype, stream)


def raw_mx4_contiguous(a, a_scale, b, b_scale, grouped_layout, d, M, N, K, G, out_dtype, stream=0) -> int:
    """K counts E2M1 elements (rows are K/2 bytes)."""
    return load_library().grouped_mxfp4_gemm_contiguous(a, a_scale, b, b_scale, grouped_layout, d,
                                                        M, N, K, G, out_dtype, stream)


def raw_mx4_masked(a, a_scale, b, b_scale, masked_m, d, G, M_max, N, K, out_dtype, stream=0) -> int:
    return load_library().grouped_mxfp4_gemm_masked(a, a_scale, b, b_scale, masked_m, d,
                                                    G, M_max, N, K, out_dtype, stream)


def raw_mx4_silu_mul_contiguous(a, a_scale, b, b_scale, grouped_layout, d, M, I, K, G, out_dtype, stream=0) -> int:
    """a4w4 gemm1 + silu_mul; K counts E2M1 elements, B has 2*I rows."""
    return load_library().grouped_mxfp4_gemm_silu_mul_contiguous(a, a_scale, b, b_scale, grouped_layout, d,
                                                                 M, I, K, G, out_dtype, stream)


def raw_mx4_silu_mul_masked(a, a_scale, b, b_scale, masked_m, d, G, M_max, I, K, out_dtype, stream=0) -> int:
    return load_library().grouped_mxfp4_gemm_silu_mul_masked(a, a_scale, b, b_scale, masked_m, d,
                                                             G, M_max, I, K, out_dtype, stream)


def raw_quantize_act_device(x, in_dtype, G, M, K, q, scale_t, stream=0) -> int:
    return load_library().fp8_quantize_act_1x128_device(x, in_dtype, G, M, K, q, scale_t, stream)


# ------------------------------------------------------------------ torch-facing calls
def _torch():
    import torch
    return torch


def _dev_ptr(t, name, dtypes, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr()


def _out_code(d):
    torch = _torch()
    if d.dtype == torch.bfloat16:
        return OUT_BF16
    if d.dtype == torch.float16:
        return OUT_F16
    raise TypeError(f"d has dtype {d.dtype}; expected bfloat16 or float16")


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def grouped_fp8_gemm_contiguous(a, a_scale, b, b_scale, grouped_layout, d, stream=None):
    """D[rows of expert g] = A[rows] . B[g]^T on the GPU (asynchronous on ``stream``).

    a [M, K] e4m3 (torch.float8_e4m3fn or uint8 codes), a_scale [ceil(K/128), M] uint8 E8M0,
    b [G, N, K] e4m3, b_scale [G, ceil(N/128), ceil(K/128)] uint8, grouped_layout [M] int32,
    d [M, N] bfloat16/float16 (padding rows untouched).  All on the same GPU, contiguous.
    """
    torch = _torch()
    dev = d.device
    f8 = (torch.uint8, torch.float8_e4m3fn)
    M, K = a.shape
    G, N, Kb = b.shape
    if Kb != K or tuple(d.shape) != (M, N) or tuple(grouped_layout.shape) != (M,):
        raise ValueError("shape mismatch between a, b, grouped_layout and d")
    if tuple(a_scale.shape) != (-(-K // 128), M) or tuple(b_scale.shape) != (G, -(-N // 128), -(-K // 128)):
        raise ValueError("scale tensor shapes do not match the (1,128)/(128,128) layouts")
    _check(raw_contiguous(
        _dev_ptr(a, "a", f8, dev), _dev_ptr(a_scale, "a_scale", (torch.uint8,), dev),
        _dev_ptr(b, "b", f8, dev), _dev_ptr(b_scale, "b_scale", (torch.uint8,), dev),
        _dev_ptr(grouped_layout, "grouped_layout", (torch.int32,), dev),
        _dev_ptr(d, "d", (torch.bfloat16, torch.float16), dev),
        M, N, K, G, _out_code(d), _stream_handle(stream, dev)))
    return d


def grouped_fp8_gemm_masked(a, a_scale, b, b_scale, masked_m, d, stream=None):
    """D[g, m < masked_m[g]] = A[g, m] . B[g]^T on the GPU (asynchronous on ``stream``).

    a [G, M_max, K] e4m3, a_scale [G, ceil(K/128), M_max] uint8, b [G, N, K], b_scale
    [G, ceil(N/128), ceil(K/128)], masked_m [G] int32 (device), d [G, M_max, N].
    """
    torch = _torch()
    dev = d.device
    f8 = (torch.uint8, torch.float8_e4m3fn)
    G, Mmax, K = a.shape
    Gb, N, Kb = b.shape
    if Gb != G or Kb != K or tuple(d.shape) != (G, Mmax, N) or tuple(masked_m.shape) != (G,):
        raise ValueError("shape mismatch between a, b, masked_m and d")
    if tuple(a_scale.shape) != (G, -(-K // 128), Mmax) or tuple(b_scale.shape) != (G, -(-N // 128), -(-K // 128)):
        raise ValueError("scale tensor shapes do not match the (1,128)/(128,128) layouts")
    _check(raw_masked(
        _dev_ptr(a, "a", f8, dev), _dev_ptr(a_scale, "a_scale", (torch.uint8,), dev),
        _dev_ptr(b, "b", f8, dev), _dev_ptr(b_scale, "b_scale", (torch.uint8,), dev),
        _dev_ptr(masked_m, "masked_m", (torch.int32,), dev),
        _dev_ptr(d, "d", (torch.bfloat16, torch.float16), dev),
        G, Mmax, N, K, _out_code(d), _stream_handle(stream, dev)))
    return d


def grouped_fp8_gemm_silu_mul_contiguous(a, a_scale, b, b_scale, grouped_layout, d, stream=None):
    """gemm1 + silu_mul, contiguous layout: for rows of expert g, ``h = A[row] . B[g]^T``
    and ``d[row] = silu(h[:I]) * h[I:]`` (asynchronous on ``stream``).

    b [G, 2I, K] e4m3 (gate rows then up rows), b_scale [G, 2I/128, ceil(K/128)],
    d [M, I] bfloat16/float16; a, a_scale, grouped_layout as for the GEMM.
    """
    torch = _torch()
    dev = d.device
    f8 = (torch.uint8, torch.float8_e4m3fn)
    M, K = a.shape
    G, N2, Kb = b.shape
    if N2 % 2 or Kb != K or tuple(d.shape) != (M, N2 // 2) or tuple(grouped_layout.shape) != (M,):
        raise ValueError("shape mismatch between a, b [G, 2I, K], grouped_layout and d [M, I]")
    if tuple(a_scale.shape) != (-(-K // 128), M) or tuple(b_scale.shape) != (G, -(-N2 // 128), -(-K // 128)):
        raise ValueError("scale tensor shapes do not match the (1,128)/(128,128) layouts")
    _check(raw_silu_mul_contiguous(
        _dev_ptr(a, "a", f8, dev), _dev_ptr(a_scale, "a_scale", (torch.uint8,), dev),
        _dev_ptr(b, "b", f8, dev), _dev_ptr(b_scale, "b_scale", (torch.uint8,), dev),
        _dev_ptr(grouped_layout, "grouped_layout", (torch.int32,), dev),
        _dev_ptr(d, "d", (torch.bfloat16, torch.float16), dev),
        M, N2 // 2, K, G, _out_code(d), _stream_handle(stream, dev)))
    return d


def grouped_fp8_gemm_silu_mul_masked(a, a_scale, b, b_scale, masked_m, d, stream=None):
    """gemm1 + silu_mul, masked layout: rows m < masked_m[g] of group g get
    ``silu(h[:I]) * h[I:]`` with ``h = A[g, m] . B[g]^T``; d [G, M_max, I]."""
    torch = _torch()
    dev = d.device
    f8 = (torch.uint8, torch.float8_e4m3fn)
    G, Mmax, K = a.shape
    Gb, N2, Kb = b.shape
    if N2 % 2 or Gb != G or Kb != K or tuple(d.shape) != (G, Mmax, N2 // 2) or tuple(masked_m.shape) != (G,):
        raise ValueError("shape mismatch between a, b [G, 2I, K], masked_m and d [G, M_max, I]")
    if tuple(a_scale.shape) != (G, -(-K // 128), Mmax) or tuple(b_scale.shape) != (G, -(-N2 // 128), -(-K // 128)):
        raise ValueError("scale tensor shapes do not match the (1,128)/(128,128) layouts")
    _check(raw_silu_mul_masked(
        _dev_ptr(a, "a", f8, dev), _dev_ptr(a_scale, "a_scale", (torch.uint8,), dev),
        _dev_ptr(b, "b", f8, dev), _dev_ptr(b_scale, "b_scale", (torch.uint8,), dev),
        _dev_ptr(masked_m, "masked_m", (torch.int32,), dev),
        _dev_ptr(d, "d", (torch.bfloat16, torch.float16), dev),
        G, Mmax, N2 // 2, K, _out_code(d), _stream_handle(stream, dev)))
    return d


def grouped_mxfp8_gemm_contiguous(a, a_scale, b, b_scale, grouped_layout, d, stream=None):
    """MXFP8 contiguous grouped GEMM: a [M, K] e4m3 with a_scale [K/32, M], b [G, N, K] with
    b_scale [G, K/32, N] (one E8M0 byte per 32 K elements of a row), d [M, N]."""
    torch = _torch()
    dev = d.device
    f8 = (torch.uint8, torch.float8_e4m3fn)
    M, K = a.shape
    G, N, Kb = b.shape
    if Kb != K or tuple(d.shape) != (M, N) or tuple(grouped_layout.shape) != (M,):
        raise ValueError("shape mismatch between a, b, grouped_layout and d")
    if K % 32 or tuple(a_scale.shape) != (K // 32, M) or tuple(b_scale.shape) != (G, K // 32, N):
        raise ValueError("scale tensor shapes do not match the MX (1,32) layouts")
    _check(raw_mx_contiguous(
        _dev_ptr(a, "a", f8, dev), _dev_ptr(a_scale, "a_scale", (torch.uint8,), dev),
        _dev_ptr(b, "b", f8, dev), _dev_ptr(b_scale, "b_scale", (torch.uint8,), dev),
        _dev_ptr(grouped_layout, "grouped_layout", (torch.int32,), dev),
        _dev_ptr(d, "d", (torch.bfloat16, torch.float16), dev),
        M, N, K, G, _out_code(d), _stream_handle(stream, dev)))
    return d


def grouped_mxfp8_gemm_masked(a, a_scale, b, b_scale, masked_m, d, stream=None):
    """MXFP8 masked grouped GEMM: a [G, M_max, K] with a_scale [G, K/32, M_max], b [G, N, K]
    with b_scale [G, K/32, N], masked_m [G] int32 (device), d [G, M_max, N]."""
    torch = _torch()
    dev = d.device
    f8 = (torch.uint8, torch.float8_e4m3fn)
    G, Mmax, K = a.shape
    Gb, N, Kb = b.shape
    if Gb != G or Kb != K or tuple(d.shape) != (G, Mmax, N) or tuple(masked_m.shape) != (G,):
        raise ValueError("shape mismatch between a, b, masked_m and d")
    if K % 32 or tuple(a_scale.shape) != (G, K // 32, Mmax) or tuple(b_scale.shape) != (G, K // 32, N):
        raise ValueError("scale tensor shapes do not match the MX (1,32) layouts")
    _check(raw_mx_masked(
        _dev_ptr(a, "a", f8, dev), _dev_ptr(a_scale, "a_scale", (torch.uint8,), dev),
        _dev_ptr(b, "b", f8, dev), _dev_ptr(b_scale, "b_scale", (torch.uint8,), dev),
        _dev_ptr(masked_m, "masked_m", (torch.int32,), dev),
        _dev_ptr(d, "d", (torch.bfloat16, torch.float16), dev),
        G, Mmax, N, K, _out_code(d), _stream_handle(stream, dev)))
    return d


def fp8_quantize_act_1x128_device(x, q=None, scale_t=None, stream=None):
    """Per-token (1,128) ceil-E8M0 quantization on the GPU (asynchronous on ``stream``).

    x [M, K] or [G, M, K] float32 or bfloat16 on a GPU, K a multiple of 128 ->
    (q uint8 e4m3 codes of x's shape, scale_t uint8 [ceil(K/128), M] or
    [G, ceil(K/128), M]).  ``q`` and ``scale_t`` may be passed in (contiguous
    uint8 / float8_e4m3fn tensors of those shapes on x's device); otherwise
    they are allocated here with torch.
    """
    torch = _torch()
    dev = x.device
    if x.dim() not in (2, 3):
        raise ValueError("x must be [M, K] or [G, M, K]")
    G, M, K = (1, *x.shape) if x.dim() == 2 else tuple(x.shape)
    lead = () if x.dim() == 2 else (G,)
    if q is None:
        q = torch.empty(tuple(x.shape), dtype=torch.uint8, device=dev)
    if scale_t is None:
        scale_t = torch.empty(lead + (-(-K // 128), M), dtype=torch.uint8, device=dev)
    if tuple(q.shape) != tuple(x.shape) or tuple(scale_t.shape) != lead + (-(-K // 128), M):
        raise ValueError("q / scale_t shapes do not match x")
    code = IN_F32 if x.dtype == torch.float32 else IN_BF16
    _check(raw_quantize_act_device(
        _dev_ptr(x, "x", (torch.float32, torch.bfloat16), dev), code, G, M, K,
        _dev_ptr(q, "q", (torch.uint8, torch.float8_e4m3fn), dev),
        _dev_ptr(scale_t, "scale_t", (torch.uint8,), dev), _stream_handle(stream, dev)))
    return q, scale_t


# ------------------------------------------------------------------ host quantizers
def _host_f32(x, name):
    x = np.ascontiguousarray(np.asarray(x), dtype=np.float32)
    return x


def fp8_quantize_act_1x128(x):
    """x [M, K] float32 (host) -> (q [M, K] uint8 e4m3, scale_t [ceil(K/128), M] uint8)."""
    x = _host_f32(x, "x")
    M, K = x.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty((-(-K // 128), M), np.uint8)
    _check(load_library().fp8_quantize_act_1x128(x.ctypes.data, M, K, q.ctypes.data, s.ctypes.data))
    return q, s


def fp8_quantize_act_masked(x):
    """x [G, M_max, K] float32 -> (q [G, M_max, K], scale_t [G, ceil(K/128), M_max])."""
    x = _host_f32(x, "x")
    G, Mmax, K = x.shape
    q = np.empty((G, Mmax, K), np.uint8)
    s = np.empty((G, -(-K // 128), Mmax), np.uint8)
    lib = load_library()
    for g in range(G):
        _check(lib.fp8_quantize_act_1x128(x[g].ctypes.data, Mmax, K, q[g].ctypes.data, s[g].ctypes.data))
    return q, s


def fp8_quantize_weight_128x128(w):
    """w [G, N, K] float32 (host) -> (q [G, N, K] uint8, scale [G, ceil(N/128), ceil(K/128)] uint8)."""
    w = _host_f32(w, "w")
    G, N, K = w.shape
    q = np.empty((G, N, K), np.uint8)
    s = np.empty((G, -(-N // 128), -(-K // 128)), np.uint8)
    _check(load_library().fp8_quantize_weight_128x128(w.ctypes.data, G, N, K, q.ctypes.data, s.ctypes.data))
    return q, s


def fp8_quantize_mx_1x32(x):
    """MX quantization on the host: x [R, K] or [G, R, K] float32 ->
    (q of the same shape, uint8 e4m3; scale_t [K/32, R] or [G, K/32, R], uint8 E8M0)."""
    x = _host_f32(x, "x")
    squeeze = x.ndim == 2
    x3 = x[None] if squeeze else x
    G, R, K = x3.shape
    q = np.empty((G, R, K), np.uint8)
    s = np.empty((G, K // 32, R), np.uint8)
    _check(load_library().fp8_quantize_mx_1x32(x3.ctypes.data, G, R, K, q.ctypes.data, s.ctypes.data))
    return (q[0], s[0]) if squeeze else (q, s)


def fp4_quantize_mx_1x32(x):
    """MXFP4 quantization on the host: x [R, K] or [G, R, K] float32 (K a multiple
    of 128) -> (q [..., R, K/2] uint8, two E2M1 codes per byte, low nibble first;
    scale_t [..., K/32, R])."""
    x = _host_f32(x, "x")
    squeeze = x.ndim == 2
    x3 = x[None] if squeeze else x
    G, R, K = x3.shape
    q = np.empty((G, R, K // 2), np.uint8)
    s = np.empty((G, K // 32, R), np.uint8)
    _check(load_library().fp4_quantize_mx_1x32(x3.ctypes.data, G, R, K, q.ctypes.data, s.ctypes.data))
    return (q[0], s[0]) if squeeze else (q, s)


def grouped_mxfp4_gemm_contiguous(a, a_scale, b, b_scale, grouped_layout, d, stream=None):
    """MXFP4 contiguous grouped GEMM: a [M, K/2] uint8 (E2M1 pairs, low nibble first), a_scale
    [K/32, M], b [G, N, K/2], b_scale [G, K/32, N], d [M, N]."""
    torch = _torch()
    dev = d.device
    M, Kh = a.shape
    G, N, Kb = b.shape
    K = 2 * Kh
    if Kb != Kh or tuple(d.shape) != (M, N) or tuple(grouped_layout.shape) != (M,):
        raise ValueError("shape mismatch between a, b, grouped_layout and d")
    if tuple(a_scale.shape) != (K // 32, M) or tuple(b_scale.shape) != (G, K // 32, N):
        raise ValueError("scale tensor shapes do not match the MX (1,32) layouts")
    u8 = (torch.uint8,)
    _check(raw_mx4_contiguous(
        _dev_ptr(a, "a", u8, dev), _dev_ptr(a_scale, "a_scale", u8, dev), _dev_ptr(b, "b", u8, dev),
        _dev_ptr(b_scale, "b_scale", u8, dev), _dev_ptr(grouped_layout, "grouped_layout", (torch.int32,), dev),
        _dev_ptr(d, "d", (torch.bfloat16, torch.float16), dev), M, N, K, G, _out_code(d), _stream_handle(stream, dev)))
    return d


def grouped_mxfp4_gemm_masked(a, a_scale, b, b_scale, masked_m, d, stream=None):
    """MXFP4 masked grouped GEMM: a [G, M_max, K/2], a_scale [G, K/32, M_max], b [G, N, K/2],
    b_scale [G, K/32, N], masked_m [G] int32 (device), d [G, M_max, N]."""
    torch = _torch()
    dev = d.device
    G, Mmax, Kh = a.shape
    Gb, N, Kb = b.shape
    K = 2 * Kh
    if Gb != G or Kb != Kh or tuple(d.shape) != (G, Mmax, N) or tuple(masked_m.shape) != (G,):
        raise ValueError("shape mismatch between a, b, masked_m and d")
    if tuple(a_scale.shape) != (G, K // 32, Mmax) or tuple(b_scale.shape) != (G, K // 32, N):
        raise ValueError("scale tensor shapes do not match the MX (1,32) layouts")
    u8 = (torch.uint8,)
    _check(raw_mx4_masked(
        _dev_ptr(a, "a", u8, dev), _dev_ptr(a_scale, "a_scale", u8, dev), _dev_ptr(b, "b", u8, dev),
        _dev_ptr(b_scale, "b_scale", u8, dev), _dev_ptr(masked_m, "masked_m", (torch.int32,), dev),
        _dev_ptr(d, "d", (torch.bfloat16, torch.float16), dev), G, Mmax, N, K, _out_code(d),
        _stream_handle(stream, dev)))
    return d


def grouped_mxfp4_gemm_silu_mul_contiguous(a, a_scale, b, b_scale, grouped_layout, d, stream=None):
    """a4w4 gemm1 + silu_mul, contiguous layout: a [M, K/2] uint8 (E2M1 pairs), a_scale [K/32, M],
    b [G, 2I, K/2] (gate rows then up rows), b_scale [G, K/32, 2I], d [M, I]: for rows of
    expert g, ``h = A[row] . B[g]^T`` and ``d[row] = silu(h[:I]) * h[I:]``."""
    torch = _torch()
    dev = d.device
    M, Kh = a.shape
    G, N2, Kb = b.shape
    K = 2 * Kh
    if N2 % 2 or Kb != Kh or tuple(d.shape) != (M, N2 // 2) or tuple(grouped_layout.shape) != (M,):
        raise ValueError("shape mismatch between a, b [G, 2I, K/2], grouped_layout and d [M, I]")
    if tuple(a_scale.shape) != (K // 32, M) or tuple(b_scale.shape) != (G, K // 32, N2):
        raise ValueError("scale tensor shapes do not match the MX (1,32) layouts")
    u8 = (torch.uint8,)
    _check(raw_mx4_silu_mul_contiguous(
        _dev_ptr(a, "a", u8, dev), _dev_ptr(a_scale, "a_scale", u8, dev), _dev_ptr(b, "b", u8, dev),
        _dev_ptr(b_scale, "b_scale", u8, dev), _dev_ptr(grouped_layout, "grouped_layout", (torch.int32,), dev),
        _dev_ptr(d, "d", (torch.bfloat16, torch.float16), dev), M, N2 // 2, K, G, _out_code(d),
        _stream_handle(stream, dev)))
    return d


def grouped_mxfp4_gemm_silu_mul_masked(a, a_scale, b, b_scale, masked_m, d, stream=None):
    """a4w4 gemm1 + silu_mul, masked layout: a [G, M_max, K/2], a_scale [G, K/32, M_max],
    b [G, 2I, K/2], b_scale [G, K/32, 2I], masked_m [G] int32 (device), d [G, M_max, I]."""
    torch = _torch()
    dev = d.device
    G, Mmax, Kh = a.shape
    Gb, N2, Kb = b.shape
    K = 2 * Kh
    if N2 % 2 or Gb != G or Kb != Kh or tuple(d.shape) != (G, Mmax, N2 // 2) or tuple(masked_m.shape) != (G,):
        raise ValueError("shape mismatch between a, b [G, 2I, K/2], masked_m and d [G, M_max, I]")
    if tuple(a_scale.shape) != (G, K // 32, Mmax) or tuple(b_scale.shape) != (G, K // 32, N2):
        raise ValueError("scale tensor shapes do not match the MX (1,32) layouts")
    u8 = (torch.uint8,)
    _check(raw_mx4_silu_mul_masked(
        _dev_ptr(a, "a", u8, dev), _dev_ptr(a_scale, "a_scale", u8, dev), _dev_ptr(b, "b", u8, dev),
        _dev_ptr(b_scale, "b_scale", u8, dev), _dev_ptr(masked_m, "masked_m", (torch.int32,), dev),
        _dev_ptr(d, "d", (torch.bfloat16, torch.float16), dev), G, Mmax, N2 // 2, K, _out_code(d),
        _stream_handle(stream, dev)))
    return d
