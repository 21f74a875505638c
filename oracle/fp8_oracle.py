"""CPU oracle for the grouped FP8 (e4m3) block-scaled GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
constants with the HIP library; it is plain numpy in float64.

What it computes follows the first page of the reference material, the FlyDSL
pull request "Grouped and Batched GEMM kernels with blockscaling matching
DeepGEMM API" (sections "Summary" and "DeepGEMM conformance details"):

* activations carry one scale per token per 128 channels (a (1,128) block),
  stored transposed as ``[ceil(K/128), M]``;
* weights carry one scale per (128,128) block;
* scales are E8M0 (a bare power of two) rounded *up* (``ceil_to_ue8m0``) so
  that ``|x / scale|`` never exceeds the FP8 maximum 448;
* the contiguous op maps each row of A to an expert through
  ``grouped_layout`` (-1 marks padding rows); the masked op computes, for each
  group g, only rows ``m < masked_m[g]`` of a ``[G, M_max, K]`` batch;
* ``D[g] = A[g] . B[g]^T`` ("nt": K is the contiguous axis of both operands).

The scales are powers of two and are applied exactly, so the method reaches
"dequantize, then multiply" up to summation order; that plain definition is
what this module writes out (dequantize exactly in float64, multiply with a
float64 matmul).

Readings of points the pages leave open (each one is also listed in the
design notes of the repository):

* FP8 is OCP E4M3FN (bias 7, max 448, no infinity, NaN = S.1111.111); the
  page fixes the maximum as 448 but not the rounding.  Rounding is
  round-to-nearest, ties to the even code.
* ``ceil_to_ue8m0`` is taken exactly: the scale exponent t is the smallest
  integer with ``448 * 2**t >= amax``.  An all-zero block gets t = 0
  (byte 127); a block whose t falls outside the E8M0 range [-127, 127] is
  an error.
* ``calc_diff`` ("cosine-similarity-style normalized error") is
  ``1 - 2*sum(x*y) / sum(x*x + y*y)``.
* Rows that are padding (``grouped_layout`` outside [0, G)) or masked off
  (``m >= masked_m[g]``) keep whatever the output buffer held.
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0          # largest finite E4M3FN value (page 1, conformance section)
BLOCK = 128              # scale block edge along K (and along N for weights)


# ---------------------------------------------------------------- FP8 E4M3FN
def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3FN byte, in float64 (OCP FP8 definition).

    sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
    exponent 0 is subnormal: m * 2**-9.  exponent 15 with mantissa 7 is NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7 == 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = m * 2.0 ** -9
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def encode_e4m3_rne(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code to each float64 value, ties to the even code.

    Inputs must satisfy |x| <= 448 (the quantizer guarantees it).  The
    spacing of representable values is 2**(E-3) in the binade [2**E, 2**(E+1))
    for E >= -6 and 2**-9 below 2**-6 (subnormals); dividing by that power of
    two is exact, and ``np.rint`` rounds half to even, which is the even
    mantissa code.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("encode_e4m3_rne: non-finite input")
    if np.any(np.abs(x) > FP8_MAX):
        raise ValueError("encode_e4m3_rne: |x| > 448")
    a = np.abs(x)
    _, p = np.frexp(a)                          # a = f * 2**p, f in [0.5, 1)
    E = np.maximum(p - 1, -6)                   # binade exponent, subnormals share -6
    quantum = np.exp2(E - 3.0)
    r = np.rint(a / quantum) * quantum          # rounded magnitude, exact
    _, p2 = np.frexp(r)
    E2 = np.where(r >= 2.0 ** -6, p2 - 1, 0)
    mant = np.where(r >= 2.0 ** -6, r / np.exp2(E2.astype(np.float64)) * 8 - 8, r * 2.0 ** 9)
    expo = np.where(r >= 2.0 ** -6, E2 + 7, 0)
    code = (expo.astype(np.int64) << 3) | mant.astype(np.int64)
    code = code | np.where(np.signbit(x), 0x80, 0)
    if np.any((code & 0x7F) > 0x7E):
        raise ValueError("encode_e4m3_rne: rounded past 448")
    return code.astype(np.uint8)


# ---------------------------------------------------------------- E8M0 scale
def e8m0_ceil_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer t with 448 * 2**t >= amax (t = 0 where amax == 0).

    This is ``ceil(log2(amax / 448))`` evaluated exactly: start one below the
    frexp estimate and step up while the bound fails.  Every comparison is
    exact in float64 because 448 * 2**t is a power-of-two multiple of 448.
    """
    amax = np.asarray(amax, dtype=np.float64)
    if np.any(~np.isfinite(amax)) or np.any(amax < 0):
        raise ValueError("e8m0_ceil_exponent: amax must be finite and >= 0")
    _, p = np.frexp(np.where(amax > 0, amax, 1.0))
    t = p.astype(np.int64) - 10                 # 448 = 0.875 * 2**9, so t >= p - 10
    for _ in range(4):
        t = np.where(FP8_MAX * np.exp2(t.astype(np.float64)) < amax, t + 1, t)
    assert np.all(FP8_MAX * np.exp2(t.astype(np.float64)) >= amax)
    t = np.where(amax > 0, t, 0)
    if np.any(t < -127) or np.any(t > 127):
        raise ValueError("e8m0_ceil_exponent: scale outside the E8M0 range")
    return t


def e8m0_value(byte: np.ndarray) -> np.ndarray:
    """2**(b - 127) for an E8M0 byte b; 255 is NaN."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


# ---------------------------------------------------------------- quantizers
def _pad_to(x: np.ndarray, axis: int, mult: int) -> np.ndarray:
    n = x.shape[axis]
    extra = (-n) % mult
    if extra == 0:
        return x
    widths = [(0, 0)] * x.ndim
    widths[axis] = (0, extra)
    return np.pad(x, widths)


def quantize_act_1x128(x: np.ndarray):
    """Per-token (1,128) quantization of activations x[M, K] (float32).

    Returns ``(q [M, K] uint8 e4m3, scale_t [ceil(K/128), M] uint8 e8m0)``:
    for every row m and K-block kb, amax = max |x[m, 128kb : 128kb+128]|,
    t = e8m0 exponent of amax, byte = t + 127, q = RNE_e4m3(x / 2**t).
    The scale is stored transposed, [K-block, row], as the page specifies.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    M, K = x.shape
    kb = -(-K // BLOCK)
    xp = _pad_to(x, 1, BLOCK).reshape(M, kb, BLOCK)
    amax = np.abs(xp).max(axis=2)                       # [M, kb]
    t = e8m0_ceil_exponent(amax)                        # [M, kb]
    q = encode_e4m3_rne(xp / np.exp2(t[:, :, None].astype(np.float64)))
    q = q.reshape(M, kb * BLOCK)[:, :K]
    return np.ascontiguousarray(q), np.ascontiguousarray((t + 127).astype(np.uint8).T)


def quantize_weight_128x128(w: np.ndarray):
    """Per-block (128,128) quantization of weights w[G, N, K] (float32).

    Returns ``(q [G, N, K] uint8 e4m3, scale [G, ceil(N/128), ceil(K/128)] uint8)``.
    One scale per (group, N-block, K-block), K-block fastest in memory.
    """
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    G, N, K = w.shape
    nb, kb = -(-N // BLOCK), -(-K // BLOCK)
    wp = _pad_to(_pad_to(w, 1, BLOCK), 2, BLOCK).reshape(G, nb, BLOCK, kb, BLOCK)
    amax = np.abs(wp).max(axis=(2, 4))                  # [G, nb, kb]
    t = e8m0_ceil_exponent(amax)
    q = encode_e4m3_rne(wp / np.exp2(t[:, :, None, :, None].astype(np.float64)))
    q = q.reshape(G, nb * BLOCK, kb * BLOCK)[:, :N, :K]
    return np.ascontiguousarray(q), (t + 127).astype(np.uint8)


def dequantize_act(q: np.ndarray, scale_t: np.ndarray) -> np.ndarray:
    """A_dq[m, k] = e4m3(q[m, k]) * 2**(scale_t[k // 128, m] - 127), float64."""
    M, K = q.shape
    s = e8m0_value(scale_t).T                            # [M, kb]
    return decode_e4m3(q) * np.repeat(s, BLOCK, axis=1)[:, :K]


def dequantize_weight(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """B_dq[g, n, k] = e4m3(q[g, n, k]) * 2**(scale[g, n // 128, k // 128] - 127)."""
    G, N, K = q.shape
    s = e8m0_value(scale)
    s = np.repeat(np.repeat(s, BLOCK, axis=1), BLOCK, axis=2)[:, :N, :K]
    return decode_e4m3(q) * s


# ---------------------------------------------------------------- grouped GEMMs
def grouped_gemm_contiguous(q_a, scale_a, q_b, scale_b, grouped_layout, d_init=None):
    """Contiguous grouped GEMM, float64.

    For each expert g: ``D[rows with grouped_layout == g] = A_dq[rows] @ B_dq[g]^T``.
    Rows whose layout entry is outside [0, G) (padding, -1) keep ``d_init``
    (NaN when no initial buffer is given).
    """
    a = dequantize_act(q_a, scale_a)
    b = dequantize_weight(q_b, scale_b)
    layout = np.asarray(grouped_layout, dtype=np.int64)
    M, N = a.shape[0], b.shape[1]
    d = np.full((M, N), np.nan) if d_init is None else np.array(d_init, dtype=np.float64)
    for g in range(b.shape[0]):
        rows = np.nonzero(layout == g)[0]
        if rows.size:
            d[rows] = a[rows] @ b[g].T
    return d


def grouped_gemm_masked(q_a, scale_a, q_b, scale_b, masked_m, d_init=None):
    """Masked grouped GEMM, float64.

    q_a is [G, M_max, K] with scale_a [G, ceil(K/128), M_max]; for each group g
    only rows ``m < masked_m[g]`` (clamped to [0, M_max]) are computed:
    ``D[g, :mm] = A_dq[g, :mm] @ B_dq[g]^T``; other rows keep ``d_init``.
    """
    G, Mmax, K = q_a.shape
    b = dequantize_weight(q_b, scale_b)
    N = b.shape[1]
    d = np.full((G, Mmax, N), np.nan) if d_init is None else np.array(d_init, dtype=np.float64)
    for g in range(G):
        mm = int(min(max(int(masked_m[g]), 0), Mmax))
        if mm:
            a = dequantize_act(q_a[g, :mm], scale_a[g][:, :mm])
            d[g, :mm] = a @ b[g].T
    return d


def quantize_act_masked(x: np.ndarray):
    """Per-group (1,128) quantization of a masked batch x[G, M_max, K].

    Returns ``(q [G, M_max, K], scale_t [G, ceil(K/128), M_max])``: the page's
    transposed activation-scale layout, one such matrix per group.
    """
    qs, ss = zip(*(quantize_act_1x128(xg) for xg in np.asarray(x)))
    return np.stack(qs), np.stack(ss)


# ---------------------------------------------------------------- gemm1 + silu_mul
# The expert MLP's first GEMM projects each token to a gate half and an up
# half and multiplies silu(gate) into up (page 3, the RadeonFlow pull request
# "flydsl mxfp4 a4w4 MoE: bring gemm1/gemm2 to parity with the HIP backend",
# section "Changes", item gemm1: the silu_mul epilogue, with the exponential
# taken by the hardware base-2 exponential).  Readings of what the page leaves
# open: B[g] holds 2*I rows, rows [0, I) the gate projection and rows [I, 2*I)
# the up projection; silu(x) = x / (1 + e**-x); out = silu(gate) * up, an
# [M, I] (or [G, M_max, I]) result over the same valid rows as the GEMM.

def silu(x: np.ndarray) -> np.ndarray:
    """silu(x) = x / (1 + exp(-x)), float64 (x * logistic sigmoid of x)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def _silu_mul_rows(d: np.ndarray) -> np.ndarray:
    """[..., 2I] gate|up → [..., I] silu(gate) * up."""
    half = d.shape[-1] // 2
    return silu(d[..., :half]) * d[..., half:]


def grouped_gemm_silu_mul_contiguous(q_a, scale_a, q_b, scale_b, grouped_layout, out_init=None):
    """Contiguous gemm1 with silu_mul, float64.

    q_b is [G, 2I, K].  For each expert g and each row with
    ``grouped_layout == g``: ``h = A_dq[row] @ B_dq[g]^T`` (length 2I) and
    ``out[row] = silu(h[:I]) * h[I:]``.  Padding rows keep ``out_init`` (NaN
    when none is given).
    """
    d = grouped_gemm_contiguous(q_a, scale_a, q_b, scale_b, grouped_layout)
    M, half = d.shape[0], d.shape[1] // 2
    out = np.full((M, half), np.nan) if out_init is None else np.array(out_init, dtype=np.float64)
    layout = np.asarray(grouped_layout, dtype=np.int64)
    rows = np.nonzero((layout >= 0) & (layout < q_b.shape[0]))[0]
    out[rows] = _silu_mul_rows(d[rows])
    return out


def grouped_gemm_silu_mul_masked(q_a, scale_a, q_b, scale_b, masked_m, out_init=None):
    """Masked gemm1 with silu_mul, float64: rows ``m < masked_m[g]`` of group g
    get ``silu(h[:I]) * h[I:]`` with ``h = A_dq[g, m] @ B_dq[g]^T``; other rows
    keep ``out_init``."""
    d = grouped_gemm_masked(q_a, scale_a, q_b, scale_b, masked_m)
    G, Mmax, half = d.shape[0], d.shape[1], d.shape[2] // 2
    out = np.full((G, Mmax, half), np.nan) if out_init is None else np.array(out_init, dtype=np.float64)
    for g in range(G):
        mm = int(min(max(int(masked_m[g]), 0), Mmax))
        if mm:
            out[g, :mm] = _silu_mul_rows(d[g, :mm])
    return out


# ---------------------------------------------------------------- MXFP8 (1 x 32 blocks)
# The MX variant (third reference page, "[RadeonFlow] flydsl mxfp4 a4w4 MoE:
# bring gemm1/gemm2 to parity with the HIP backend": the MoE kernels there are
# "mxfp4 (a4w4)" with E8M0 scales under a rounding the section "Notes" calls
# "Even").  MX formats share one E8M0 scale per 32 consecutive elements along
# K, for activations and weights alike.  Readings of what the page leaves
# open, for the FP8 (E4M3) element type:
#   * "Even" is a rounding of the scale: the block's amax is first rounded to
#     the element format's precision (E4M3: 3 fraction bits), to nearest with
#     ties to even, and the scale exponent is then
#     t = floor(log2(rounded amax)) - 8, where 8 is the exponent of E4M3's
#     largest power of two (256).  Without the rounding step this is the plain
#     floor rule; with it, a block whose amax is within half an E4M3 step of
#     the next power of two takes the larger scale;
#   * elements are x / 2**t rounded to nearest, ties to even, and clamped to
#     +-448 (scaled values in (448, 496) saturate);
#   * an all-zero block gets t = 0 (byte 127); t outside [-127, 127] is an error;
#   * both scale tensors are stored transposed, one row of bytes per 32-wide
#     K block: ``[K/32, M]`` for A, ``[G, K/32, N]`` for B.

MX_BLOCK = 32
MX_EMAX = 8                # E4M3: largest power of two is 2**8
MX_MBITS = 3               # E4M3 fraction bits


def _even_scale_exponent(amax: np.ndarray, mbits: int, emax: int, name: str) -> np.ndarray:
    """t = floor(log2(RNE(amax at mbits fraction bits))) - emax, exactly; 0 where amax == 0.

    amax = f * 2**p with f in [0.5, 1) (frexp), so its significand is 2f in
    [1, 2) and floor(log2(amax)) = p - 1.  2f * 2**mbits is exact in float64;
    rounding it to an integer (numpy's rint: nearest, ties to even) rounds the
    significand to mbits fraction bits, and the result reaches 2 * 2**mbits
    exactly when the rounding carries into the next power of two.
    """
    amax = np.asarray(amax, dtype=np.float64)
    if np.any(~np.isfinite(amax)) or np.any(amax < 0):
        raise ValueError(f"{name}: amax must be finite and >= 0")
    f, p = np.frexp(np.where(amax > 0, amax, 1.0))
    carry = np.rint(2.0 * f * 2.0 ** mbits) >= 2.0 ** (mbits + 1)
    t = np.where(amax > 0, p.astype(np.int64) - 1 + carry.astype(np.int64) - emax, 0)
    if np.any(t < -127) or np.any(t > 127):
        raise ValueError(f"{name}: scale outside the E8M0 range")
    return t


def mx_exponent(amax: np.ndarray) -> np.ndarray:
    """E4M3 MX scale exponent under the "Even" rule (3 fraction bits, emax 8)."""
    return _even_scale_exponent(amax, MX_MBITS, MX_EMAX, "mx_exponent")


def quantize_mx_1x32(x: np.ndarray):
    """MX quantization of x[..., R, K] along K (K a multiple of 32).

    Returns ``(q [..., R, K] uint8 e4m3, scale_t [..., K/32, R] uint8 e8m0)``
    with, per row r and 32-wide block j: t = mx_exponent(max |block|),
    q = RNE_e4m3(clamp(x / 2**t, -448, 448)), byte = t + 127.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    *lead, R, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("quantize_mx_1x32: K must be a multiple of 32")
    xb = x.reshape(*lead, R, K // MX_BLOCK, MX_BLOCK)
    t = mx_exponent(np.abs(xb).max(axis=-1))                         # [..., R, K/32]
    v = np.clip(xb / np.exp2(t[..., None].astype(np.float64)), -FP8_MAX, FP8_MAX)
    q = encode_e4m3_rne(v).reshape(*lead, R, K)
    st = np.swapaxes((t + 127).astype(np.uint8), -1, -2)             # [..., K/32, R]
    return np.ascontiguousarray(q), np.ascontiguousarray(st)


def dequantize_mx(q: np.ndarray, scale_t: np.ndarray) -> np.ndarray:
    """X_dq[..., r, k] = e4m3(q[..., r, k]) * 2**(scale_t[..., k // 32, r] - 127)."""
    s = np.swapaxes(e8m0_value(scale_t), -1, -2)                     # [..., R, K/32]
    return decode_e4m3(q) * np.repeat(s, MX_BLOCK, axis=-1)


def grouped_gemm_mx_contiguous(q_a, scale_a, q_b, scale_b, grouped_layout, d_init=None):
    """Contiguous grouped GEMM on MX operands, float64: A [M, K] with scale_a
    [K/32, M], B [G, N, K] with scale_b [G, K/32, N];
    ``D[rows with grouped_layout == g] = A_dq[rows] @ B_dq[g]^T``, other rows
    keep ``d_init``."""
    a = dequantize_mx(q_a, scale_a)
    b = dequantize_mx(q_b, scale_b)
    layout = np.asarray(grouped_layout, dtype=np.int64)
    M, N = a.shape[0], b.shape[1]
    d = np.full((M, N), np.nan) if d_init is None else np.array(d_init, dtype=np.float64)
    for g in range(b.shape[0]):
        rows = np.nonzero(layout == g)[0]
        if rows.size:
            d[rows] = a[rows] @ b[g].T
    return d


def grouped_gemm_mx_masked(q_a, scale_a, q_b, scale_b, masked_m, d_init=None):
    """Masked grouped GEMM on MX operands: A [G, M_max, K] with scale_a
    [G, K/32, M_max]; rows m < masked_m[g] computed, others keep ``d_init``."""
    G, Mmax, K = q_a.shape
    b = dequantize_mx(q_b, scale_b)
    N = b.shape[1]
    d = np.full((G, Mmax, N), np.nan) if d_init is None else np.array(d_init, dtype=np.float64)
    for g in range(G):
        mm = int(min(max(int(masked_m[g]), 0), Mmax))
        if mm:
            a = dequantize_mx(q_a[g, :mm], scale_a[g][:, :mm])
            d[g, :mm] = a @ b[g].T
    return d


# ---------------------------------------------------------------- MXFP4 (E2M1, 1 x 32 blocks)
# The page's own element type: "mxfp4 (a4w4)" (third reference page, section
# "Summary").  E2M1 (OCP FP4): 1 sign, 2 exponent bits (bias 1), 1 mantissa
# bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinity or NaN.  Readings
# of what the page leaves open:
#   * the scale follows the same "Even" rule as MXFP8 at E2M1's precision:
#     amax rounded to 1 fraction bit (nearest, ties to even), then
#     t = floor(log2(rounded amax)) - 2 (2 is the exponent of E2M1's largest
#     power of two, 4), so a block whose amax significand is at least 1.75
#     takes the larger scale and its largest element never lies above 7
#     after scaling;
#   * elements x / 2**t rounded to nearest, ties to the even code, clamped to
#     +-6; all-zero block t = 0;
#   * two elements per byte, the lower K index in the low nibble;
#   * scales as for MXFP8: [K/32, M] for A and [G, K/32, N] for B.

E2M1_MAX = 6.0
MX4_EMAX = 2
MX4_MBITS = 1              # E2M1 fraction bits


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """Value of each 4-bit E2M1 code (0..15), float64."""
    c = np.asarray(codes, dtype=np.int64) & 15
    s, e, m = c >> 3, (c >> 1) & 3, c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def encode_e2m1_rne(x: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code to each value with |x| <= 6, ties to the even code.

    The positive codes 0..7 are in increasing order of value, so the nearest
    code is found by comparing against the midpoints between neighbours; a
    value exactly on a midpoint takes the code with an even mantissa bit.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E2M1_MAX) or np.any(~np.isfinite(x)):
        raise ValueError("encode_e2m1_rne: |x| must be <= 6")
    vals = decode_e2m1(np.arange(8))                     # 0, .5, 1, 1.5, 2, 3, 4, 6
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.int64)
    for c in range(7):
        mid = (vals[c] + vals[c + 1]) / 2.0
        up = (a > mid) | ((a == mid) & ((c + 1) % 2 == 0))
        code = np.where(up & (code == c), c + 1, code)
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def mx4_exponent(amax: np.ndarray) -> np.ndarray:
    """E2M1 MX scale exponent under the "Even" rule (1 fraction bit, emax 2)."""
    return _even_scale_exponent(amax, MX4_MBITS, MX4_EMAX, "mx4_exponent")


def quantize_mx4_1x32(x: np.ndarray):
    """MXFP4 quantization of x[..., R, K] along K (K a multiple of 32).

    Returns ``(q [..., R, K/2] uint8, scale_t [..., K/32, R] uint8)``: codes
    RNE_e2m1(clamp(x / 2**t, -6, 6)) packed two per byte (element 2i in the
    low nibble of byte i), t = mx4_exponent(max |block|) per 32-wide block.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    *lead, R, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("quantize_mx4_1x32: K must be a multiple of 32")
    xb = x.reshape(*lead, R, K // MX_BLOCK, MX_BLOCK)
    t = mx4_exponent(np.abs(xb).max(axis=-1))
    v = np.clip(xb / np.exp2(t[..., None].astype(np.float64)), -E2M1_MAX, E2M1_MAX)
    codes = encode_e2m1_rne(v).reshape(*lead, R, K)
    q = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    st = np.swapaxes((t + 127).astype(np.uint8), -1, -2)
    return np.ascontiguousarray(q), np.ascontiguousarray(st)


def dequantize_mx4(q: np.ndarray, scale_t: np.ndarray) -> np.ndarray:
    """X_dq[..., r, k] = e2m1(nibble k of row r) * 2**(scale_t[..., k // 32, r] - 127)."""
    q = np.asarray(q, dtype=np.uint8)
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(*q.shape[:-1], 2 * q.shape[-1])
    s = np.swapaxes(e8m0_value(scale_t), -1, -2)
    return decode_e2m1(codes) * np.repeat(s, MX_BLOCK, axis=-1)


def grouped_gemm_mx4_contiguous(q_a, scale_a, q_b, scale_b, grouped_layout, d_init=None):
    """Contiguous grouped GEMM on MXFP4 operands (A [M, K/2] packed, B [G, N, K/2]),
    float64; other rows keep ``d_init``."""
    a = dequantize_mx4(q_a, scale_a)
    b = dequantize_mx4(q_b, scale_b)
    layout = np.asarray(grouped_layout, dtype=np.int64)
    M, N = a.shape[0], b.shape[1]
    d = np.full((M, N), np.nan) if d_init is None else np.array(d_init, dtype=np.float64)
    for g in range(b.shape[0]):
        rows = np.nonzero(layout == g)[0]
        if rows.size:
            d[rows] = a[rows] @ b[g].T
    return d


def grouped_gemm_mx4_masked(q_a, scale_a, q_b, scale_b, masked_m, d_init=None):
    """Masked grouped GEMM on MXFP4 operands: A [G, M_max, K/2] with scale_a
    [G, K/32, M_max]; rows m < masked_m[g] computed, others keep ``d_init``."""
    G, Mmax, _ = q_a.shape
    b = dequantize_mx4(q_b, scale_b)
    N = b.shape[1]
    d = np.full((G, Mmax, N), np.nan) if d_init is None else np.array(d_init, dtype=np.float64)
    for g in range(G):
        mm = int(min(max(int(masked_m[g]), 0), Mmax))
        if mm:
            a = dequantize_mx4(q_a[g, :mm], scale_a[g][:, :mm])
            d[g, :mm] = a @ b[g].T
    return d


# ---------------------------------------------------------------- a4w4 gemm1 with silu_mul
# The third reference page's gemm1 runs on "mxfp4 (a4w4)" operands and ends in
# the silu_mul epilogue (section "Changes", item gemm1).  Written out, it is the
# MXFP4 grouped GEMM above followed by the silu_mul of the gemm1 section, under
# the same gate|up reading: B[g] has 2I rows, gate rows [0, I) and up rows
# [I, 2I), and out[m, j] = silu(h[j]) * h[I + j] with h = A_dq[m] . B_dq[g]^T.
def grouped_gemm_mx4_silu_mul_contiguous(q_a, scale_a, q_b, scale_b, grouped_layout, out_init=None):
    """Contiguous a4w4 gemm1 with silu_mul, float64.

    q_a [M, K/2] and q_b [G, 2I, K/2] hold E2M1 codes two per byte, with
    scales [K/32, M] and [G, K/32, 2I].  Rows with ``grouped_layout == g`` get
    ``silu(h[:I]) * h[I:]``; padding rows keep ``out_init`` (NaN when none).
    """
    d = grouped_gemm_mx4_contiguous(q_a, scale_a, q_b, scale_b, grouped_layout)
    M, half = d.shape[0], d.shape[1] // 2
    out = np.full((M, half), np.nan) if out_init is None else np.array(out_init, dtype=np.float64)
    layout = np.asarray(grouped_layout, dtype=np.int64)
    rows = np.nonzero((layout >= 0) & (layout < q_b.shape[0]))[0]
    out[rows] = _silu_mul_rows(d[rows])
    return out


def grouped_gemm_mx4_silu_mul_masked(q_a, scale_a, q_b, scale_b, masked_m, out_init=None):
    """Masked a4w4 gemm1 with silu_mul, float64: q_a [G, M_max, K/2] with
    scale_a [G, K/32, M_max]; rows ``m < masked_m[g]`` of group g get
    ``silu(h[:I]) * h[I:]``, other rows keep ``out_init``."""
    d = grouped_gemm_mx4_masked(q_a, scale_a, q_b, scale_b, masked_m)
    G, Mmax, half = d.shape[0], d.shape[1], d.shape[2] // 2
    out = np.full((G, Mmax, half), np.nan) if out_init is None else np.array(out_init, dtype=np.float64)
    for g in range(G):
        mm = int(min(max(int(masked_m[g]), 0), Mmax))
        if mm:
            out[g, :mm] = _silu_mul_rows(d[g, :mm])
    return out


# ---------------------------------------------------------------- metrics
def calc_diff(x, y) -> float:
    """1 - 2*sum(x*y) / sum(x*x + y*y), in float64 ("cosine-similarity-style")."""
    x = np.asarray(x, dtype=np.float64).ravel()
    y = np.asarray(y, dtype=np.float64).ravel()
    denom = np.sum(x * x + y * y)
    if denom == 0.0:
        return 0.0
    return float(1.0 - 2.0 * np.sum(x * y) / denom)


def max_rel_err_rowfloor(got, ref, floor: float = 1e-3) -> float:
    """max |got - ref| / max(|ref|, floor * max_n |ref[m, n]|) over all elements.

    The denominator is floored per row (per token), which matches the
    per-token scaling: an output near zero is judged against the size of
    its row rather than against itself.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rowmax = np.abs(ref).max(axis=-1, keepdims=True)
    den = np.maximum(np.abs(ref), floor * rowmax)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(got - ref) / den))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), as float64.

    bfloat16 keeps 8 significant bits; the spacing in binade [2**E, 2**(E+1))
    is 2**(E-7).  Exact for inputs inside the bfloat16 normal range.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, p = np.frexp(np.where(a > 0, a, 1.0))
    quantum = np.exp2(np.maximum(p - 1, -126) - 7.0)
    return np.copysign(np.rint(a / quantum) * quantum, x)


def round_to_f16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest IEEE half (ties to even), as float64.

    Half keeps 11 significant bits; spacing 2**(E-10), subnormal spacing 2**-24.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, p = np.frexp(np.where(a > 0, a, 1.0))
    quantum = np.exp2(np.maximum(p - 1, -14) - 10.0)
    return np.copysign(np.rint(a / quantum) * quantum, x)
