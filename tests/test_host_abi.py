"""CPU tests of the C-ABI library: it loads, exports every declared symbol, its
host quantizers are bit-exact with the oracle's, and its argument checks
return the documented status codes before anything touches a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import fp8_block_scaled_amd as gfg
from fp8_block_scaled_amd import workloads as wl
from oracle import fp8_oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for h in os.listdir(os.path.join(ROOT, "include")):
        if h.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", h)).read()
            names += re.findall(r"GFG_API\s+[\w\s\*]+?\b(\w+)\s*\(", txt)
    return names


def test_library_exports_every_declared_symbol():
    lib = gfg.load_library()
    names = _declared_functions()
    assert {"grouped_fp8_gemm_contiguous", "grouped_fp8_gemm_masked", "fp8_quantize_act_1x128",
            "fp8_quantize_weight_128x128", "grouped_fp8_last_error", "gfg_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        gfg.load_library(str(tmp_path / "nope.so"))


@pytest.mark.parametrize("shape", [(1, 128), (7, 260), (300, 1000), (64, 7168)])
def test_act_quantizer_bit_exact(shape):
    rng = np.random.default_rng(sum(shape))
    x = (rng.standard_normal(shape) * 10.0 ** rng.uniform(-3, 3, (shape[0], 1))).astype(np.float32)
    if shape[0] > 2:
        x[1, :] = 0.0                         # all-zero blocks
    q, s = gfg.fp8_quantize_act_1x128(x)
    qo, so = o.quantize_act_1x128(x)
    assert np.array_equal(q, qo) and np.array_equal(s, so)


@pytest.mark.parametrize("shape", [(1, 128, 128), (2, 130, 260), (3, 384, 1000)])
def test_weight_quantizer_bit_exact(shape):
    rng = np.random.default_rng(sum(shape))
    w = (rng.standard_normal(shape) * 3).astype(np.float32)
    q, s = gfg.fp8_quantize_weight_128x128(w)
    qo, so = o.quantize_weight_128x128(w)
    assert np.array_equal(q, qo) and np.array_equal(s, so)


def test_quantizers_bit_exact_on_workload_slices():
    for idx in range(5):
        w = wl.workload(idx)
        x = wl.draw(wl.Workload(w.name, "contiguous", 1, 128, w.K, w.out_dtype, w.seed,
                                m_per_group=[200], row_log10_range=w.row_log10_range))
        q, s = gfg.fp8_quantize_act_1x128(x["a"])
        qo, so = o.quantize_act_1x128(x["a"])
        assert np.array_equal(q, qo) and np.array_equal(s, so)
        qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
        qbo, sbo = o.quantize_weight_128x128(x["b"])
        assert np.array_equal(qb, qbo) and np.array_equal(sb, sbo)


def test_quantizer_boundaries_bit_exact():
    # amax exactly at and next to 448 * 2^t, every midpoint of the e4m3 grid
    vals = np.array(sorted({float(v) for v in o.decode_e4m3(np.arange(0, 127, dtype=np.uint8))}))
    mids = (vals[1:] + vals[:-1]) / 2
    row = np.concatenate([vals, mids, -mids])
    row = np.resize(row, 4 * 128).astype(np.float32)
    x = np.stack([row, row * 2.0 ** -5, np.nextafter(row, np.float32(np.inf)).astype(np.float32)])
    q, s = gfg.fp8_quantize_act_1x128(x)
    qo, so = o.quantize_act_1x128(x)
    assert np.array_equal(q, qo) and np.array_equal(s, so)


def test_masked_quantizer_matches_oracle():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 50, 256)).astype(np.float32)
    q, s = gfg.fp8_quantize_act_masked(x)
    qo, so = o.quantize_act_masked(x)
    assert np.array_equal(q, qo) and np.array_equal(s, so)


def test_quantizer_range_errors():
    with pytest.raises(gfg.GfgError) as e:
        gfg.fp8_quantize_act_1x128(np.full((2, 128), np.nan, np.float32))
    assert e.value.code == 4
    with pytest.raises(gfg.GfgError) as e:
        gfg.fp8_quantize_act_1x128(np.full((2, 128), 1e-44, np.float32))   # scale below 2^-127
    assert e.value.code == 4
    with pytest.raises(gfg.GfgError) as e:
        gfg.fp8_quantize_weight_128x128(np.full((1, 128, 128), np.inf, np.float32))
    assert e.value.code == 4


def test_quantizer_argument_errors():
    lib = gfg.load_library()
    assert lib.fp8_quantize_act_1x128(None, 4, 128, None, None) == 1
    assert lib.fp8_quantize_act_1x128(None, -1, 128, None, None) == 1
    assert lib.fp8_quantize_act_1x128(None, 0, 128, None, None) == 0      # empty: no-op
    assert lib.fp8_quantize_weight_128x128(None, 0, 128, 128, None, None) == 1


def test_device_quantizer_argument_errors():
    # host-side checks that return before any HIP call (fake addresses are never touched)
    q = gfg.raw_quantize_act_device
    assert q(0x1000, 2, 1, 4, 128, 0x1000, 0x1000) == 1          # bad in_dtype
    assert q(0x1000, 0, 0, 4, 128, 0x1000, 0x1000) == 1          # G = 0
    assert q(0x1000, 0, 1, -1, 128, 0x1000, 0x1000) == 1         # negative M
    assert q(None, 0, 1, 0, 128, None, None) == 0                # empty: no-op
    assert q(None, 1, 1, 4, 0, None, None) == 0
    assert q(None, 0, 1, 4, 128, 0x1000, 0x1000) == 1            # null x
    assert q(0x1000, 0, 1, 4, 200, 0x1000, 0x1000) == 2          # K not a multiple of 128
    assert q(0x1000, 0, 1, 4, (1 << 24) + 128, 0x1000, 0x1000) == 2   # K above 2^24
    assert q(0x1000, 0, 1, (1 << 30) + 1, 128, 0x1000, 0x1000) == 2   # M above 2^30
    assert q(0x1000, 0, 65535, 1 << 20, 1 << 14, 0x1000, 0x1000) == 2  # 2^31 or more triples
    assert "2^31" in gfg.load_library().grouped_fp8_last_error().decode()
    assert q(0x1008, 0, 1, 4, 128, 0x1000, 0x1000) == 1          # x not 16-byte aligned
    assert "16-byte" in gfg.load_library().grouped_fp8_last_error().decode()


# Host-side argument checks of the GEMM entry points: these return before any
# HIP call, so fake non-null addresses are never dereferenced.
FAKE = 0x1000


def _c(**kw):
    args = dict(a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, meta=FAKE, d=FAKE, M=256, N=256, K=256, G=2, dt=0)
    args.update(kw)
    return gfg.raw_contiguous(args["a"], args["sa"], args["b"], args["sb"], args["meta"], args["d"],
                              args["M"], args["N"], args["K"], args["G"], args["dt"], 0)


def _m(**kw):
    args = dict(a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, meta=FAKE, d=FAKE, G=2, Mmax=256, N=256, K=256, dt=0)
    args.update(kw)
    return gfg.raw_masked(args["a"], args["sa"], args["b"], args["sb"], args["meta"], args["d"],
                          args["G"], args["Mmax"], args["N"], args["K"], args["dt"], 0)


@pytest.mark.parametrize("fn", [_c, _m])
def test_gemm_argument_errors(fn):
    for k in ("a", "sa", "b", "sb", "meta", "d"):
        assert fn(**{k: None}) == 1, k
    assert fn(dt=2) == 1
    assert fn(G=0) == 1
    assert fn(G=70000) == 1
    assert fn(N=0) == 1
    assert fn(K=-128) == 1
    assert fn(N=200) == 2          # ragged N: outside the kernels' tiling
    assert fn(K=300) == 2
    msg = gfg.load_library().grouped_fp8_last_error().decode()
    assert "multiples of 128" in msg


def test_gemm_empty_and_oversize():
    assert _c(M=0) == 0            # empty: no launch
    assert _m(Mmax=0) == 0
    assert _c(M=-1) == 1
    assert _m(Mmax=-5) == 1
    assert _c(M=4096 * 128 + 1) == 2
    assert _m(G=33, Mmax=128 * 128) == 2


def test_32bit_extent_bounds():
    """One expert's B (N*K bytes) and the A-scale tensor are addressed with
    32-bit offsets in the kernels; larger extents are refused before any launch
    (including the up rows of silu_mul, which lie N/2 rows past the gate rows).
    The accepted edge cases use zero rows, so nothing is launched."""
    assert _c(N=1 << 20, K=1 << 12) == 2                      # N*K = 2^32
    assert "2^32" in gfg.load_library().grouped_fp8_last_error().decode()
    assert _c(N=1 << 19, K=1 << 12, M=0) == 0                 # 2^31: accepted
    assert _sc(I=1 << 19, K=1 << 13) == 2                     # 2I*K = 2^33
    assert _sm(I=1 << 19, K=1 << 13) == 2
    assert _sc(I=1 << 17, K=1 << 13, M=0) == 0                # 2^31: accepted
    # A-scale tensor [K/128][M]: 2^19 rows x 2^16 blocks = 2^35 bytes
    assert _c(M=1 << 19, N=128, K=1 << 23) == 2
    assert "A-scale" in gfg.load_library().grouped_fp8_last_error().decode()
    assert _m(G=1, Mmax=1 << 19, N=128, K=1 << 23) == 2
    # MXFP8: one scale byte per 32 K elements: 2^19 rows x 2^13 = 2^32
    assert gfg.raw_mx_contiguous(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 19, 256, 1 << 18, 1, 0, 0) == 2
    assert gfg.raw_mx_contiguous(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 256, 1 << 18, 1, 0, 0) == 0


def _sc(**kw):
    args = dict(a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, meta=FAKE, d=FAKE, M=256, I=256, K=256, G=2, dt=0)
    args.update(kw)
    return gfg.raw_silu_mul_contiguous(args["a"], args["sa"], args["b"], args["sb"], args["meta"], args["d"],
                                       args["M"], args["I"], args["K"], args["G"], args["dt"], 0)


def _sm(**kw):
    args = dict(a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, meta=FAKE, d=FAKE, G=2, Mmax=256, I=256, K=256, dt=0)
    args.update(kw)
    return gfg.raw_silu_mul_masked(args["a"], args["sa"], args["b"], args["sb"], args["meta"], args["d"],
                                   args["G"], args["Mmax"], args["I"], args["K"], args["dt"], 0)


@pytest.mark.parametrize("fn", [_sc, _sm])
def test_silu_mul_argument_errors(fn):
    for k in ("a", "sa", "b", "sb", "meta", "d"):
        assert fn(**{k: None}) == 1, k
    assert fn(dt=2) == 1
    assert fn(G=0) == 1
    assert fn(I=0) == 1
    assert fn(I=-128) == 1
    assert fn(K=300) == 2
    assert fn(I=192) == 2          # I must be a multiple of 128 (the output tile)
    assert "multiple of 128" in gfg.load_library().grouped_fp8_last_error().decode()
    assert fn(sa=FAKE + 2) == 2    # the packed A-scale words need 4-byte alignment
    rows = {"M": 258} if fn is _sc else {"Mmax": 258}
    assert fn(**rows) == 2         # scale rows not a multiple of 4
    assert "multiple of 4" in gfg.load_library().grouped_fp8_last_error().decode()


def test_silu_mul_empty_is_noop():
    assert _sc(M=0) == 0
    assert _sm(Mmax=0) == 0
    assert _sc(M=-4) == 1
    assert _sm(Mmax=-4) == 1


# ------------------------------------------------------------------ MXFP8
@pytest.mark.parametrize("shape", [(1, 32), (7, 96), (65, 256), (3, 40, 128)])
def test_mx_quantizer_bit_exact(shape):
    rng = np.random.default_rng(sum(shape))
    x = (rng.standard_normal(shape) * 10.0 ** rng.uniform(-4, 4, shape[:-1] + (1,))).astype(np.float32)
    q, s = gfg.fp8_quantize_mx_1x32(x)
    oq, os_ = o.quantize_mx_1x32(x)
    assert np.array_equal(q, oq) and np.array_equal(s, os_)


def test_mx_quantizer_boundaries_bit_exact():
    """Blocks at the exponent edges (amax = 256*2^t and one float32 ulp
    below), at the "Even" carry point (amax = 496*2^t, the tie that rounds up
    to 512*2^t, and one ulp below, which does not), saturating blocks (scaled
    maximum in (448, 496)), subnormal elements, an all-zero block and negative
    zeros."""
    f32_below = lambda v: float(np.nextafter(np.float32(v), np.float32(0)))
    blocks = []
    for t in (-30, -1, 0, 5, 60):
        for amax in (256.0 * 2.0 ** t, f32_below(256.0 * 2.0 ** t), 496.0 * 2.0 ** t, f32_below(496.0 * 2.0 ** t),
                     500.0 * 2.0 ** t, 480.0 * 2.0 ** t, 448.0 * 2.0 ** t):
            b = np.linspace(-1, 1, 32) * amax
            b[7] = amax
            blocks.append(b)
    z = np.zeros(32)
    z[3] = -0.0
    blocks.append(z)
    tiny = np.full(32, 2.0 ** -20)
    tiny[0] = 1.0
    blocks.append(tiny)
    x = np.stack(blocks).astype(np.float32).reshape(1, -1)
    x = np.concatenate([x, -x[:, ::-1]])
    q, s = gfg.fp8_quantize_mx_1x32(x)
    oq, os_ = o.quantize_mx_1x32(x)
    assert np.array_equal(s, os_) and np.array_equal(q, oq)


def test_mx_quantizer_errors():
    lib = gfg.load_library()
    x = np.zeros((2, 64), np.float32)
    q = np.empty((2, 64), np.uint8)
    s = np.empty((2, 2), np.uint8)
    assert lib.fp8_quantize_mx_1x32(x.ctypes.data, 1, 2, 48, q.ctypes.data, s.ctypes.data) == 2   # K % 32
    assert lib.fp8_quantize_mx_1x32(None, 1, 2, 64, q.ctypes.data, s.ctypes.data) == 1
    assert lib.fp8_quantize_mx_1x32(x.ctypes.data, 0, 2, 64, q.ctypes.data, s.ctypes.data) == 1
    x[1, 40] = np.nan
    assert lib.fp8_quantize_mx_1x32(x.ctypes.data, 1, 2, 64, q.ctypes.data, s.ctypes.data) == 4
    x[1, 40] = 1e-37                         # t = -131
    assert lib.fp8_quantize_mx_1x32(x.ctypes.data, 1, 2, 64, q.ctypes.data, s.ctypes.data) == 4


def _mc(**kw):
    args = dict(a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, meta=FAKE, d=FAKE, M=256, N=256, K=256, G=2, dt=0)
    args.update(kw)
    return gfg.raw_mx_contiguous(args["a"], args["sa"], args["b"], args["sb"], args["meta"], args["d"],
                                 args["M"], args["N"], args["K"], args["G"], args["dt"], 0)


def _mm(**kw):
    args = dict(a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, meta=FAKE, d=FAKE, G=2, Mmax=256, N=256, K=256, dt=0)
    args.update(kw)
    return gfg.raw_mx_masked(args["a"], args["sa"], args["b"], args["sb"], args["meta"], args["d"],
                             args["G"], args["Mmax"], args["N"], args["K"], args["dt"], 0)


@pytest.mark.parametrize("fn", [_mc, _mm])
def test_mx_gemm_argument_errors(fn):
    for k in ("a", "sa", "b", "sb", "meta", "d"):
        assert fn(**{k: None}) == 1, k
    assert fn(dt=2) == 1
    assert fn(G=0) == 1
    assert fn(K=300) == 2
    assert fn(N=384) == 2          # N must be a multiple of 256
    assert "multiple of 256" in gfg.load_library().grouped_fp8_last_error().decode()
    assert fn(sa=FAKE + 1) == 2
    assert fn(sb=FAKE + 2) == 2
    rows = {"M": 130} if fn is _mc else {"Mmax": 130}
    assert fn(**rows) == 2
    empty = {"M": 0} if fn is _mc else {"Mmax": 0}
    assert fn(**empty) == 0


# ------------------------------------------------------------------ MXFP4
@pytest.mark.parametrize("shape", [(1, 128), (7, 256), (3, 40, 384)])
def test_mx4_quantizer_bit_exact(shape):
    rng = np.random.default_rng(sum(shape) + 4)
    x = (rng.standard_normal(shape) * 10.0 ** rng.uniform(-4, 4, shape[:-1] + (1,))).astype(np.float32)
    q, s = gfg.fp4_quantize_mx_1x32(x)
    oq, os_ = o.quantize_mx4_1x32(x)
    assert np.array_equal(q, oq) and np.array_equal(s, os_)


def test_mx4_quantizer_boundaries_bit_exact():
    """Exponent edges (amax = 4*2^t and one float32 ulp below), the "Even"
    carry point (amax = 7*2^t, the tie that rounds up to 8*2^t, and one ulp
    below), saturating blocks (scaled maximum in (6, 7)), every E2M1 midpoint,
    an all-zero block and negative zeros."""
    f32_below = lambda v: float(np.nextafter(np.float32(v), np.float32(0)))
    blocks = []
    for t in (-30, -1, 0, 5, 60):
        for amax in (4.0 * 2.0 ** t, f32_below(4.0 * 2.0 ** t), 7.0 * 2.0 ** t, f32_below(7.0 * 2.0 ** t),
                     7.5 * 2.0 ** t, 6.5 * 2.0 ** t, 6.0 * 2.0 ** t):
            b = np.linspace(-1, 1, 32) * amax
            b[9] = amax
            blocks.append(b)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    b = np.concatenate([mids, -mids, mids * 0.999, mids * 1.001])
    blocks.append(b)                        # amax 6.006 = 1.5015 * 4: t = 0, the 1.001 * 6 saturates
    z = np.zeros(32)
    z[5] = -0.0
    blocks.append(z)
    blocks.append(np.zeros(32))
    x = np.stack(blocks).astype(np.float32).reshape(1, -1)
    x = np.pad(x, ((0, 0), (0, (-x.shape[1]) % 128)))   # K a multiple of 128
    q, s = gfg.fp4_quantize_mx_1x32(x)
    oq, os_ = o.quantize_mx4_1x32(x)
    assert np.array_equal(s, os_) and np.array_equal(q, oq)


def test_mx4_quantizer_errors():
    lib = gfg.load_library()
    x = np.zeros((2, 128), np.float32)
    q = np.empty((2, 64), np.uint8)
    s = np.empty((4, 2), np.uint8)
    assert lib.fp4_quantize_mx_1x32(x.ctypes.data, 1, 2, 96, q.ctypes.data, s.ctypes.data) == 2   # K % 128
    assert lib.fp4_quantize_mx_1x32(None, 1, 2, 128, q.ctypes.data, s.ctypes.data) == 1
    x[1, 40] = np.inf
    assert lib.fp4_quantize_mx_1x32(x.ctypes.data, 1, 2, 128, q.ctypes.data, s.ctypes.data) == 4


@pytest.mark.parametrize("contig", [True, False])
def test_mx4_gemm_argument_errors(contig):
    def call(**kw):
        a = dict(a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, meta=FAKE, d=FAKE, M=256, N=256, K=512, G=2, dt=0)
        a.update(kw)
        if contig:
            return gfg.raw_mx4_contiguous(a["a"], a["sa"], a["b"], a["sb"], a["meta"], a["d"], a["M"], a["N"], a["K"],
                                          a["G"], a["dt"], 0)
        return gfg.raw_mx4_masked(a["a"], a["sa"], a["b"], a["sb"], a["meta"], a["d"], a["G"], a["M"], a["N"], a["K"],
                                  a["dt"], 0)
    for k in ("a", "sa", "b", "sb", "meta", "d"):
        assert call(**{k: None}) == 1, k
    assert call(K=0) == 1
    assert call(K=384) == 2            # K (elements) must be a multiple of 256
    assert "multiple of 256" in gfg.load_library().grouped_fp8_last_error().decode()
    assert call(N=384) == 2
    assert call(M=130) == 2
    assert call(sb=FAKE + 2) == 2
    assert call(M=0) == 0


# ------------------------------------------------------------------ a4w4 gemm1 with silu_mul
@pytest.mark.parametrize("contig", [True, False])
def test_mx4_silu_mul_argument_errors(contig):
    def call(**kw):
        a = dict(a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, meta=FAKE, d=FAKE, M=256, I=256, K=512, G=2, dt=0)
        a.update(kw)
        if contig:
            return gfg.raw_mx4_silu_mul_contiguous(a["a"], a["sa"], a["b"], a["sb"], a["meta"], a["d"], a["M"],
                                                   a["I"], a["K"], a["G"], a["dt"], 0)
        return gfg.raw_mx4_silu_mul_masked(a["a"], a["sa"], a["b"], a["sb"], a["meta"], a["d"], a["G"], a["M"],
                                           a["I"], a["K"], a["dt"], 0)
    for k in ("a", "sa", "b", "sb", "meta", "d"):
        assert call(**{k: None}) == 1, k
    assert call(dt=2) == 1
    assert call(G=0) == 1
    assert call(K=0) == 1
    assert call(I=0) == 1
    assert call(K=384) == 2            # K (E2M1 elements) must be a multiple of 256
    assert "multiple of 256" in gfg.load_library().grouped_fp8_last_error().decode()
    assert call(I=192) == 2            # I must be a multiple of 128 (the output tile)
    assert "multiple of 128" in gfg.load_library().grouped_fp8_last_error().decode()
    assert call(M=130) == 2            # scale rows not a multiple of 4
    assert call(sa=FAKE + 2) == 2
    assert call(sb=FAKE + 2) == 2
    assert call(M=0) == 0
    assert call(M=-4) == 1


def test_launch_settings_argument_errors():
    lib = gfg.load_library()
    assert lib.grouped_fp8_set_tile_order(0, 0) == 1
    assert lib.grouped_fp8_set_tile_order(9, 0) == 1
    assert lib.grouped_fp8_set_tile_order(8, -1) == 1
    assert lib.grouped_fp8_set_tile_order(8, 65) == 1
    assert lib.grouped_fp8_set_tile_shape(3) == 1
    assert lib.grouped_fp8_set_tile_shape(-1) == 1
    assert lib.grouped_fp8_set_grid_limit(-1) == 1
    assert lib.grouped_fp8_set_tile_order(1, 4) == 0 and lib.grouped_fp8_set_tile_order(8, 0) == 0
    assert lib.grouped_fp8_set_tile_shape(2) == 0 and lib.grouped_fp8_set_tile_shape(0) == 0
    assert lib.grouped_fp8_set_grid_limit(16) == 0 and lib.grouped_fp8_set_grid_limit(0) == 0


def test_ceiling_argument_errors():
    """The ceiling kernels' host checks (no launch happens)."""
    with pytest.raises(gfg.GfgError) as e:
        gfg.ceiling_copy(16, 32, 17)
    assert e.value.code == 1
    with pytest.raises(gfg.GfgError) as e:
        gfg.ceiling_mfma(32, 16, 1, 64, 1 << 20)
    assert e.value.code == 1
    with pytest.raises(gfg.GfgError) as e:
        gfg.ceiling_mfma_16x16x128(32, 16, 1, 64, 1 << 20)
    assert e.value.code == 1
    with pytest.raises(gfg.GfgError) as e:
        gfg.ceiling_read(16, 24, 64, 1 << 20)          # bytes not a multiple of 16
    assert e.value.code == 1
    with pytest.raises(gfg.GfgError) as e:
        gfg.ceiling_read(8, 32, 64, 1 << 20)           # src not 16-byte aligned
    assert e.value.code == 1
    lib = gfg.load_library()
    assert lib.gfg_device_peak(None, None, None) == 1
