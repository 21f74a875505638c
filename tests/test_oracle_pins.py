"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test ties a part of the oracle to something fixed outside it: the OCP
FP8 format definition (hand-derived golden files), a library cast (torch's
float8_e4m3fn / bfloat16, numpy's float16), brute force on tiny inputs in
pure Python, closed forms, exact integer arithmetic and the error bound the
first reference page states (calc_diff <= 1e-3 against the pre-quantization
FP32 product, section "DeepGEMM conformance details").
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import fp8_oracle as o
from fp8_block_scaled_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name, cols=2):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split()[:cols])
    return rows


# ------------------------------------------------------------------ brute force helpers
def _all_e4m3_values():
    """(code, value) for every finite E4M3FN code, from the bit-field definition."""
    out = []
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        out.append((c, -v if s else v))
    return out


_TABLE = _all_e4m3_values()


def _bf_encode(x: float) -> int:
    """Nearest finite E4M3FN code by exhaustive search; ties go to the even code."""
    best = None
    for c, v in _TABLE:
        if v == 0.0 and (c >> 7) != (1 if math.copysign(1, x) < 0 else 0):
            continue  # keep the sign of zero
        d = abs(v - x)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _bf_exponent(amax: float) -> int:
    if amax == 0.0:
        return 0
    for t in range(-140, 140):
        if 448.0 * 2.0 ** t >= amax:
            return t
    raise AssertionError


def _bf_quant_act(x):
    M, K = x.shape
    kb = -(-K // 128)
    q = np.zeros((M, K), np.uint8)
    s = np.zeros((kb, M), np.uint8)
    for m in range(M):
        for b in range(kb):
            blk = [float(v) for v in x[m, 128 * b:128 * b + 128]]
            t = _bf_exponent(max(abs(v) for v in blk))
            s[b, m] = t + 127
            for j, v in enumerate(blk):
                q[m, 128 * b + j] = _bf_encode(v / 2.0 ** t)
    return q, s


def _bf_quant_weight(w):
    G, N, K = w.shape
    nb, kb = -(-N // 128), -(-K // 128)
    q = np.zeros((G, N, K), np.uint8)
    s = np.zeros((G, nb, kb), np.uint8)
    for g in range(G):
        for i in range(nb):
            for b in range(kb):
                blk = w[g, 128 * i:128 * i + 128, 128 * b:128 * b + 128].astype(np.float64)
                t = _bf_exponent(float(np.abs(blk).max()))
                s[g, i, b] = t + 127
                for r in range(blk.shape[0]):
                    for j in range(blk.shape[1]):
                        q[g, 128 * i + r, 128 * b + j] = _bf_encode(float(blk[r, j]) / 2.0 ** t)
    return q, s


def _val(code):
    return dict(_TABLE)[int(code)]


def _bf_gemm_rows(qa, sa, qb, sb, rows_a, g):
    """fsum triple loop: D[r, n] = sum_k (A value * 2^(sa-127)) * (B value * 2^(sb-127))."""
    N, K = qb.shape[1], qb.shape[2]
    out = np.zeros((len(rows_a), N))
    for i, r in enumerate(rows_a):
        a = [_val(qa[r, k]) * 2.0 ** (int(sa[k // 128, r]) - 127) for k in range(K)]
        for n in range(N):
            out[i, n] = math.fsum(
                a[k] * _val(qb[g, n, k]) * 2.0 ** (int(sb[g, n // 128, k // 128]) - 127)
                for k in range(K))
    return out


# ------------------------------------------------------------------ format pins
def test_decode_golden_codes():
    for code, val in _read_golden("e4m3_codes.txt"):
        got = o.decode_e4m3(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code


def test_decode_matches_bitfield_table():
    codes = np.array([c for c, _ in _TABLE], np.uint8)
    assert np.array_equal(o.decode_e4m3(codes), np.array([v for _, v in _TABLE]))


def test_encode_matches_torch_cast_at_every_midpoint():
    vals = np.array(sorted({v for _, v in _TABLE}))
    mids = (vals[1:] + vals[:-1]) / 2          # every tie, exactly representable in f32
    x = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    x = x[np.abs(x) <= 448].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.encode_e4m3_rne(x.astype(np.float64)), ref)


def test_encode_matches_torch_cast_random():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-448, 448, 200000),
                        rng.standard_normal(200000) * 10.0 ** rng.uniform(-4, 2, 200000)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.encode_e4m3_rne(x.astype(np.float64)), ref)


def test_encode_bruteforce_sample():
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.uniform(-448, 448, 300), rng.uniform(-0.02, 0.02, 300),
                        [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -11, 447.99, 2.0 ** -6 - 2.0 ** -11]])
    got = o.encode_e4m3_rne(x)
    assert [int(c) for c in got] == [_bf_encode(float(v)) for v in x]


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        o.encode_e4m3_rne(np.array([448.5]))
    with pytest.raises(ValueError):
        o.encode_e4m3_rne(np.array([np.nan]))


def test_e8m0_golden():
    for amax, byte in _read_golden("e8m0_ceil.txt"):
        t = o.e8m0_ceil_exponent(np.array([float(amax)]))[0]
        assert t + 127 == int(byte), amax


def test_e8m0_bruteforce():
    rng = np.random.default_rng(7)
    a = np.concatenate([10.0 ** rng.uniform(-6, 4, 2000), 448.0 * 2.0 ** np.arange(-20, 20),
                        np.nextafter(448.0 * 2.0 ** np.arange(-20, 20), np.inf),
                        np.nextafter(448.0 * 2.0 ** np.arange(-20, 20), 0)])
    got = o.e8m0_ceil_exponent(a)
    assert [int(t) for t in got] == [_bf_exponent(float(v)) for v in a]


def test_e8m0_value_and_nan():
    v = o.e8m0_value(np.array([0, 127, 128, 254, 255]))
    assert v[1] == 1.0 and v[2] == 2.0 and v[0] == 2.0 ** -127 and v[3] == 2.0 ** 127
    assert np.isnan(v[4])


def test_e8m0_rejects_out_of_range():
    with pytest.raises(ValueError):
        o.e8m0_ceil_exponent(np.array([1e-45]))      # would need t < -127


# ------------------------------------------------------------------ quantizer pins
def test_ceil_invariant_on_workload_blocks():
    """Every block: amax / s <= 448 and amax / (s/2) > 448 (the scale is minimal)."""
    w = wl.workload(4)                                 # log-uniform per-token magnitudes
    rng = np.random.default_rng(8)
    x = rng.standard_normal((256, 2304)).astype(np.float32)
    x *= np.power(10.0, rng.uniform(-2, 2, (256, 1))).astype(np.float32)
    q, s = o.quantize_act_1x128(x)
    amax = np.abs(x.astype(np.float64).reshape(256, 18, 128)).max(axis=2)
    scale = 2.0 ** (s.T.astype(np.float64) - 127)
    assert np.all(amax / scale <= 448.0)
    assert np.all(amax / (scale / 2) > 448.0)
    assert np.all(np.abs(o.decode_e4m3(q)) <= 448.0)
    bw = wl.draw(wl.Workload("t", "contiguous", 1, 256, 512, "bf16", w.seed, m_per_group=[1]))["b"]
    qb, sb = o.quantize_weight_128x128(bw)
    amaxb = np.abs(bw.astype(np.float64).reshape(1, 2, 128, 4, 128)).max(axis=(2, 4))
    sc = 2.0 ** (sb.astype(np.float64) - 127)
    assert np.all(amaxb / sc <= 448.0) and np.all(amaxb / (sc / 2) > 448.0)


def test_quantizers_bruteforce_tiny_ragged():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((5, 260)) * 10.0 ** rng.uniform(-3, 3, (5, 1))).astype(np.float32)
    x[2, 128:256] = 0.0                                # an all-zero block
    q, s = o.quantize_act_1x128(x)
    bq, bs = _bf_quant_act(x)
    assert np.array_equal(q, bq) and np.array_equal(s, bs)
    w = rng.standard_normal((2, 130, 260)).astype(np.float32) * 3
    qw, sw = o.quantize_weight_128x128(w)
    bqw, bsw = _bf_quant_weight(w)
    assert np.array_equal(qw, bqw) and np.array_equal(sw, bsw)


def test_masked_quantizer_layout():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((3, 7, 256)).astype(np.float32)
    q, s = o.quantize_act_masked(x)
    assert q.shape == (3, 7, 256) and s.shape == (3, 2, 7)
    for g in range(3):
        qg, sg = _bf_quant_act(x[g])
        assert np.array_equal(q[g], qg) and np.array_equal(s[g], sg)


# ------------------------------------------------------------------ GEMM pins
def test_contiguous_gemm_bruteforce_tiny():
    rng = np.random.default_rng(11)
    layout = np.array([0, 0, 0, -1, 1, 1, -1, -1, 1], np.int32)   # ragged, padding inside
    K, N = 260, 130
    a = rng.standard_normal((layout.size, K)).astype(np.float32)
    b = rng.standard_normal((2, N, K)).astype(np.float32)
    qa, sa = o.quantize_act_1x128(a)
    qb, sb = o.quantize_weight_128x128(b)
    d0 = np.full((layout.size, N), -7.0)
    d = o.grouped_gemm_contiguous(qa, sa, qb, sb, layout, d0)
    for g in range(2):
        rows = [r for r in range(layout.size) if layout[r] == g]
        ref = _bf_gemm_rows(qa, sa, qb, sb, rows, g)
        np.testing.assert_allclose(d[rows], ref, rtol=1e-12, atol=1e-12)
    assert np.all(d[layout < 0] == -7.0)


def test_masked_gemm_bruteforce_tiny():
    rng = np.random.default_rng(12)
    G, Mmax, N, K = 3, 6, 130, 260
    a = rng.standard_normal((G, Mmax, K)).astype(np.float32)
    b = rng.standard_normal((G, N, K)).astype(np.float32)
    masked_m = np.array([4, 0, 6], np.int32)
    qa, sa = o.quantize_act_masked(a)
    qb, sb = o.quantize_weight_128x128(b)
    d0 = np.full((G, Mmax, N), 3.5)
    d = o.grouped_gemm_masked(qa, sa, qb, sb, masked_m, d0)
    for g in range(G):
        mm = masked_m[g]
        if mm:
            ref = _bf_gemm_rows(qa[g], sa[g], qb, sb, list(range(mm)), g)
            np.testing.assert_allclose(d[g, :mm], ref, rtol=1e-12, atol=1e-12)
        assert np.all(d[g, mm:] == 3.5)


def test_exact_integer_special_case():
    """Integer FP8 inputs with scales 2^0..2^2: D equals the exact integer product."""
    case = wl.integer_case(13, G=2, rows=5, N=256, K=384)
    table = {int(i): int(c, 16) for i, c in _read_golden("e4m3_small_integers.txt")}
    qa = np.vectorize(table.get)(case["ints_a"]).astype(np.uint8)
    qb = np.vectorize(table.get)(case["ints_b"]).astype(np.uint8)
    d = o.grouped_gemm_contiguous(qa, case["scale_a"], qb, case["scale_b"], case["grouped_layout"])
    ia, ib = case["ints_a"], case["ints_b"]
    sa = case["scale_a"].astype(np.int64) - 127
    sb = case["scale_b"].astype(np.int64) - 127
    for r in range(ia.shape[0]):
        g = int(case["grouped_layout"][r])
        for n in range(0, 256, 37):
            exact = sum(int(ia[r, k]) * int(ib[g, n, k]) * 2 ** int(sa[k // 128, r] + sb[g, n // 128, k // 128])
                        for k in range(384))
            assert d[r, n] == exact


def test_cross_layout_masked_equals_contiguous():
    rng = np.random.default_rng(14)
    counts = [5, 0, 9]
    N, K, Mmax = 128, 256, 16
    b = rng.standard_normal((3, N, K)).astype(np.float32)
    a_m = rng.standard_normal((3, Mmax, K)).astype(np.float32)
    layout = wl.contiguous_layout(counts, align=16)
    a_c = np.zeros((layout.size, K), np.float32)
    pos = 0
    for g, c in enumerate(counts):
        a_c[pos:pos + c] = a_m[g, :c]
        pos += -(-c // 16) * 16
    qb, sb = o.quantize_weight_128x128(b)
    qa, sa = o.quantize_act_masked(a_m)
    dm = o.grouped_gemm_masked(qa, sa, qb, sb, np.array(counts))
    qc, sc = o.quantize_act_1x128(a_c)
    dc = o.grouped_gemm_contiguous(qc, sc, qb, sb, layout)
    pos = 0
    for g, c in enumerate(counts):
        assert np.array_equal(dm[g, :c], dc[pos:pos + c])
        pos += -(-c // 16) * 16


@pytest.mark.parametrize("idx,rows", [(0, None), (1, 256), (2, 300), (4, 256)])
def test_fp32_product_bound(idx, rows):
    """calc_diff(oracle, pre-quantization fp32 product) <= 1e-3 (page 1's threshold)."""
    w = wl.workload(idx)
    if rows is not None:                               # a slice of the workload's rows
        w = wl.Workload(w.name, "contiguous", 2, w.N, w.K, w.out_dtype, w.seed,
                        m_per_group=[rows // 2, rows - rows // 2], row_log10_range=w.row_log10_range)
        w.N = min(w.N, 1024)
    x = wl.draw(w)
    qa, sa = o.quantize_act_1x128(x["a"])
    qb, sb = o.quantize_weight_128x128(x["b"])
    d = o.grouped_gemm_contiguous(qa, sa, qb, sb, x["grouped_layout"])
    lay = x["grouped_layout"]
    ref = np.full_like(d, np.nan)
    for g in range(w.G):
        rows_g = lay == g
        ref[rows_g] = x["a"][rows_g].astype(np.float64) @ x["b"][g].astype(np.float64).T
    valid = lay >= 0
    diff = o.calc_diff(d[valid], ref[valid])
    assert diff <= 1e-3, diff
    assert diff > 1e-6                                  # quantization error is really present


def test_calc_diff_closed_forms():
    rng = np.random.default_rng(15)
    x = rng.standard_normal(1000)
    assert o.calc_diff(x, x) == pytest.approx(0.0, abs=1e-15)
    assert o.calc_diff(x, -x) == pytest.approx(2.0)
    assert o.calc_diff(x, 2 * x) == pytest.approx(0.2)              # 1 - 4/5
    y = rng.standard_normal(1000)
    assert o.calc_diff(x, y) == pytest.approx(np.sum((x - y) ** 2) / np.sum(x * x + y * y))


def test_max_rel_err_rowfloor():
    ref = np.array([[100.0, 1e-9, -50.0], [0.0, 0.0, 0.0]])
    got = ref + np.array([[1.0, 0.05, 0.0], [0.0, 0.0, 0.0]])
    # element (0,1): |0.05| / max(1e-9, 1e-3*100) = 0.5; element (0,0): 1/100
    assert o.max_rel_err_rowfloor(got, ref) == pytest.approx(0.5)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(16)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-5, 5, 100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(o.round_to_bf16(x.astype(np.float64)), ref)


def test_round_f16_matches_numpy():
    rng = np.random.default_rng(17)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-6, 4, 100000))
    x = x[np.abs(x) < 65504]
    assert np.array_equal(o.round_to_f16(x), x.astype(np.float16).astype(np.float64))


# ------------------------------------------------------------------ planted mistakes
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle (on the CPU) and check a pin fails."""
    failures = 0
    # floor instead of ceil for the scale exponent
    real = o.e8m0_ceil_exponent
    monkeypatch.setattr(o, "e8m0_ceil_exponent",
                        lambda a: np.where(np.asarray(a) > 0, np.floor(np.log2(np.where(np.asarray(a) > 0, a, 1) / 448)), 0).astype(np.int64))
    try:
        test_e8m0_golden()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "e8m0_ceil_exponent", real)
    # weight scale read transposed (K-block index used as N-block index)
    real_dw = o.dequantize_weight

    def wrong_dw(q, scale):
        return real_dw(q, np.ascontiguousarray(np.swapaxes(scale, 1, 2)) if scale.shape[1] == scale.shape[2] else scale[:, ::-1])
    monkeypatch.setattr(o, "dequantize_weight", wrong_dw)
    try:
        test_contiguous_gemm_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "dequantize_weight", real_dw)
    # B used untransposed-by-group: group index off by one
    real_gc = o.grouped_gemm_contiguous

    def wrong_gc(qa, sa, qb, sb, layout, d_init=None):
        return real_gc(qa, sa, qb[::-1].copy(), sb[::-1].copy(), layout, d_init)
    monkeypatch.setattr(o, "grouped_gemm_contiguous", wrong_gc)
    try:
        test_contiguous_gemm_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "grouped_gemm_contiguous", real_gc)
    # truncating encoder: round toward zero instead of to nearest even
    real_enc = o.encode_e4m3_rne

    def trunc_enc(x):
        c = real_enc(x)
        over = np.abs(o.decode_e4m3(c)) > np.abs(np.asarray(x, np.float64))
        return np.where(over, c - 1, c).astype(np.uint8)
    monkeypatch.setattr(o, "encode_e4m3_rne", trunc_enc)
    try:
        test_encode_bruteforce_sample()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "encode_e4m3_rne", real_enc)
    # activation scale dropped in the dequantization
    real_da = o.dequantize_act
    monkeypatch.setattr(o, "dequantize_act", lambda q, s: o.decode_e4m3(q))
    try:
        test_contiguous_gemm_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "dequantize_act", real_da)
    # E8M0 bias off by one (2^(b-128))
    real_ev = o.e8m0_value
    monkeypatch.setattr(o, "e8m0_value", lambda b: real_ev(b) / 2)
    try:
        test_masked_gemm_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "e8m0_value", real_ev)
    # masked op computing every row of the group buffer, not only m < masked_m
    real_gm = o.grouped_gemm_masked

    def wrong_gm(qa, sa, qb, sb, masked_m, d_init=None):
        return real_gm(qa, sa, qb, sb, np.full_like(np.asarray(masked_m), qa.shape[1]), d_init)
    monkeypatch.setattr(o, "grouped_gemm_masked", wrong_gm)
    try:
        test_masked_gemm_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "grouped_gemm_masked", real_gm)
    assert failures == 7


# ------------------------------------------------------------------ gemm1 + silu_mul pins
def test_silu_closed_forms():
    """silu against what mathematics fixes independently of its formula:
    silu(0) = 0; silu(1) = 1/(1 + 1/e) and silu(-1) = silu(1) - 1 (printed
    constants); the odd part silu(x) - silu(-x) = x; the tanh form
    x * (1 + tanh(x/2)) / 2; scipy's logistic function; the limits at large |x|."""
    import scipy.special
    assert o.silu(np.array(0.0)) == 0.0
    assert abs(float(o.silu(np.array(1.0))) - 0.7310585786300049) < 1e-15
    assert abs(float(o.silu(np.array(-1.0))) + 0.2689414213699951) < 1e-15
    x = np.linspace(-60.0, 60.0, 24001)
    np.testing.assert_allclose(o.silu(x) - o.silu(-x), x, rtol=0, atol=1e-12)
    # (1 + tanh) cancels for large negative x: an absolute bound there
    np.testing.assert_allclose(o.silu(x), x * (1.0 + np.tanh(x / 2.0)) / 2.0, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o.silu(x), x * scipy.special.expit(x), rtol=1e-13, atol=1e-300)
    big = np.array([-1000.0, -800.0, 800.0])
    got = o.silu(big)
    assert got[0] == 0.0 and got[1] == 0.0 and got[2] == 800.0


def _tanh_silu(v: float) -> float:
    return v * (1.0 + math.tanh(v / 2.0)) / 2.0


def test_silu_mul_contiguous_bruteforce_tiny():
    """Gate rows [0, I) and up rows [I, 2I) of each expert's B: every valid row
    against an fsum triple loop and the tanh form of silu; padding rows keep
    the initial buffer."""
    rng = np.random.default_rng(21)
    layout = np.array([1, 1, -1, 0, 0, 0, -1, 1], np.int32)
    K, I = 256, 128
    a = rng.standard_normal((layout.size, K)).astype(np.float32)
    b = rng.standard_normal((2, 2 * I, K)).astype(np.float32)
    qa, sa = o.quantize_act_1x128(a)
    qb, sb = o.quantize_weight_128x128(b)
    out0 = np.full((layout.size, I), 9.25)
    out = o.grouped_gemm_silu_mul_contiguous(qa, sa, qb, sb, layout, out0)
    assert out.shape == (layout.size, I)
    for g in range(2):
        rows = [r for r in range(layout.size) if layout[r] == g]
        h = _bf_gemm_rows(qa, sa, qb, sb, rows, g)
        for i, r in enumerate(rows):
            for n in range(0, I, 7):
                ref = _tanh_silu(h[i, n]) * h[i, I + n]
                assert abs(out[r, n] - ref) <= 1e-12 * max(1.0, abs(ref))
    assert np.all(out[layout < 0] == 9.25)


def test_silu_mul_masked_bruteforce_tiny():
    rng = np.random.default_rng(22)
    G, Mmax, K, I = 3, 5, 256, 128
    a = rng.standard_normal((G, Mmax, K)).astype(np.float32)
    b = rng.standard_normal((G, 2 * I, K)).astype(np.float32)
    masked_m = np.array([2, 5, 0], np.int32)
    qa, sa = o.quantize_act_masked(a)
    qb, sb = o.quantize_weight_128x128(b)
    out0 = np.full((G, Mmax, I), -1.5)
    out = o.grouped_gemm_silu_mul_masked(qa, sa, qb, sb, masked_m, out0)
    assert out.shape == (G, Mmax, I)
    for g in range(G):
        mm = int(masked_m[g])
        if mm:
            h = _bf_gemm_rows(qa[g], sa[g], qb, sb, list(range(mm)), g)
            for m in range(mm):
                for n in range(0, I, 11):
                    ref = _tanh_silu(h[m, n]) * h[m, I + n]
                    assert abs(out[g, m, n] - ref) <= 1e-12 * max(1.0, abs(ref))
        assert np.all(out[g, mm:] == -1.5)


def test_silu_mul_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible gemm1 mistakes in the oracle (on the CPU): gate and up
    halves exchanged, the x factor of silu dropped (a bare sigmoid), and the
    activation applied to every row including padding."""
    failures = 0
    real_rows = o._silu_mul_rows

    def swapped(d):
        half = d.shape[-1] // 2
        return o.silu(d[..., half:]) * d[..., :half]
    monkeypatch.setattr(o, "_silu_mul_rows", swapped)
    try:
        test_silu_mul_contiguous_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "_silu_mul_rows", real_rows)
    real_silu = o.silu
    monkeypatch.setattr(o, "silu", lambda x: 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64))))
    try:
        test_silu_mul_masked_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "silu", real_silu)
    real_gc = o.grouped_gemm_contiguous

    def all_rows(qa, sa, qb, sb, layout, d_init=None):
        return real_gc(qa, sa, qb, sb, np.where(np.asarray(layout) < 0, 0, layout), d_init)
    monkeypatch.setattr(o, "grouped_gemm_contiguous", all_rows)
    real_sc = o.grouped_gemm_silu_mul_contiguous

    def silu_all_rows(qa, sa, qb, sb, layout, out_init=None):
        return real_sc(qa, sa, qb, sb, np.where(np.asarray(layout) < 0, 0, layout), out_init)
    monkeypatch.setattr(o, "grouped_gemm_silu_mul_contiguous", silu_all_rows)
    try:
        test_silu_mul_contiguous_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "grouped_gemm_contiguous", real_gc)
    monkeypatch.setattr(o, "grouped_gemm_silu_mul_contiguous", real_sc)
    assert failures == 3


# ------------------------------------------------------------------ MXFP8 (1 x 32) pins
def _bf_even_exponent(a: float, mbits: int, emax: int) -> int:
    """The "Even" scale exponent by brute force: the nearest value with mbits
    fraction bits, found by trying every candidate j * 2**(e - mbits) of a's
    binade [2**e, 2**(e+1)] (ties to the even j), then the integer t with
    2**(t + emax) <= that value < 2**(t + emax + 1) by linear search."""
    if a == 0:
        return 0
    e = next(k for k in range(-200, 200) if 2.0 ** k <= a < 2.0 ** (k + 1))
    step = 2.0 ** (e - mbits)
    best = min((abs(j * step - a), j % 2, j * step) for j in range(2 ** mbits, 2 ** (mbits + 1) + 1))[2]
    return next(k for k in range(-200, 200) if 2.0 ** k <= best < 2.0 ** (k + 1)) - emax


def test_mx_exponent_golden():
    """E4M3 column of the hand-derived "Even" table."""
    rows = _read_golden("mx_e8m0_even.txt", cols=3)
    amax = np.array([float(a) for a, _, _ in rows])
    want = np.array([int(b) for _, b, _ in rows])
    assert np.array_equal(o.mx_exponent(amax) + 127, want)


def test_mx_exponent_bruteforce():
    rng = np.random.default_rng(31)
    p2 = 2.0 ** rng.integers(-100, 100, 50).astype(np.float64)
    amax = np.concatenate([rng.uniform(0, 1, 500) * 10.0 ** rng.uniform(-30, 30, 500), p2, np.nextafter(p2, 0),
                           p2 * 1.9375, np.nextafter(p2 * 1.9375, 0), p2 * 1.96875, p2 * 1.875])
    t = o.mx_exponent(amax)
    for a, ti in zip(amax, t):
        want = _bf_even_exponent(float(a), 3, 8)
        assert ti == want, (a, ti, want)
    with pytest.raises(ValueError):
        o.mx_exponent(np.array([1e-37]))            # t = -131: below E8M0's range


def test_mx_even_scale_bounds_the_scaled_block():
    """What the "Even" rounding buys: the scaled block maximum stays below the
    midpoint above the format's top power of two (E4M3: 496 = 1.9375 * 256;
    E2M1: 7 = 1.75 * 4), and at or above half that power's binade."""
    rng = np.random.default_rng(35)
    amax = rng.uniform(0, 1, 2000) * 10.0 ** rng.uniform(-20, 20, 2000)
    for fn, hi, lo in ((o.mx_exponent, 496.0, 128.0), (o.mx4_exponent, 7.0, 2.0)):
        v = amax / np.exp2(fn(amax).astype(np.float64))
        assert np.all(v < hi) and np.all(v >= lo)


def _bf_quant_mx(x):
    """Per row, per 32-wide block: brute-force "Even" exponent, clamp, exhaustive RNE encode."""
    R, K = x.shape
    q = np.zeros((R, K), np.uint8)
    s = np.zeros((K // 32, R), np.uint8)
    for r in range(R):
        for j in range(K // 32):
            blk = [float(v) for v in x[r, 32 * j:32 * j + 32]]
            amax = max(abs(v) for v in blk)
            t = _bf_even_exponent(amax, 3, 8)
            s[j, r] = t + 127
            for i, v in enumerate(blk):
                q[r, 32 * j + i] = _bf_encode(min(max(v / 2.0 ** t, -448.0), 448.0))
    return q, s


def test_mx_quantizer_bruteforce_tiny():
    """Ragged magnitudes, an all-zero block, blocks whose scaled maximum lies
    in (448, 496) (saturating to +-448), and a block whose amax rounds up to
    the next power of two (the larger scale, no saturation)."""
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((5, 128)) * 10.0 ** rng.uniform(-3, 3, (5, 1))).astype(np.float32)
    x[1, 32:64] = 0.0
    x[2, 64:96] = rng.uniform(-1, 1, 32).astype(np.float32) * 7.0
    x[2, 70] = 7.5             # 1.875 * 4: t = -6, scaled 480, saturates to 448
    x[3, 0:32] = np.float32(460.0)
    x[3, 5] = np.float32(-470.0)   # amax 470 = 1.836 * 256: t = 0, +-460/470 saturate to +-448
    x[4, 96:128] = np.float32(1.0)
    x[4, 100] = np.float32(-7.75)  # 1.9375 * 4 rounds to 8: t = -5, -7.75 * 32 = -248 -> -256
    q, s = o.quantize_mx_1x32(x)
    bq, bs = _bf_quant_mx(x)
    assert np.array_equal(s, bs)
    assert np.array_equal(q, bq)
    assert q[2, 70] == 0x7E                               # saturated to 448
    assert q[3, 0] == 0x7E and q[3, 5] == 0xFE           # saturated to +-448
    assert s[3, 4] == 122 and q[4, 100] == 0xF8          # t = -5; -256 = -(2^8)


def _bf_mx_gemm_rows(qa, sa, qb, sb, rows_a, g):
    """fsum triple loop with per-32 scales on both operands."""
    N, K = qb.shape[1], qb.shape[2]
    out = np.zeros((len(rows_a), N))
    for i, r in enumerate(rows_a):
        a = [_val(qa[r, k]) * 2.0 ** (int(sa[k // 32, r]) - 127) for k in range(K)]
        for n in range(N):
            out[i, n] = math.fsum(a[k] * _val(qb[g, n, k]) * 2.0 ** (int(sb[g, k // 32, n]) - 127)
                                  for k in range(K))
    return out


def test_mx_contiguous_gemm_bruteforce_tiny():
    rng = np.random.default_rng(33)
    layout = np.array([0, -1, 1, 1, 0, -1], np.int32)
    K, N = 96, 40
    a = (rng.standard_normal((layout.size, K)) * 10.0 ** rng.uniform(-2, 2, (layout.size, 1))).astype(np.float32)
    b = rng.standard_normal((2, N, K)).astype(np.float32)
    qa, sa = o.quantize_mx_1x32(a)
    qb, sb = o.quantize_mx_1x32(b)
    assert sa.shape == (K // 32, layout.size) and sb.shape == (2, K // 32, N)
    d = o.grouped_gemm_mx_contiguous(qa, sa, qb, sb, layout, np.full((layout.size, N), 5.5))
    for g in range(2):
        rows = [r for r in range(layout.size) if layout[r] == g]
        np.testing.assert_allclose(d[rows], _bf_mx_gemm_rows(qa, sa, qb, sb, rows, g), rtol=1e-12, atol=1e-12)
    assert np.all(d[layout < 0] == 5.5)


def test_mx_masked_gemm_bruteforce_tiny():
    rng = np.random.default_rng(34)
    G, Mmax, K, N = 2, 4, 64, 24
    a = rng.standard_normal((G, Mmax, K)).astype(np.float32)
    b = rng.standard_normal((G, N, K)).astype(np.float32)
    masked_m = np.array([3, 1], np.int32)
    qa, sa = o.quantize_mx_1x32(a)
    qb, sb = o.quantize_mx_1x32(b)
    assert sa.shape == (G, K // 32, Mmax)
    d = o.grouped_gemm_mx_masked(qa, sa, qb, sb, masked_m, np.full((G, Mmax, N), -2.0))
    for g in range(G):
        mm = int(masked_m[g])
        np.testing.assert_allclose(d[g, :mm], _bf_mx_gemm_rows(qa[g], sa[g], qb, sb, list(range(mm)), g),
                                   rtol=1e-12, atol=1e-12)
        assert np.all(d[g, mm:] == -2.0)


def test_mx_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible MX mistakes in the oracle (on the CPU): the ceil rule of
    the (1,128) path instead of "Even", the plain floor rule (no rounding of
    amax) instead of "Even", scales applied per 128 instead of per 32, and no
    saturation before encoding."""
    failures = 0
    real_exp = o.mx_exponent
    monkeypatch.setattr(o, "mx_exponent", lambda a: o.e8m0_ceil_exponent(a))
    try:
        test_mx_exponent_golden()
    except AssertionError:
        failures += 1

    def floor_rule(a):
        a = np.asarray(a, np.float64)
        _, p = np.frexp(np.where(a > 0, a, 1.0))
        return np.where(a > 0, p.astype(np.int64) - 1 - 8, 0)
    monkeypatch.setattr(o, "mx_exponent", floor_rule)
    for pin in (test_mx_exponent_golden, test_mx_quantizer_bruteforce_tiny):
        try:
            pin()
        except AssertionError:
            failures += 1
    monkeypatch.setattr(o, "mx_exponent", real_exp)
    real_dq = o.dequantize_mx

    def per128(q, scale_t):
        st = np.repeat(np.take(scale_t, np.arange(0, scale_t.shape[-2], 4), axis=-2), 4, axis=-2)
        return real_dq(q, st[..., :scale_t.shape[-2], :])
    monkeypatch.setattr(o, "dequantize_mx", per128)
    try:
        test_mx_contiguous_gemm_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "dequantize_mx", real_dq)
    real_clip = np.clip
    monkeypatch.setattr(o.np, "clip", lambda v, lo, hi: v)
    try:
        test_mx_quantizer_bruteforce_tiny()
    except (AssertionError, ValueError):
        failures += 1
    monkeypatch.setattr(o.np, "clip", real_clip)
    assert failures == 5


# ------------------------------------------------------------------ MXFP4 (E2M1) pins
def test_e2m1_decode_golden():
    rows = _read_golden("e2m1_codes.txt")
    codes = np.array([int(c, 16) for c, _ in rows])
    vals = np.array([float(v) for _, v in rows])
    got = o.decode_e2m1(codes)
    assert np.array_equal(got, vals) and np.array_equal(np.signbit(got), np.signbit(vals))


def _bf_e2m1(v: float) -> int:
    """Nearest E2M1 code by exhaustive search over the 16 codes; ties to the even code."""
    table = [(c, float(o.decode_e2m1(np.array(c)))) for c in range(16)]
    neg = math.copysign(1.0, v) < 0
    best = None
    for c, val in table:
        if val == 0.0 and bool(c >> 3) != neg:
            continue                     # keep the sign of zero
        key = (abs(val - v), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_e2m1_encode_bruteforce():
    rng = np.random.default_rng(51)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    x = np.concatenate([rng.uniform(-6, 6, 3000), np.array(mids), -np.array(mids),
                        np.array([0.0, -0.0, 6.0, -6.0, 5.999, 0.2500001, 0.2499999])])
    got = o.encode_e2m1_rne(x)
    want = np.array([_bf_e2m1(float(v)) for v in x])
    assert np.array_equal(got, want)
    with pytest.raises(ValueError):
        o.encode_e2m1_rne(np.array([6.5]))


def test_mx4_exponent_golden():
    """E2M1 column of the hand-derived "Even" table."""
    rows = _read_golden("mx_e8m0_even.txt", cols=3)
    amax = np.array([float(a) for a, _, _ in rows])
    want = np.array([int(c) for _, _, c in rows])
    assert np.array_equal(o.mx4_exponent(amax) + 127, want)


def test_mx4_exponent_bruteforce():
    rng = np.random.default_rng(52)
    p2 = 2.0 ** rng.integers(-100, 100, 40).astype(np.float64)
    amax = np.concatenate([rng.uniform(0, 1, 400) * 10.0 ** rng.uniform(-30, 30, 400), p2, p2 * 1.75,
                           np.nextafter(p2 * 1.75, 0), p2 * 1.5, p2 * 1.25,
                           np.array([0.0, 4.0, 6.0, 6.999, 7.0, 7.999, 8.0])])
    t = o.mx4_exponent(amax)
    for a, ti in zip(amax, t):
        want = _bf_even_exponent(float(a), 1, 2)
        assert ti == want, (a, ti, want)


def _bf_quant_mx4(x):
    R, K = x.shape
    q = np.zeros((R, K // 2), np.uint8)
    s = np.zeros((K // 32, R), np.uint8)
    for r in range(R):
        for j in range(K // 32):
            blk = [float(v) for v in x[r, 32 * j:32 * j + 32]]
            amax = max(abs(v) for v in blk)
            t = _bf_even_exponent(amax, 1, 2)
            s[j, r] = t + 127
            for i, v in enumerate(blk):
                k = 32 * j + i
                c = _bf_e2m1(min(max(v / 2.0 ** t, -6.0), 6.0))
                q[r, k // 2] |= c << (4 * (k % 2))      # element 2i: low nibble of byte i
    return q, s


def test_mx4_quantizer_bruteforce_tiny():
    rng = np.random.default_rng(53)
    x = (rng.standard_normal((4, 96)) * 10.0 ** rng.uniform(-3, 3, (4, 1))).astype(np.float32)
    x[1, 32:64] = 0.0
    x[2, 0:32] = np.float32(6.5)        # amax 6.8 = 1.7 * 4: t = 0, 6.5 saturates to 6
    x[2, 3] = np.float32(-6.8)
    x[3, 64:96] = np.float32(0.5)
    x[3, 70] = np.float32(7.0)          # 1.75 * 4 rounds to 8: t = 1; 7 / 2 = 3.5 -> 4 (tie, even code)
    q, s = o.quantize_mx4_1x32(x)
    bq, bs = _bf_quant_mx4(x)
    assert np.array_equal(s, bs) and np.array_equal(q, bq)
    assert q[2, 0] == 0x77 and (q[2, 1] >> 4) == 0xF
    assert s[2, 3] == 128 and (q[3, 35] & 15) == 6      # code 6 = 4.0


def test_mx4_dequantize_nibble_order():
    """Byte 0x21 holds element 0 = code 1 (0.5) in its low nibble and element
    1 = code 2 (1.0) in its high nibble; scale byte 128 doubles both.  (A
    swap applied to both GEMM operands alike cancels in the dot product, so
    the order is pinned here directly.)"""
    q = np.zeros((1, 16), np.uint8)
    q[0, 0] = 0x21
    q[0, 15] = 0xF7                       # element 30 = 6.0, element 31 = -6.0
    got = o.dequantize_mx4(q, np.array([[128]], np.uint8))
    assert got[0, 0] == 1.0 and got[0, 1] == 2.0
    assert got[0, 30] == 12.0 and got[0, 31] == -12.0
    assert np.all(got[0, 2:30] == 0.0)


def _bf_mx4_gemm_rows(qa, sa, qb, sb, rows_a, g):
    N, Kh = qb.shape[1], qb.shape[2]
    val = lambda byte, k: float(o.decode_e2m1(np.array((int(byte) >> (4 * (k % 2))) & 15)))
    out = np.zeros((len(rows_a), N))
    for i, r in enumerate(rows_a):
        a = [val(qa[r, k // 2], k) * 2.0 ** (int(sa[k // 32, r]) - 127) for k in range(2 * Kh)]
        for n in range(N):
            out[i, n] = math.fsum(a[k] * val(qb[g, n, k // 2], k) * 2.0 ** (int(sb[g, k // 32, n]) - 127)
                                  for k in range(2 * Kh))
    return out


def test_mx4_contiguous_gemm_bruteforce_tiny():
    rng = np.random.default_rng(54)
    layout = np.array([1, 1, -1, 0, 0], np.int32)
    K, N = 64, 24
    a = rng.standard_normal((layout.size, K)).astype(np.float32)
    b = rng.standard_normal((2, N, K)).astype(np.float32)
    qa, sa = o.quantize_mx4_1x32(a)
    qb, sb = o.quantize_mx4_1x32(b)
    assert qa.shape == (layout.size, K // 2) and sb.shape == (2, K // 32, N)
    d = o.grouped_gemm_mx4_contiguous(qa, sa, qb, sb, layout, np.full((layout.size, N), 1.25))
    for g in range(2):
        rows = [r for r in range(layout.size) if layout[r] == g]
        np.testing.assert_allclose(d[rows], _bf_mx4_gemm_rows(qa, sa, qb, sb, rows, g), rtol=1e-12, atol=1e-12)
    assert np.all(d[layout < 0] == 1.25)


def test_mx4_masked_gemm_bruteforce_tiny():
    rng = np.random.default_rng(55)
    G, Mmax, K, N = 2, 3, 64, 16
    a = rng.standard_normal((G, Mmax, K)).astype(np.float32)
    b = rng.standard_normal((G, N, K)).astype(np.float32)
    masked_m = np.array([2, 3], np.int32)
    qa, sa = o.quantize_mx4_1x32(a)
    qb, sb = o.quantize_mx4_1x32(b)
    d = o.grouped_gemm_mx4_masked(qa, sa, qb, sb, masked_m, np.full((G, Mmax, N), 7.0))
    for g in range(G):
        mm = int(masked_m[g])
        np.testing.assert_allclose(d[g, :mm], _bf_mx4_gemm_rows(qa[g], sa[g], qb, sb, list(range(mm)), g),
                                   rtol=1e-12, atol=1e-12)
        assert np.all(d[g, mm:] == 7.0)


def test_mx4_pins_catch_planted_mistakes(monkeypatch):
    """Planted MXFP4 mistakes (on the CPU): nibbles in the wrong order, the
    FP8 exponent rule instead of FP4's, the plain floor rule (no rounding of
    amax) instead of "Even", and no saturation."""
    failures = 0
    real_dq = o.dequantize_mx4

    def swapped(q, scale_t):
        q = np.asarray(q, np.uint8)
        return real_dq(((q << 4) | (q >> 4)).astype(np.uint8), scale_t)
    monkeypatch.setattr(o, "dequantize_mx4", swapped)
    try:
        test_mx4_dequantize_nibble_order()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "dequantize_mx4", real_dq)
    real_exp = o.mx4_exponent
    monkeypatch.setattr(o, "mx4_exponent", lambda a: o.mx_exponent(a))
    try:
        test_mx4_exponent_bruteforce()
    except AssertionError:
        failures += 1

    def floor_rule(a):
        a = np.asarray(a, np.float64)
        _, p = np.frexp(np.where(a > 0, a, 1.0))
        return np.where(a > 0, p.astype(np.int64) - 1 - 2, 0)
    monkeypatch.setattr(o, "mx4_exponent", floor_rule)
    for pin in (test_mx4_exponent_golden, test_mx4_quantizer_bruteforce_tiny):
        try:
            pin()
        except AssertionError:
            failures += 1
    monkeypatch.setattr(o, "mx4_exponent", real_exp)
    real_clip = np.clip
    monkeypatch.setattr(o.np, "clip", lambda v, lo, hi: v)
    try:
        test_mx4_quantizer_bruteforce_tiny()
    except (AssertionError, ValueError):
        failures += 1
    monkeypatch.setattr(o.np, "clip", real_clip)
    assert failures == 5


# ------------------------------------------------------------------ a4w4 gemm1 with silu_mul pins
def test_mx4_silu_mul_contiguous_bruteforce_tiny():
    """Every valid row against an fsum loop over E2M1 nibbles and the tanh
    form of silu: gate rows [0, I), up rows [I, 2I); padding rows keep the
    initial buffer."""
    rng = np.random.default_rng(61)
    layout = np.array([0, -1, 1, 1, 0, -1], np.int32)
    K, I = 64, 12
    a = rng.standard_normal((layout.size, K)).astype(np.float32)
    b = rng.standard_normal((2, 2 * I, K)).astype(np.float32)
    qa, sa = o.quantize_mx4_1x32(a)
    qb, sb = o.quantize_mx4_1x32(b)
    out = o.grouped_gemm_mx4_silu_mul_contiguous(qa, sa, qb, sb, layout, np.full((layout.size, I), 3.5))
    assert out.shape == (layout.size, I)
    for g in range(2):
        rows = [r for r in range(layout.size) if layout[r] == g]
        h = _bf_mx4_gemm_rows(qa, sa, qb, sb, rows, g)
        for i, r in enumerate(rows):
            for n in range(I):
                ref = _tanh_silu(h[i, n]) * h[i, I + n]
                assert abs(out[r, n] - ref) <= 1e-12 * max(1.0, abs(ref))
    assert np.all(out[layout < 0] == 3.5)


def test_mx4_silu_mul_masked_bruteforce_tiny():
    rng = np.random.default_rng(62)
    G, Mmax, K, I = 3, 4, 64, 8
    a = rng.standard_normal((G, Mmax, K)).astype(np.float32)
    b = rng.standard_normal((G, 2 * I, K)).astype(np.float32)
    masked_m = np.array([3, 0, 4], np.int32)
    qa, sa = o.quantize_mx4_1x32(a)
    qb, sb = o.quantize_mx4_1x32(b)
    out = o.grouped_gemm_mx4_silu_mul_masked(qa, sa, qb, sb, masked_m, np.full((G, Mmax, I), -2.0))
    assert out.shape == (G, Mmax, I)
    for g in range(G):
        mm = int(masked_m[g])
        if mm:
            h = _bf_mx4_gemm_rows(qa[g], sa[g], qb, sb, list(range(mm)), g)
            for m in range(mm):
                for n in range(I):
                    ref = _tanh_silu(h[m, n]) * h[m, I + n]
                    assert abs(out[g, m, n] - ref) <= 1e-12 * max(1.0, abs(ref))
        assert np.all(out[g, mm:] == -2.0)


def test_mx4_silu_mul_pins_catch_planted_mistakes(monkeypatch):
    """Planted a4w4 gemm1 mistakes (on the CPU): gate and up halves
    exchanged, the FP8 element decode in place of E2M1's, and padding rows
    given outputs."""
    failures = 0
    real_rows = o._silu_mul_rows

    def swapped(d):
        half = d.shape[-1] // 2
        return o.silu(d[..., half:]) * d[..., :half]
    monkeypatch.setattr(o, "_silu_mul_rows", swapped)
    try:
        test_mx4_silu_mul_contiguous_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "_silu_mul_rows", real_rows)
    real_gm = o.grouped_gemm_mx4_masked

    def fp8_decode(qa, sa, qb, sb, masked_m, d_init=None):
        G, Mmax, _ = qa.shape
        codes = np.stack([qb & 15, qb >> 4], axis=-1).reshape(*qb.shape[:-1], 2 * qb.shape[-1])
        b = o.decode_e4m3(codes.astype(np.uint8)) * np.repeat(np.swapaxes(o.e8m0_value(sb), -1, -2), 32, axis=-1)
        d = np.full((G, Mmax, b.shape[1]), np.nan)
        for g in range(G):
            mm = int(masked_m[g])
            if mm:
                d[g, :mm] = o.dequantize_mx4(qa[g, :mm], sa[g][:, :mm]) @ b[g].T
        return d
    monkeypatch.setattr(o, "grouped_gemm_mx4_masked", fp8_decode)
    try:
        test_mx4_silu_mul_masked_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "grouped_gemm_mx4_masked", real_gm)
    real_sc = o.grouped_gemm_mx4_silu_mul_contiguous

    def all_rows(qa, sa, qb, sb, layout, out_init=None):
        return real_sc(qa, sa, qb, sb, np.where(np.asarray(layout) < 0, 0, layout), out_init)
    monkeypatch.setattr(o, "grouped_gemm_mx4_silu_mul_contiguous", all_rows)
    try:
        test_mx4_silu_mul_contiguous_bruteforce_tiny()
    except AssertionError:
        failures += 1
    monkeypatch.setattr(o, "grouped_gemm_mx4_silu_mul_contiguous", real_sc)
    assert failures == 3
