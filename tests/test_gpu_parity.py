"""GPU parity: the HIP path (through the C-ABI) against the fp64 CPU oracle.

The bar (stated for this path): calc_diff <= 1e-5 and row-floored max
relative error <= 1e-2 over valid rows; padding and masked-off rows keep the
caller's sentinel bit for bit; the exact-integer case matches the correctly
rounded result bit for bit; repeated calls are bit-identical.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as gfg
from fp8_block_scaled_amd import workloads as wl
from oracle import fp8_oracle as o
from parity_utils import (SENTINEL, bits, check_close, gpu_contiguous, gpu_masked, sentinel_bits,
                          to_dev, torch_dtype)

pytestmark = pytest.mark.gpu


def _contig_case(x, out_dtype):
    qa, sa = gfg.fp8_quantize_act_1x128(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    d = gpu_contiguous(qa, sa, qb, sb, x["grouped_layout"], out_dtype)
    oqa, osa = o.quantize_act_1x128(x["a"])
    oqb, osb = o.quantize_weight_128x128(x["b"])
    ref = o.grouped_gemm_contiguous(oqa, osa, oqb, osb, x["grouped_layout"])
    return d, ref


def _check_contig(d, ref, layout, out_dtype, what):
    got = d.float().cpu().numpy()
    valid = (layout >= 0)
    if valid.any():
        check_close(got[valid], ref[valid], what)
    b = bits(d)
    assert np.all(b[~valid] == sentinel_bits(out_dtype)), f"{what}: padding rows were written"


def test_small_workload_full_compare():
    w = wl.workload(0)
    x = wl.draw(w)
    d, ref = _contig_case(x, w.out_dtype)
    _check_contig(d, ref, x["grouped_layout"], w.out_dtype, w.name)


@pytest.mark.parametrize("m_per_group,N,K,out", [
    ([100, 1, 128, 129, 300], 384, 256, "bf16"),     # 128-wide N tiles, several groups, ragged
    ([5, 250], 512, 384, "f16"),                     # 256-wide N tiles, f16 out
    ([0, 128, 77], 256, 128, "bf16"),                # an empty group, a single K step
    ([1000, 30], 1280, 640, "bf16"),                 # many M tiles, 5 N tiles
    ([513, 2, 64, 700, 1, 129, 256, 90], 256, 512, "f16"),
])
def test_small_contiguous_ragged(m_per_group, N, K, out):
    x = wl.small_contiguous(sum(m_per_group) + N + K, m_per_group, N, K)
    d, ref = _contig_case(x, out)
    _check_contig(d, ref, x["grouped_layout"], out, f"contig {m_per_group} N={N} K={K}")


def test_overpadded_contiguous_layout():
    """Whole padding tiles before, between and after experts are skipped."""
    rng = np.random.default_rng(21)
    parts = [np.full(256, -1), np.full(100, 0), np.full(28, -1), np.full(384, -1),
             np.full(128, 1), np.full(60, 2), np.full(68, -1), np.full(512, -1)]
    layout = np.concatenate(parts).astype(np.int32)
    K, N = 256, 256
    a = rng.standard_normal((layout.size, K)).astype(np.float32)
    b = rng.standard_normal((3, N, K)).astype(np.float32)
    x = dict(a=a, b=b, grouped_layout=layout)
    d, ref = _contig_case(x, "bf16")
    _check_contig(d, ref, layout, "bf16", "overpadded")


@pytest.mark.parametrize("M,N", [(158, 512), (157, 384)])
def test_contiguous_unpadded_tail(M, N):
    """The last expert's run is cut short of a 128 multiple, so M is not a
    multiple of 4 and the A-scale rows are not dword aligned (byte-wise scale
    path); rows past M do not exist."""
    rng = np.random.default_rng(23 + M)
    layout = np.concatenate([np.full(100, 0), np.full(28, -1), np.full(M - 128, 1)]).astype(np.int32)
    K = 384
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[layout < 0] = 0.0
    b = rng.standard_normal((2, N, K)).astype(np.float32)
    x = dict(a=a, b=b, grouped_layout=layout)
    d, ref = _contig_case(x, "bf16")
    _check_contig(d, ref, layout, "bf16", f"unpadded tail M={M} N={N}")


def test_out_of_range_expert_ids_are_padding():
    rng = np.random.default_rng(22)
    layout = np.concatenate([np.full(128, 0), np.full(128, 7), np.full(128, -3), np.full(128, 1)]).astype(np.int32)
    a = rng.standard_normal((layout.size, 256)).astype(np.float32)
    b = rng.standard_normal((2, 256, 256)).astype(np.float32)
    x = dict(a=a, b=b, grouped_layout=layout)
    d, ref = _contig_case(x, "bf16")
    _check_contig(d, ref, np.where((layout >= 0) & (layout < 2), layout, -1), "bf16", "ids")


@pytest.mark.parametrize("masked_m,Mmax,N,K,out", [
    ([0, 1, 127, 128, 129, 200], 200, 256, 256, "bf16"),   # M_max not a multiple of 128
    ([300, 0, 512], 512, 384, 384, "f16"),
    ([-5, 700, 64], 256, 512, 128, "bf16"),                 # clamped into [0, M_max]
    ([130, 5, 77], 130, 512, 256, "bf16"),                  # M_max % 4 != 0: byte-wise A scales
    ([3, 0, 201], 201, 256, 384, "f16"),
])
def test_small_masked(masked_m, Mmax, N, K, out):
    x = wl.small_masked(Mmax + N + K, masked_m, Mmax, N, K)
    qa, sa = gfg.fp8_quantize_act_masked(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    d = gpu_masked(qa, sa, qb, sb, masked_m, out)
    oqa, osa = o.quantize_act_masked(x["a"])
    oqb, osb = o.quantize_weight_128x128(x["b"])
    ref = o.grouped_gemm_masked(oqa, osa, oqb, osb, masked_m)
    got = d.float().cpu().numpy()
    b = bits(d)
    for g, m in enumerate(masked_m):
        mm = min(max(m, 0), Mmax)
        if mm:
            check_close(got[g, :mm], ref[g, :mm], f"masked g={g}")
        assert np.all(b[g, mm:] == sentinel_bits(out)), f"masked g={g}: rows >= masked_m written"


def _int_codes(ints):
    table = {}
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e4m3_small_integers.txt")
    for line in open(path):
        line = line.split("#", 1)[0].split()
        if line:
            table[int(line[0])] = int(line[1], 16)
    return np.vectorize(table.get)(ints).astype(np.uint8)


@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_exact_integer_case_bitwise(out):
    """Integer operands, power-of-two scales: every fp32 partial sum is exact, so the
    GPU output must equal the correctly rounded exact product bit for bit."""
    case = wl.integer_case(31, G=3, rows=128, N=512, K=384, vmax=4 if out == "bf16" else 2)
    qa, qb = _int_codes(case["ints_a"]), _int_codes(case["ints_b"])
    d = gpu_contiguous(qa, case["scale_a"], qb, case["scale_b"], case["grouped_layout"], out)
    ref = o.grouped_gemm_contiguous(qa, case["scale_a"], qb, case["scale_b"], case["grouped_layout"])
    assert np.all(np.abs(ref) < 2 ** 24)
    rounded = o.round_to_bf16(ref) if out == "bf16" else o.round_to_f16(ref)
    got = d.double().cpu().numpy()
    assert np.array_equal(got, rounded)


def test_deterministic_and_stream():
    w = wl.workload(0)
    x = wl.draw(w, seed_offset=3)
    qa, sa = gfg.fp8_quantize_act_1x128(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    d1 = gpu_contiguous(qa, sa, qb, sb, x["grouped_layout"], "bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        d2 = torch.full_like(d1, SENTINEL)
        gpu_contiguous(qa, sa, qb, sb, x["grouped_layout"], "bf16", d=d2, stream=s)
    assert np.array_equal(bits(d1), bits(d2))


def test_nan_poisoned_invalid_rows_do_not_leak():
    x = wl.small_contiguous(41, [100, 60], 256, 256)
    layout = x["grouped_layout"]
    qa, sa = gfg.fp8_quantize_act_1x128(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    clean = gpu_contiguous(qa, sa, qb, sb, layout, "bf16")
    qa2, sa2 = qa.copy(), sa.copy()
    qa2[layout < 0] = 0x7F          # e4m3 NaN
    sa2[:, layout < 0] = 0xFF       # E8M0 NaN
    dirty = gpu_contiguous(qa2, sa2, qb, sb, layout, "bf16")
    assert np.array_equal(bits(clean), bits(dirty))
    # masked: poison rows >= masked_m
    xm = wl.small_masked(42, [50, 128, 0], 160, 256, 256)
    qa, sa = gfg.fp8_quantize_act_masked(xm["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(xm["b"])
    clean = gpu_masked(qa, sa, qb, sb, [50, 128, 0], "bf16")
    for g, m in enumerate([50, 128, 0]):
        qa[g, m:] = 0x7F
        sa[g][:, m:] = 0xFF
    dirty = gpu_masked(qa, sa, qb, sb, [50, 128, 0], "bf16")
    assert np.array_equal(bits(clean), bits(dirty))


def test_masked_equals_contiguous_on_same_rows():
    rng = np.random.default_rng(43)
    counts = [128, 77, 0, 256]
    Mmax, N, K = 256, 512, 256
    a_m = rng.standard_normal((4, Mmax, K)).astype(np.float32)
    b = rng.standard_normal((4, N, K)).astype(np.float32)
    layout = wl.contiguous_layout(counts)
    a_c = np.zeros((layout.size, K), np.float32)
    pos = 0
    for g, c in enumerate(counts):
        a_c[pos:pos + c] = a_m[g, :c]
        pos += -(-c // 128) * 128
    qb, sb = gfg.fp8_quantize_weight_128x128(b)
    qa, sa = gfg.fp8_quantize_act_masked(a_m)
    dm = bits(gpu_masked(qa, sa, qb, sb, counts, "bf16"))
    qc, sc = gfg.fp8_quantize_act_1x128(a_c)
    dc = bits(gpu_contiguous(qc, sc, qb, sb, layout, "bf16"))
    pos = 0
    for g, c in enumerate(counts):
        assert np.array_equal(dm[g, :c], dc[pos:pos + c])
        pos += -(-c // 128) * 128


def test_contiguous_maximum_rows():
    """The largest contiguous call the tile list takes: 4096 candidate tiles
    (524,288 rows) over three experts, K = 128, N = 256.  Every valid row
    against the oracle; every padding row keeps the sentinel."""
    rng = np.random.default_rng(71)
    counts = [200_000, 100_001, 224_000]
    layout = wl.contiguous_layout(counts)
    assert layout.size <= 4096 * 128
    layout = np.concatenate([layout, np.full(4096 * 128 - layout.size, -1, np.int32)])
    M, K, N = layout.size, 128, 256
    print(f"[parity] max rows M={M}", flush=True)
    a = rng.standard_normal((M, K), dtype=np.float32)
    a[layout < 0] = 0.0
    b = rng.standard_normal((3, N, K), dtype=np.float32)
    qa, sa = gfg.fp8_quantize_act_1x128(a)
    qb, sb = gfg.fp8_quantize_weight_128x128(b)
    d = gpu_contiguous(qa, sa, qb, sb, layout, "bf16")
    got = d.float().cpu().numpy()
    b_all = bits(d)
    assert np.all(b_all[layout < 0] == sentinel_bits("bf16"))
    del d
    rows = np.nonzero(layout >= 0)[0]
    oqa, osa = o.quantize_act_1x128(a[rows])
    oqb, osb = o.quantize_weight_128x128(b)
    ref = o.grouped_gemm_contiguous(oqa, osa, oqb, osb, layout[rows])
    check_close(got[rows], ref, "max rows")


def test_masked_maximum_tiles():
    """G * ceil(M_max / 128) = 4096 candidate tiles: 32 groups of 16,384 rows,
    masked_m from 0 to M_max.  Every valid row against the oracle."""
    rng = np.random.default_rng(72)
    G, Mmax, K, N = 32, 16384, 128, 256
    masked_m = rng.integers(0, Mmax, size=G, endpoint=True).astype(np.int32)
    masked_m[0], masked_m[1], masked_m[-1] = 0, Mmax, 1
    print(f"[parity] max masked tiles G={G} Mmax={Mmax}", flush=True)
    a = rng.standard_normal((G, Mmax, K), dtype=np.float32)
    b = rng.standard_normal((G, N, K), dtype=np.float32)
    qa, sa = gfg.fp8_quantize_act_masked(a)
    qb, sb = gfg.fp8_quantize_weight_128x128(b)
    d = gpu_masked(qa, sa, qb, sb, masked_m, "bf16")
    b_all = bits(d)
    got = d.float().cpu().numpy()
    del d
    oqa, osa = o.quantize_act_masked(a)
    oqb, osb = o.quantize_weight_128x128(b)
    ref = o.grouped_gemm_masked(oqa, osa, oqb, osb, masked_m)
    gots, refs = [], []
    for g in range(G):
        mm = int(masked_m[g])
        assert np.all(b_all[g, mm:] == sentinel_bits("bf16")), f"group {g}: rows >= masked_m written"
        gots.append(got[g, :mm])
        refs.append(ref[g, :mm])
    check_close(np.concatenate(gots), np.concatenate(refs), "max masked tiles")


def test_all_padding_and_all_masked_off_write_nothing():
    """No valid tile at all: an all-padding contiguous layout and a masked call
    whose masked_m are all zero (or negative) launch and leave the output untouched."""
    rng = np.random.default_rng(73)
    K, N = 256, 256
    layout = np.full(384, -1, np.int32)
    a = rng.standard_normal((384, K)).astype(np.float32)
    b = rng.standard_normal((2, N, K)).astype(np.float32)
    qa, sa = gfg.fp8_quantize_act_1x128(a)
    qb, sb = gfg.fp8_quantize_weight_128x128(b)
    d = gpu_contiguous(qa, sa, qb, sb, layout, "f16")
    assert np.all(bits(d) == sentinel_bits("f16"))
    am = rng.standard_normal((3, 256, K)).astype(np.float32)
    qa, sa = gfg.fp8_quantize_act_masked(am)
    qb, sb = gfg.fp8_quantize_weight_128x128(rng.standard_normal((3, N, K)).astype(np.float32))
    d = gpu_masked(qa, sa, qb, sb, np.array([0, -4, 0], np.int32), "bf16")
    assert np.all(bits(d) == sentinel_bits("bf16"))
