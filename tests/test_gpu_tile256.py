"""GPU parity of the 256 x 256-tile kernel and of the launch settings.

The plain FP8 GEMM calls pick their output tile per launch; these tests force
each shape through grouped_fp8_set_tile_shape and compare with the fp64
oracle at the usual bar (calc_diff <= 1e-5, row-floored max relative error
<= 1e-2, untouched rows bit for bit).  A grid limit makes one workgroup walk
many tiles, which is where a tile's last steps prefetch the next tile's first
stages and its output stores overlap the next tile's start.  The tile-order
settings (XCD split, grouped-M width: the locality mapping of the second
reference page, "[Kernel][MI350] Add cache-aware 8-wave BF16/FP16 GEMM",
sections "Changes" and "Testing") must give bit-identical outputs.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as gfg
from fp8_block_scaled_amd import workloads as wl
from oracle import fp8_oracle as o
from parity_utils import (SENTINEL, bits, check_close, gpu_contiguous, gpu_masked, sentinel_bits, to_dev,
                          torch_dtype)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore_settings():
    yield
    gfg.set_tile_shape(gfg.TILE_AUTO)
    gfg.set_grid_limit(0)
    gfg.set_tile_order(8, 0)


def _contig(x, out, shape):
    gfg.set_tile_shape(shape)
    qa, sa = gfg.fp8_quantize_act_1x128(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    d = gpu_contiguous(qa, sa, qb, sb, x["grouped_layout"], out)
    oqa, osa = o.quantize_act_1x128(x["a"])
    oqb, osb = o.quantize_weight_128x128(x["b"])
    return d, o.grouped_gemm_contiguous(oqa, osa, oqb, osb, x["grouped_layout"])


def _check(d, ref, layout, out, what):
    got = d.float().cpu().numpy()
    valid = layout >= 0
    check_close(got[valid], ref[valid], what)
    assert np.all(bits(d)[~valid] == sentinel_bits(out)), f"{what}: padding rows were written"


@pytest.mark.parametrize("m_per_group,N,K,out,limit,num_xcd", [
    ([256, 512], 512, 256, "bf16", 0, 8),                      # whole 256-row tiles, one K step pair
    ([100, 1, 128, 129, 300, 513], 256, 512, "f16", 0, 8),     # odd runs: 128-row tiles at run ends
    ([1000, 700, 33, 256], 768, 1024, "bf16", 8, 8),           # 8 workgroups walk every tile
    ([300, 129, 1], 512, 256, "bf16", 1, 1),                   # one workgroup, KB = 2
    ([513, 2, 640], 1280, 768, "f16", 3, 1),                   # three workgroups, KB = 6
])
def test_tile256_contiguous(m_per_group, N, K, out, limit, num_xcd):
    gfg.set_grid_limit(limit)
    gfg.set_tile_order(num_xcd, 0)
    x = wl.small_contiguous(sum(m_per_group) + N + K + 7, m_per_group, N, K)
    d, ref = _contig(x, out, gfg.TILE_256x256)
    _check(d, ref, x["grouped_layout"], out, f"256 contig {m_per_group} N={N} K={K} limit={limit}")


@pytest.mark.parametrize("masked_m,Mmax,N,K,out,limit", [
    ([0, 1, 128, 129, 256, 257], 512, 512, 256, "bf16", 0),
    ([512, 3, 300, 0], 512, 768, 512, "f16", 4),
    ([70, 1000, 513], 1024, 256, 1024, "bf16", 1),
    ([-5, 2000, 256], 1024, 512, 256, "bf16", 0),               # negative and oversized masked_m clamp
])
def test_tile256_masked(masked_m, Mmax, N, K, out, limit):
    gfg.set_grid_limit(limit)
    gfg.set_tile_shape(gfg.TILE_256x256)
    x = wl.small_masked(Mmax + N + K, masked_m, Mmax, N, K)
    qa, sa = gfg.fp8_quantize_act_masked(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    d = gpu_masked(qa, sa, qb, sb, masked_m, out)
    oqa, osa = o.quantize_act_masked(x["a"])
    oqb, osb = o.quantize_weight_128x128(x["b"])
    ref = o.grouped_gemm_masked(oqa, osa, oqb, osb, masked_m)
    got, b = d.float().cpu().numpy(), bits(d)
    gots, refs = [], []
    for g, mm in enumerate(masked_m):
        mm = min(max(mm, 0), Mmax)
        assert np.all(b[g, mm:] == sentinel_bits(out)), f"group {g}: rows >= masked_m written"
        gots.append(got[g, :mm])
        refs.append(ref[g, :mm])
    check_close(np.concatenate(gots), np.concatenate(refs), f"256 masked {masked_m} N={N} K={K} limit={limit}")


@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_tile256_exact_integer_case_bitwise(out):
    """Integer operands with scales in {127, 128, 129}: every partial sum is an
    exact small integer, so the output is the correctly rounded exact value."""
    gfg.set_tile_shape(gfg.TILE_256x256)
    gfg.set_grid_limit(2)
    c = wl.integer_case(91, 3, 256, 512, 512)
    enc = lambda v: o.encode_e4m3_rne(v.astype(np.float64))
    qa, qb = enc(c["ints_a"]), enc(c["ints_b"])
    d = gpu_contiguous(qa, c["scale_a"], qb, c["scale_b"], c["grouped_layout"], out)
    exact = o.grouped_gemm_contiguous(qa, c["scale_a"], qb, c["scale_b"], c["grouped_layout"])
    rnd = o.round_to_bf16 if out == "bf16" else o.round_to_f16
    want = torch.from_numpy(rnd(exact)).to(torch_dtype(out))
    assert np.array_equal(bits(d), bits(want))


def test_tile256_unsupported_shapes_refused():
    gfg.set_tile_shape(gfg.TILE_256x256)
    x = wl.small_contiguous(5, [128], 384, 256)            # N not a multiple of 256
    with pytest.raises(gfg.GfgError) as e:
        _contig(x, "bf16", gfg.TILE_256x256)
    assert e.value.code == 2
    x = wl.small_contiguous(6, [128], 256, 384)            # K / 128 odd
    with pytest.raises(gfg.GfgError) as e:
        _contig(x, "bf16", gfg.TILE_256x256)
    assert e.value.code == 2


def test_tile_shapes_agree_and_auto_runs():
    """Both tile shapes and the automatic choice meet the bar on one case that
    spans several tiles of each shape."""
    x = wl.small_contiguous(8, [600, 1000, 129], 1024, 1024)
    outs = {}
    for shape in (gfg.TILE_128x256, gfg.TILE_256x256, gfg.TILE_AUTO):
        d, ref = _contig(x, "bf16", shape)
        _check(d, ref, x["grouped_layout"], "bf16", f"shape {shape}")
        outs[shape] = d


@pytest.mark.parametrize("shape", [1, 2])
def test_locality_ablation_bit_identical(shape):
    """The four tile orders of the locality ablation (num_xcd 1 or 8 x
    group_m 1 or 4) compute each tile identically: outputs bit for bit equal."""
    gfg.set_tile_shape(shape)
    gfg.set_grid_limit(16)
    x = wl.small_contiguous(9, [700, 300, 1024, 77], 1024, 512)
    qa, sa = gfg.fp8_quantize_act_1x128(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    ref_bits = None
    for nx in (1, 8):
        for gm in (1, 4):
            gfg.set_tile_order(nx, gm)
            d = gpu_contiguous(qa, sa, qb, sb, x["grouped_layout"], "bf16")
            b = bits(d)
            if ref_bits is None:
                ref_bits = b
                oqa, osa = o.quantize_act_1x128(x["a"])
                oqb, osb = o.quantize_weight_128x128(x["b"])
                ref = o.grouped_gemm_contiguous(oqa, osa, oqb, osb, x["grouped_layout"])
                _check(d, ref, x["grouped_layout"], "bf16", f"ablation shape {shape}")
            assert np.array_equal(b, ref_bits), f"num_xcd={nx} group_m={gm} differs"
