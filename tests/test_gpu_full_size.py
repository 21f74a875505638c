"""GPU parity at full size, every output compared.

Each workload runs once on the GPU in the launch configuration the benchmark
times (every expert's weights in their own device buffers), then the oracle
recomputes all of its valid outputs, one chunk at a time so that no single
test holds more than a slice of the fp64 work: a chunk is one expert (one
group for the masked layout), or, for the workloads whose 385 experts share 8
weight draws, the rows of every expert that uses one draw.  Per chunk:

  * the library's quantized bytes (A rows, their scales, the chunk's B and
    its scales) equal the oracle's quantizer's bytes;
  * every valid output meets the bar: calc_diff <= 1e-5 and row-floored max
    relative error <= 1e-2 (tests/parity_utils.py);
  * no valid output still holds the sentinel the output was filled with,
    unless the oracle's value itself is that number to within 1%;
  * the first chunk also checks that every padding / masked-off row of the
    whole output kept the sentinel, bit for bit.

The five FP8 GEMM workloads run a second time with the other output tile
(the one the automatic choice does not pick) forced, to the same checks.
Four more shapes near the automatic choice's threshold run under it.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as gfg
from fp8_block_scaled_amd import workloads as wl
from oracle import fp8_oracle as o
from parity_utils import SENTINEL, bits, check_close, sentinel_bits, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

# how each op quantizes (library, oracle) and which entry point it calls
_LIB_QUANT = {"gemm": (gfg.fp8_quantize_act_1x128, gfg.fp8_quantize_weight_128x128),
              "silu_mul": (gfg.fp8_quantize_act_1x128, gfg.fp8_quantize_weight_128x128),
              "mx": (gfg.fp8_quantize_mx_1x32, gfg.fp8_quantize_mx_1x32),
              "mx4": (gfg.fp4_quantize_mx_1x32, gfg.fp4_quantize_mx_1x32),
              "mx4_silu": (gfg.fp4_quantize_mx_1x32, gfg.fp4_quantize_mx_1x32)}
_ORACLE_QUANT = {"gemm": (o.quantize_act_1x128, o.quantize_weight_128x128),
                 "silu_mul": (o.quantize_act_1x128, o.quantize_weight_128x128),
                 "mx": (o.quantize_mx_1x32, o.quantize_mx_1x32),
                 "mx4": (o.quantize_mx4_1x32, o.quantize_mx4_1x32),
                 "mx4_silu": (o.quantize_mx4_1x32, o.quantize_mx4_1x32)}
_ORACLE_GEMM = {"gemm": o.grouped_gemm_contiguous,
                "silu_mul": o.grouped_gemm_silu_mul_contiguous,
                "mx": o.grouped_gemm_mx_contiguous,
                "mx4": o.grouped_gemm_mx4_contiguous,
                "mx4_silu": o.grouped_gemm_mx4_silu_mul_contiguous}
_ENTRY = {"gemm": gfg.grouped_fp8_gemm_contiguous,
          "silu_mul": gfg.grouped_fp8_gemm_silu_mul_contiguous,
          "mx": gfg.grouped_mxfp8_gemm_contiguous,
          "mx4": gfg.grouped_mxfp4_gemm_contiguous,
          "mx4_silu": gfg.grouped_mxfp4_gemm_silu_mul_contiguous}

_run_cache = {}


def _gpu_run(name, tile=gfg.TILE_AUTO):
    """The workload's inputs, the library's bytes and the GPU output with the
    given tile shape (cached: the chunks of one workload share a single
    launch)."""
    if (name, tile) in _run_cache:
        return _run_cache[(name, tile)]
    _run_cache.clear()
    w = wl.workload(name)
    print(f"[full] launch {w.name} layout={w.layout} op={w.op} G={w.G} N={w.N} K={w.K} tile={tile}", flush=True)
    x = wl.draw(w)
    qact, qw = _LIB_QUANT[w.op]
    if w.layout == "masked":
        qa, sa = gfg.fp8_quantize_act_masked(x["a"])
    else:
        qa, sa = qact(x["a"])
    qb, sb = qw(x["b"])
    qb_d, sb_d = to_dev(qb), to_dev(sb)
    if w.b_distinct:                    # every expert its own copy in device memory
        idx = torch.from_numpy(x["b_index"]).cuda()
        qb_d, sb_d = qb_d.index_select(0, idx), sb_d.index_select(0, idx)
    out_cols = w.I if w.op in ("silu_mul", "mx4_silu") else w.N
    shape = (w.G, w.M_max, out_cols) if w.layout == "masked" else (w.M, out_cols)
    d = torch.full(shape, SENTINEL, dtype=torch_dtype(w.out_dtype), device="cuda")
    gfg.set_tile_shape(tile)
    try:
        if w.layout == "masked":
            gfg.grouped_fp8_gemm_masked(to_dev(qa), to_dev(sa), qb_d, sb_d, to_dev(x["masked_m"]), d)
        else:
            _ENTRY[w.op](to_dev(qa), to_dev(sa), qb_d, sb_d, to_dev(x["grouped_layout"]), d)
        torch.cuda.synchronize()
    finally:
        gfg.set_tile_shape(gfg.TILE_AUTO)
    del qb_d, sb_d
    r = dict(w=w, x=x, qa=qa, sa=sa, qb=qb, sb=sb, bits=bits(d), got=d.float().cpu().numpy())
    del d
    _run_cache[(name, tile)] = r
    return r


def _chunks(w):
    if w.b_distinct:
        return w.b_distinct
    return w.G


# (workload, chunk) cases: one per expert / group, or per weight draw
_WORKLOADS = ["contig_g4_m1024_n2048_k7168", "contig_g8_mrand_n7168_k2304", "masked_g8_m1024_n2048_k7168",
              "contig_g8_m4096_n7168_k2304_logmag", "dense_g1_m4096_n4096_k16384", "kimi_tp4_gemm1_t4096",
              "mx_contig_g4_m1024_n2048_k7168", "mx_kimi_tp4_gemm1_t4096", "mx4_contig_g4_m1024_n2048_k7168",
              "mx4_kimi_tp4_gemm1_t4096", "mx4_silu_kimi_tp4_gemm1_t4096"]
_CASES = [(n, c) for n in _WORKLOADS for c in range(_chunks(wl.workload(n)))]


def _no_stray_sentinel(b_rows, ref, out_dtype, what):
    stray = b_rows == sentinel_bits(out_dtype)
    if stray.any():
        assert np.all(np.abs(ref[stray] - SENTINEL) <= 0.01 * abs(SENTINEL)), \
            f"{what}: {int(stray.sum())} valid outputs still hold the sentinel"


# The FP8 workloads again with the tile shape the automatic choice does not
# take, forced: the 256 x 256 kernel on the one-round and masked shapes, the
# 128 x 256 kernel on the many-tile (including the ragged one) and long-K ones.
_OTHER = {"contig_g4_m1024_n2048_k7168": gfg.TILE_256x256, "contig_g8_mrand_n7168_k2304": gfg.TILE_128x256,
          "masked_g8_m1024_n2048_k7168": gfg.TILE_256x256,
          "contig_g8_m4096_n7168_k2304_logmag": gfg.TILE_128x256, "dense_g1_m4096_n4096_k16384": gfg.TILE_128x256}
_OTHER_CASES = [(n, c) for n in _OTHER for c in range(_chunks(wl.workload(n)))]


# Shapes near the automatic tile choice's threshold (rounds of tiles over the
# CUs: 1 against 2 with a long K loop, 2 against 3, 3 against 5, and a masked
# launch of 3 against 6), every output under the automatic choice.
_THRESHOLD = ["contig_g8_m1024_n2048_k7168", "contig_g8_m1280_n2048_k7168", "contig_g8_m1280_n4096_k2304",
              "masked_g8_m1536_n4096_k2304"]
_THRESHOLD_CASES = [(n, c) for n in _THRESHOLD for c in range(_chunks(wl.workload(n)))]


@pytest.mark.parametrize("name,chunk", _CASES, ids=[f"{n}-{c}" for n, c in _CASES])
def test_full_size_every_output(name, chunk):
    _check_chunk(name, chunk, gfg.TILE_AUTO)


@pytest.mark.parametrize("name,chunk", _OTHER_CASES, ids=[f"{n}-{c}" for n, c in _OTHER_CASES])
def test_full_size_other_tile_shape(name, chunk):
    _check_chunk(name, chunk, _OTHER[name])


@pytest.mark.parametrize("name,chunk", _THRESHOLD_CASES, ids=[f"{n}-{c}" for n, c in _THRESHOLD_CASES])
def test_full_size_tile_choice_threshold(name, chunk):
    _check_chunk(name, chunk, gfg.TILE_AUTO)


def _check_chunk(name, chunk, tile):
    r = _gpu_run(name, tile)
    w, x = r["w"], r["x"]
    qact_o, qw_o = _ORACLE_QUANT[w.op]
    what = f"{w.name} tile {tile} chunk {chunk}"
    print(f"[full] {what}", flush=True)
    if w.layout == "masked":
        g, mm = chunk, int(x["masked_m"][chunk])
        if chunk == 0:
            for gg, m in enumerate(x["masked_m"]):
                assert np.all(r["bits"][gg, m:] == sentinel_bits(w.out_dtype)), f"group {gg}: rows >= masked_m written"
        if mm == 0:
            return
        oqa, osa = o.quantize_act_masked(x["a"][g:g + 1])
        oqb, osb = qw_o(x["b"][g:g + 1])
        assert np.array_equal(r["qa"][g:g + 1], oqa) and np.array_equal(r["sa"][g:g + 1], osa)
        assert np.array_equal(r["qb"][g:g + 1], oqb) and np.array_equal(r["sb"][g:g + 1], osb)
        ref = o.grouped_gemm_masked(oqa, osa, oqb, osb, [mm])[0, :mm]
        got, b_rows = r["got"][g, :mm], r["bits"][g, :mm]
    else:
        layout = x["grouped_layout"]
        if chunk == 0:
            assert np.all(r["bits"][layout < 0] == sentinel_bits(w.out_dtype)), "padding rows were written"
        if w.b_distinct:       # every expert whose weights are draw `chunk`
            experts = np.nonzero(x["b_index"] == chunk)[0]
            rows = np.nonzero(np.isin(layout, experts))[0]
        else:
            rows = np.nonzero(layout == chunk)[0]
        if not rows.size:
            return
        oqa, osa = qact_o(x["a"][rows])
        oqb, osb = qw_o(x["b"][chunk:chunk + 1])
        assert np.array_equal(r["qa"][rows], oqa) and np.array_equal(r["sa"][:, rows], osa)
        assert np.array_equal(r["qb"][chunk:chunk + 1], oqb) and np.array_equal(r["sb"][chunk:chunk + 1], osb)
        ref = _ORACLE_GEMM[w.op](oqa, osa, oqb, osb, np.zeros(rows.size, np.int32))
        got, b_rows = r["got"][rows], r["bits"][rows]
    check_close(got, ref, what)
    _no_stray_sentinel(b_rows, ref, w.out_dtype, what)
