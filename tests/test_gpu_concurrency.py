"""Launches in flight at the same time on different streams share nothing:
the kernels keep their tile lists in LDS and use no global scratch, so each
output equals the same launch run alone, bit for bit.  Three launches per
round (the 128 x 256 kernel, the 256 x 256 kernel forced, and the masked
layout) on three streams, ten rounds queued before one synchronization."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as gfg
from fp8_block_scaled_amd import workloads as wl
from parity_utils import SENTINEL, bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore_settings():
    yield
    gfg.set_tile_shape(gfg.TILE_AUTO)


def _contig(seed, m_per_group, N, K):
    x = wl.small_contiguous(seed, m_per_group, N, K)
    qa, sa = gfg.fp8_quantize_act_1x128(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    args = [to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), to_dev(x["grouped_layout"].astype(np.int32))]
    return args, (qa.shape[0], qb.shape[1])


def test_three_streams_concurrent_bitwise():
    dev = torch.device("cuda:0")
    a_args, a_shape = _contig(71, [700, 300, 1024, 77], 1024, 1024)     # 128 x 256 tiles
    b_args, b_shape = _contig(72, [1000, 513, 640], 1280, 512)          # 256 x 256 tiles (forced)
    xm = wl.small_masked(73, [0, 500, 1024, 3], 1024, 768, 1024)
    qa, sa = gfg.fp8_quantize_act_masked(xm["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(xm["b"])
    c_args = [to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), to_dev(np.asarray(xm["masked_m"], np.int32))]
    c_shape = (qa.shape[0], qa.shape[1], qb.shape[1])

    def launch(which, d, stream):
        if which == "a":
            gfg.set_tile_shape(gfg.TILE_AUTO)
            gfg.grouped_fp8_gemm_contiguous(*a_args, d, stream=stream)
        elif which == "b":
            gfg.set_tile_shape(gfg.TILE_256x256)
            gfg.grouped_fp8_gemm_contiguous(*b_args, d, stream=stream)
        else:
            gfg.set_tile_shape(gfg.TILE_AUTO)
            gfg.grouped_fp8_gemm_masked(*c_args, d, stream=stream)

    shapes = {"a": a_shape, "b": b_shape, "c": c_shape}
    new = lambda k: torch.full(shapes[k], SENTINEL, dtype=torch.bfloat16, device=dev)
    ref = {}
    for k in "abc":                                   # each alone, on the default stream
        ref[k] = new(k)
        launch(k, ref[k], None)
        torch.cuda.synchronize()
        ref[k] = bits(ref[k])
    streams = {k: torch.cuda.Stream(dev) for k in "abc"}
    outs = []
    for _ in range(10):
        ds = {k: new(k) for k in "abc"}
        torch.cuda.synchronize()                      # the sentinel fills are done before the launches
        for k in "abc":
            launch(k, ds[k], streams[k])
        outs.append(ds)
    torch.cuda.synchronize()
    for r, ds in enumerate(outs):
        for k in "abc":
            assert np.array_equal(bits(ds[k]), ref[k]), f"round {r}: launch {k} differs from its solo run"
