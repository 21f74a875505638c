"""The GEMM launches inside a captured HIP graph.

The entry points allocate, free and synchronize nothing and record no
memset, so a caller may capture them.  The graph below holds both tile shapes
and both layouts; it is replayed several times with eager work and
synchronizations in between, and every replay must reproduce the eager
launches' outputs bit for bit.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as gfg
from fp8_block_scaled_amd import workloads as wl
from parity_utils import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore_settings():
    yield
    gfg.set_tile_shape(gfg.TILE_AUTO)


def _raw_call(fn, *args):
    rc = fn(*args)
    if rc:
        raise gfg.GfgError(rc, gfg.load_library().grouped_fp8_last_error().decode())


def test_graph_replays_match_eager():
    dev = torch.device("cuda:0")
    xc = wl.small_contiguous(31, [600, 129, 1000, 0, 300], 1024, 1024)
    qa, sa = gfg.fp8_quantize_act_1x128(xc["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(xc["b"])
    A, SA, B, SB, LAY = to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), to_dev(xc["grouped_layout"])
    M, N, K, G = qa.shape[0], 1024, 1024, qb.shape[0]
    xm = wl.small_masked(32, [300, 0, 513, 1024], 1024, 512, 512)
    mqa, msa = gfg.fp8_quantize_act_masked(xm["a"])
    mqb, msb = gfg.fp8_quantize_weight_128x128(xm["b"])
    MA, MSA, MB, MSB, MM = to_dev(mqa), to_dev(msa), to_dev(mqb), to_dev(msb), to_dev(np.asarray(xm["masked_m"], np.int32))
    outs = [torch.full((M, N), -7.0, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    mout = torch.full((4, 1024, 512), -7.0, dtype=torch.bfloat16, device=dev)

    s = torch.cuda.Stream(dev)
    h = s.cuda_stream

    def launches():
        gfg.set_tile_shape(gfg.TILE_128x256)
        _raw_call(gfg.raw_contiguous, A.data_ptr(), SA.data_ptr(), B.data_ptr(), SB.data_ptr(), LAY.data_ptr(),
                  outs[0].data_ptr(), M, N, K, G, gfg.OUT_BF16, h)
        gfg.set_tile_shape(gfg.TILE_256x256)
        _raw_call(gfg.raw_contiguous, A.data_ptr(), SA.data_ptr(), B.data_ptr(), SB.data_ptr(), LAY.data_ptr(),
                  outs[1].data_ptr(), M, N, K, G, gfg.OUT_BF16, h)
        gfg.set_tile_shape(gfg.TILE_AUTO)
        _raw_call(gfg.raw_masked, MA.data_ptr(), MSA.data_ptr(), MB.data_ptr(), MSB.data_ptr(), MM.data_ptr(),
                  mout.data_ptr(), 4, 1024, 512, 512, gfg.OUT_BF16, h)

    with torch.cuda.stream(s):
        launches()
    torch.cuda.synchronize(dev)
    eager = [o.clone() for o in outs] + [mout.clone()]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        launches()
    for r in range(4):
        for o in outs + [mout]:
            o.fill_(3.0)                     # eager work between replays
        torch.cuda.synchronize(dev)
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize(dev)
        for k, (o, e) in enumerate(zip(outs + [mout], eager)):
            if k < 2:
                # rows outside every expert keep what the eager fill left there
                valid = torch.from_numpy(xc["grouped_layout"] >= 0).to(dev)
                assert torch.equal(o[valid].view(torch.int16), e[valid].view(torch.int16)), f"replay {r}, output {k}"
            else:
                for gi, mm in enumerate(xm["masked_m"]):
                    assert torch.equal(o[gi, :mm].view(torch.int16), e[gi, :mm].view(torch.int16)), f"replay {r}, group {gi}"
