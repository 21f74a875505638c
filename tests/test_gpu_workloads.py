"""GPU parity at the five reference workloads' full sizes, in the launch
configuration the benchmark times.

The GPU computes every output; the oracle recomputes a sample of them: in each
expert, the first, last and six random valid rows, crossed with four random
128-column blocks plus the last one.  Weight quantization is per (128,128)
block, so quantizing only the sampled column blocks gives the oracle the same
operands the full quantization would.  Every padding / masked-off row of the
full output is checked against the sentinel, and the packer's bytes for the
sampled rows and blocks are checked against the oracle's quantizer.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as gfg
from fp8_block_scaled_amd import workloads as wl
from oracle import fp8_oracle as o
from parity_utils import SENTINEL, bits, check_close, sentinel_bits, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _sample(rng, valid_rows, N):
    rows = []
    if len(valid_rows):
        rows = sorted(set([valid_rows[0], valid_rows[-1]] +
                          list(rng.choice(valid_rows, size=min(6, len(valid_rows)), replace=False))))
    nblocks = N // 128
    cols = sorted(int(c) for c in rng.choice(nblocks - 1, size=min(4, nblocks - 1), replace=False)) + [nblocks - 1]
    return np.asarray(rows, np.int64), cols


def _oracle_rows(a_rows_f32, b_g_f32, col_blocks):
    """Oracle outputs for the given A rows against the given 128-column blocks of one expert."""
    qa, sa = o.quantize_act_1x128(a_rows_f32)
    bsub = np.concatenate([b_g_f32[128 * c:128 * c + 128] for c in col_blocks])[None]
    qb, sb = o.quantize_weight_128x128(bsub)
    ref = o.grouped_gemm_contiguous(qa, sa, qb, sb, np.zeros(len(a_rows_f32), np.int32))
    return ref, (qa, sa, qb, sb)


def _cols(col_blocks):
    return np.concatenate([np.arange(128 * c, 128 * c + 128) for c in col_blocks])


@pytest.mark.parametrize("idx", [1, 2, 4, "dense_g1_m4096_n4096_k16384"])
def test_contiguous_workload_full_size(idx):
    w = wl.workload(idx)
    print(f"[workload] {w.name} M={w.M} N={w.N} K={w.K} G={w.G}", flush=True)
    x = wl.draw(w)
    layout = x["grouped_layout"]
    qa, sa = gfg.fp8_quantize_act_1x128(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    d = torch.full((w.M, w.N), SENTINEL, dtype=torch_dtype(w.out_dtype), device="cuda")
    gfg.grouped_fp8_gemm_contiguous(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), to_dev(layout), d)
    torch.cuda.synchronize()
    b_all = bits(d)
    assert np.all(b_all[layout < 0] == sentinel_bits(w.out_dtype)), "padding rows were written"
    got_all = d.float().cpu().numpy()
    del d
    rng = np.random.default_rng(w.seed)
    gots, refs = [], []
    for g in range(w.G):
        rows, cblk = _sample(rng, np.nonzero(layout == g)[0], w.N)
        if not len(rows):
            continue
        ref, (oqa, osa, oqb, osb) = _oracle_rows(x["a"][rows], x["b"][g], cblk)
        cols = _cols(cblk)
        # the packer's bytes for these rows / blocks equal the oracle's
        assert np.array_equal(qa[rows], oqa) and np.array_equal(sa[:, rows], osa)
        assert np.array_equal(qb[g][cols], oqb[0])
        assert np.array_equal(sb[g][cblk], osb[0])
        gots.append(got_all[np.ix_(rows, cols)])
        refs.append(ref)
    check_close(np.concatenate(gots), np.concatenate(refs), w.name)


def test_masked_workload_full_size():
    w = wl.workload(3)
    print(f"[workload] {w.name} G={w.G} M_max={w.M_max} N={w.N} K={w.K} masked_m={w.masked_m}", flush=True)
    x = wl.draw(w)
    qa, sa = gfg.fp8_quantize_act_masked(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    d = torch.full((w.G, w.M_max, w.N), SENTINEL, dtype=torch_dtype(w.out_dtype), device="cuda")
    gfg.grouped_fp8_gemm_masked(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb),
                                to_dev(np.asarray(w.masked_m, np.int32)), d)
    torch.cuda.synchronize()
    b_all = bits(d)
    got_all = d.float().cpu().numpy()
    del d
    rng = np.random.default_rng(w.seed)
    gots, refs = [], []
    for g, mm in enumerate(w.masked_m):
        assert np.all(b_all[g, mm:] == sentinel_bits(w.out_dtype)), f"group {g}: rows >= masked_m written"
        rows, cblk = _sample(rng, np.arange(mm), w.N)
        if not len(rows):
            continue
        ref, (oqa, osa, oqb, osb) = _oracle_rows(x["a"][g][rows], x["b"][g], cblk)
        assert np.array_equal(qa[g][rows], oqa) and np.array_equal(sa[g][:, rows], osa)
        gots.append(got_all[g][np.ix_(rows, _cols(cblk))])
        refs.append(ref)
    check_close(np.concatenate(gots), np.concatenate(refs), w.name)
