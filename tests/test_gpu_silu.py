"""GPU parity of gemm1 with silu_mul against the fp64 CPU oracle.

out[m, j] = silu(h[j]) * h[I + j] with h = A[m] . B[g]^T: the HIP path computes
h in fp32 MFMAs, silu with the hardware base-2 exponential and reciprocal, and
rounds once to bf16/f16.  The bar is that of the GEMM (calc_diff <= 1e-5,
row-floored max relative error <= 1e-2 over valid rows); rows that are
padding or masked off keep the caller's sentinel bit for bit.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as gfg
from fp8_block_scaled_amd import workloads as wl
from oracle import fp8_oracle as o
from parity_utils import SENTINEL, bits, check_close, sentinel_bits, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _contig(x, out_dtype):
    qa, sa = gfg.fp8_quantize_act_1x128(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    M, I = qa.shape[0], qb.shape[1] // 2
    d = torch.full((M, I), SENTINEL, dtype=torch_dtype(out_dtype), device="cuda")
    gfg.grouped_fp8_gemm_silu_mul_contiguous(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb),
                                             to_dev(x["grouped_layout"]), d)
    torch.cuda.synchronize()
    oqa, osa = o.quantize_act_1x128(x["a"])
    oqb, osb = o.quantize_weight_128x128(x["b"])
    ref = o.grouped_gemm_silu_mul_contiguous(oqa, osa, oqb, osb, x["grouped_layout"])
    return d, ref


@pytest.mark.parametrize("m_per_group,I,K,out", [
    ([100, 1, 128, 129, 300], 256, 256, "bf16"),     # several groups, ragged rows, 2 output tiles
    ([5, 250], 128, 384, "f16"),                     # one output tile, f16
    ([0, 128, 77], 384, 128, "bf16"),                # an empty group, a single K step
    ([1000, 30], 640, 640, "bf16"),                  # many M tiles, 5 output tiles
])
def test_silu_mul_contiguous_small(m_per_group, I, K, out):
    what = f"silu contig {m_per_group} I={I} K={K} {out}"
    print(f"[silu] {what}", flush=True)
    x = wl.small_contiguous(sum(m_per_group) + I + K, m_per_group, 2 * I, K)
    d, ref = _contig(x, out)
    layout = x["grouped_layout"]
    valid = layout >= 0
    check_close(d.float().cpu().numpy()[valid], ref[valid], what)
    assert np.all(bits(d)[~valid] == sentinel_bits(out)), f"{what}: padding rows were written"


@pytest.mark.parametrize("masked_m,Mmax,I,K,out", [
    ([0, 64, 200], 256, 256, 384, "bf16"),
    ([512, 3, 129, 0], 512, 128, 256, "f16"),
])
def test_silu_mul_masked_small(masked_m, Mmax, I, K, out):
    what = f"silu masked {masked_m} Mmax={Mmax} I={I} K={K} {out}"
    print(f"[silu] {what}", flush=True)
    x = wl.small_masked(sum(masked_m) + Mmax + I, masked_m, Mmax, 2 * I, K)
    qa, sa = gfg.fp8_quantize_act_masked(x["a"])
    qb, sb = gfg.fp8_quantize_weight_128x128(x["b"])
    G = len(masked_m)
    d = torch.full((G, Mmax, I), SENTINEL, dtype=torch_dtype(out), device="cuda")
    gfg.grouped_fp8_gemm_silu_mul_masked(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb),
                                         to_dev(np.asarray(masked_m, np.int32)), d)
    torch.cuda.synchronize()
    oqa, osa = o.quantize_act_masked(x["a"])
    oqb, osb = o.quantize_weight_128x128(x["b"])
    ref = o.grouped_gemm_silu_mul_masked(oqa, osa, oqb, osb, masked_m)
    got = d.float().cpu().numpy()
    b = bits(d)
    gots, refs = [], []
    for g, mm in enumerate(masked_m):
        assert np.all(b[g, mm:] == sentinel_bits(out)), f"{what}: group {g} rows >= masked_m written"
        gots.append(got[g, :mm])
        refs.append(ref[g, :mm])
    check_close(np.concatenate(gots), np.concatenate(refs), what)


def test_silu_mul_repeatable():
    x = wl.small_contiguous(77, [300, 200], 512, 512)
    d1, _ = _contig(x, "bf16")
    d2, _ = _contig(x, "bf16")
    assert torch.equal(d1, d2)
