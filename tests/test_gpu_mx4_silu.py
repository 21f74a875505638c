"""GPU parity of the a4w4 gemm1 with silu_mul (MXFP4 operands, E2M1 two per
byte with one E8M0 scale per 32 K elements of every row; out[m, j] =
silu(h[j]) * h[I + j] with h = A[m] . B[g]^T) against the fp64 CPU oracle.

The GPU gets the host quantizer's bytes and the oracle its own, after a check
that the two are equal.  The bar is the GEMM's (calc_diff <= 1e-5, row-floored
max relative error <= 1e-2 over valid rows); padding and masked-off rows keep
the caller's sentinel bit for bit.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as gfg
from fp8_block_scaled_amd import workloads as wl
from oracle import fp8_oracle as o
from parity_utils import SENTINEL, bits, check_close, sentinel_bits, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _quant(x):
    q, s = gfg.fp4_quantize_mx_1x32(x)
    oq, os_ = o.quantize_mx4_1x32(x)
    assert np.array_equal(s, os_) and np.array_equal(q, oq), "quantizer bytes differ from the oracle"
    return q, s, oq, os_


def _contig(x, out):
    qa, sa, oqa, osa = _quant(x["a"])
    qb, sb, oqb, osb = _quant(x["b"])
    M, I = qa.shape[0], qb.shape[1] // 2
    d = torch.full((M, I), SENTINEL, dtype=torch_dtype(out), device="cuda")
    gfg.grouped_mxfp4_gemm_silu_mul_contiguous(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb),
                                               to_dev(x["grouped_layout"]), d)
    torch.cuda.synchronize()
    ref = o.grouped_gemm_mx4_silu_mul_contiguous(oqa, osa, oqb, osb, x["grouped_layout"])
    return d, ref


@pytest.mark.parametrize("m_per_group,I,K,out", [
    ([100, 1, 128, 129, 300], 128, 256, "bf16"),     # one output tile, a single K step
    ([5, 250], 256, 768, "f16"),
    ([0, 128, 77], 384, 512, "bf16"),                # an empty group, 3 output tiles
    ([1000, 30], 640, 1280, "bf16"),                 # many M tiles, 5 output tiles, 5 K steps
])
def test_mx4_silu_contiguous_small(m_per_group, I, K, out):
    what = f"mx4 silu contig {m_per_group} I={I} K={K} {out}"
    print(f"[mx4_silu] {what}", flush=True)
    x = wl.small_contiguous(sum(m_per_group) + I + K + 11, m_per_group, 2 * I, K)
    d, ref = _contig(x, out)
    valid = x["grouped_layout"] >= 0
    check_close(d.float().cpu().numpy()[valid], ref[valid], what)
    assert np.all(bits(d)[~valid] == sentinel_bits(out)), f"{what}: padding rows were written"


@pytest.mark.parametrize("masked_m,Mmax,I,K,out", [
    ([0, 64, 200], 256, 256, 512, "bf16"),
    ([512, 3, 129, 0], 512, 128, 256, "f16"),
    ([-3, 300, 44], 320, 384, 768, "bf16"),          # a negative count clamps to 0
])
def test_mx4_silu_masked_small(masked_m, Mmax, I, K, out):
    what = f"mx4 silu masked {masked_m} Mmax={Mmax} I={I} K={K} {out}"
    print(f"[mx4_silu] {what}", flush=True)
    x = wl.small_masked(Mmax + I + K + 13, [max(m, 0) for m in masked_m], Mmax, 2 * I, K)
    qa, sa, oqa, osa = _quant(x["a"])
    qb, sb, oqb, osb = _quant(x["b"])
    G = len(masked_m)
    d = torch.full((G, Mmax, I), SENTINEL, dtype=torch_dtype(out), device="cuda")
    gfg.grouped_mxfp4_gemm_silu_mul_masked(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb),
                                           to_dev(np.asarray(masked_m, np.int32)), d)
    torch.cuda.synchronize()
    ref = o.grouped_gemm_mx4_silu_mul_masked(oqa, osa, oqb, osb, masked_m)
    got, b = d.float().cpu().numpy(), bits(d)
    gots, refs = [], []
    for g, mm in enumerate(masked_m):
        mm = min(max(mm, 0), Mmax)
        assert np.all(b[g, mm:] == sentinel_bits(out)), f"{what}: group {g} rows >= masked_m written"
        gots.append(got[g, :mm])
        refs.append(ref[g, :mm])
    check_close(np.concatenate(gots), np.concatenate(refs), what)


def test_mx4_silu_matches_unfused_gpu_gemm():
    """The fused epilogue against the MXFP4 GEMM on the GPU followed by
    silu_mul in fp64 on the host: both start from the same fp32 accumulators,
    so the two differ only by the epilogue's own roundings."""
    x = wl.small_contiguous(91, [300, 7, 256], 2 * 256, 512)
    qa, sa = gfg.fp4_quantize_mx_1x32(x["a"])
    qb, sb = gfg.fp4_quantize_mx_1x32(x["b"])
    layout = x["grouped_layout"]
    M, I = qa.shape[0], qb.shape[1] // 2
    h = torch.full((M, 2 * I), SENTINEL, dtype=torch.float16, device="cuda")
    gfg.grouped_mxfp4_gemm_contiguous(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), to_dev(layout), h)
    d = torch.full((M, I), SENTINEL, dtype=torch.float16, device="cuda")
    gfg.grouped_mxfp4_gemm_silu_mul_contiguous(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), to_dev(layout), d)
    torch.cuda.synchronize()
    valid = layout >= 0
    hv = h.float().cpu().numpy().astype(np.float64)[valid]
    unfused = o.silu(hv[:, :I]) * hv[:, I:]
    check_close(d.float().cpu().numpy()[valid], unfused, "fused vs unfused")


def test_mx4_silu_repeatable():
    x = wl.small_contiguous(79, [300, 200], 2 * 256, 512)
    d1, _ = _contig(x, "bf16")
    d2, _ = _contig(x, "bf16")
    assert torch.equal(d1, d2)
