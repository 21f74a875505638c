"""GPU parity of the MXFP4 grouped GEMM (E2M1 elements two per byte, one E8M0
scale per 32 K elements of every row of A and B) against the fp64 CPU oracle.

The GPU gets the host quantizer's bytes and the oracle its own, after a
check that the two are equal.  The bar is the GEMM's; the integer case is
exact.
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
    """(device bytes, scales) from the product quantizer, (plain bytes, scales) from the oracle."""
    q, s = gfg.fp4_quantize_mx_1x32(x)
    oq, os_ = o.quantize_mx4_1x32(x)
    assert np.array_equal(s, os_) and np.array_equal(q, oq), "quantizer bytes differ from the oracle"
    return q, s, oq, os_


@pytest.mark.parametrize("m_per_group,N,K,out", [
    ([100, 1, 128, 129, 300], 256, 256, "bf16"),     # a single K step
    ([5, 250], 512, 768, "f16"),
    ([0, 128, 77], 768, 512, "bf16"),
    ([1000, 30], 1280, 1280, "bf16"),                # many tiles, K steps 5 (a remainder)
])
def test_mx4_contiguous_small(m_per_group, N, K, out):
    what = f"mx4 contig {m_per_group} N={N} K={K} {out}"
    print(f"[mx4] {what}", flush=True)
    x = wl.small_contiguous(sum(m_per_group) + N + K + 5, m_per_group, N, K)
    qa, sa, oqa, osa = _quant(x["a"])
    qb, sb, oqb, osb = _quant(x["b"])
    d = torch.full((qa.shape[0], N), SENTINEL, dtype=torch_dtype(out), device="cuda")
    gfg.grouped_mxfp4_gemm_contiguous(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), to_dev(x["grouped_layout"]), d)
    torch.cuda.synchronize()
    ref = o.grouped_gemm_mx4_contiguous(oqa, osa, oqb, osb, x["grouped_layout"])
    valid = x["grouped_layout"] >= 0
    check_close(d.float().cpu().numpy()[valid], ref[valid], what)
    assert np.all(bits(d)[~valid] == sentinel_bits(out)), f"{what}: padding rows were written"


@pytest.mark.parametrize("masked_m,Mmax,N,K,out", [
    ([0, 64, 200], 256, 512, 512, "bf16"),
    ([512, 3, 129, 0], 512, 256, 256, "f16"),
])
def test_mx4_masked_small(masked_m, Mmax, N, K, out):
    what = f"mx4 masked {masked_m} Mmax={Mmax} N={N} K={K} {out}"
    print(f"[mx4] {what}", flush=True)
    x = wl.small_masked(sum(masked_m) + Mmax + N + 7, masked_m, Mmax, N, K)
    qa, sa, oqa, osa = _quant(x["a"])
    qb, sb, oqb, osb = _quant(x["b"])
    G = len(masked_m)
    d = torch.full((G, Mmax, N), SENTINEL, dtype=torch_dtype(out), device="cuda")
    gfg.grouped_mxfp4_gemm_masked(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb),
                                  to_dev(np.asarray(masked_m, np.int32)), d)
    torch.cuda.synchronize()
    ref = o.grouped_gemm_mx4_masked(oqa, osa, oqb, osb, masked_m)
    got, b = d.float().cpu().numpy(), bits(d)
    gots, refs = [], []
    for g, mm in enumerate(masked_m):
        assert np.all(b[g, mm:] == sentinel_bits(out)), f"{what}: group {g} rows >= masked_m written"
        gots.append(got[g, :mm])
        refs.append(ref[g, :mm])
    check_close(np.concatenate(gots), np.concatenate(refs), what)


@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_mx4_exact_integer_case_bitwise(out):
    """E2M1 codes of the integers -4..4 (and 0.5 steps) with scale bytes 126..128
    per row and 32-wide block: every partial sum is exact, so the output is the
    correctly rounded exact product."""
    rng = np.random.default_rng(61)
    G, rows, N, K = 2, 256, 256, 512
    ca = rng.integers(0, 16, size=(G * rows, K)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(G, N, K)).astype(np.uint8)
    pack = lambda c: (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    oqa, oqb = pack(ca), pack(cb)
    sa = rng.integers(126, 128, size=(K // 32, G * rows), endpoint=True).astype(np.uint8)
    sb = rng.integers(126, 128, size=(G, K // 32, N), endpoint=True).astype(np.uint8)
    layout = np.repeat(np.arange(G, dtype=np.int32), rows)
    d = torch.full((G * rows, N), SENTINEL, dtype=torch_dtype(out), device="cuda")
    gfg.grouped_mxfp4_gemm_contiguous(to_dev(oqa), to_dev(sa), to_dev(oqb), to_dev(sb), to_dev(layout), d)
    torch.cuda.synchronize()
    exact = o.grouped_gemm_mx4_contiguous(oqa, sa, oqb, sb, layout)
    rnd = o.round_to_bf16 if out == "bf16" else o.round_to_f16
    want = torch.from_numpy(rnd(exact)).to(torch_dtype(out))
    assert np.array_equal(bits(d), bits(want))
