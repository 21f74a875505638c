"""GPU parity of the MXFP8 grouped GEMM (one E8M0 scale per 32 K elements of
every row of A and B) against the fp64 CPU oracle.

The bar is the GEMM's (calc_diff <= 1e-5, row-floored max relative error
<= 1e-2 over valid rows; untouched rows keep the sentinel bit for bit).  The
integer case, whose scales vary from one 32-wide block to the next, must
match the correctly rounded exact result bit for bit: it fails if any block
of any row meets another block's scale.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as gfg
from fp8_block_scaled_amd import workloads as wl
from oracle import fp8_oracle as o
from parity_utils import SENTINEL, bits, check_close, sentinel_bits, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _run_contig(qa, sa, qb, sb, layout, out):
    d = torch.full((qa.shape[0], qb.shape[1]), SENTINEL, dtype=torch_dtype(out), device="cuda")
    gfg.grouped_mxfp8_gemm_contiguous(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), to_dev(layout), d)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("m_per_group,N,K,out", [
    ([100, 1, 128, 129, 300], 256, 256, "bf16"),
    ([5, 250], 512, 384, "f16"),
    ([0, 128, 77], 768, 128, "bf16"),               # an empty group, a single K step
    ([1000, 30], 1280, 640, "bf16"),                # many tiles, a K-loop remainder
])
def test_mx_contiguous_small(m_per_group, N, K, out):
    what = f"mx contig {m_per_group} N={N} K={K} {out}"
    print(f"[mx] {what}", flush=True)
    x = wl.small_contiguous(sum(m_per_group) + N + K + 1, m_per_group, N, K)
    qa, sa = gfg.fp8_quantize_mx_1x32(x["a"])
    qb, sb = gfg.fp8_quantize_mx_1x32(x["b"])
    d = _run_contig(qa, sa, qb, sb, x["grouped_layout"], out)
    oqa, osa = o.quantize_mx_1x32(x["a"])
    oqb, osb = o.quantize_mx_1x32(x["b"])
    assert np.array_equal(qa, oqa) and np.array_equal(sb, osb)
    ref = o.grouped_gemm_mx_contiguous(oqa, osa, oqb, osb, x["grouped_layout"])
    valid = x["grouped_layout"] >= 0
    check_close(d.float().cpu().numpy()[valid], ref[valid], what)
    assert np.all(bits(d)[~valid] == sentinel_bits(out)), f"{what}: padding rows were written"


@pytest.mark.parametrize("masked_m,Mmax,N,K,out", [
    ([0, 64, 200], 256, 512, 384, "bf16"),
    ([512, 3, 129, 0], 512, 256, 256, "f16"),
])
def test_mx_masked_small(masked_m, Mmax, N, K, out):
    what = f"mx masked {masked_m} Mmax={Mmax} N={N} K={K} {out}"
    print(f"[mx] {what}", flush=True)
    x = wl.small_masked(sum(masked_m) + Mmax + N + 3, masked_m, Mmax, N, K)
    qa, sa = gfg.fp8_quantize_mx_1x32(x["a"])
    qb, sb = gfg.fp8_quantize_mx_1x32(x["b"])
    G = len(masked_m)
    d = torch.full((G, Mmax, N), SENTINEL, dtype=torch_dtype(out), device="cuda")
    gfg.grouped_mxfp8_gemm_masked(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb),
                                  to_dev(np.asarray(masked_m, np.int32)), d)
    torch.cuda.synchronize()
    ref = o.grouped_gemm_mx_masked(*o.quantize_mx_1x32(x["a"]), *o.quantize_mx_1x32(x["b"]), masked_m)
    got, b = d.float().cpu().numpy(), bits(d)
    gots, refs = [], []
    for g, mm in enumerate(masked_m):
        assert np.all(b[g, mm:] == sentinel_bits(out)), f"{what}: group {g} rows >= masked_m written"
        gots.append(got[g, :mm])
        refs.append(ref[g, :mm])
    check_close(np.concatenate(gots), np.concatenate(refs), what)


@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_mx_exact_integer_case_bitwise(out):
    """Integer E4M3 codes in [-4, 4] and scale bytes 127 or 128 drawn per row
    and per 32-wide block: every partial sum is exact in fp32, so the output
    is the correctly rounded exact product."""
    rng = np.random.default_rng(41)
    G, rows, N, K = 2, 256, 256, 384            # expert runs start on multiples of 128
    table = {int(o.decode_e4m3(np.uint8(c))): c for c in range(0, 0x50) if float(o.decode_e4m3(np.uint8(c))).is_integer()}
    table.update({-v: c | 0x80 for v, c in list(table.items()) if v > 0})
    ia = rng.integers(-4, 4, size=(G * rows, K), endpoint=True)
    ib = rng.integers(-4, 4, size=(G, N, K), endpoint=True)
    qa = np.vectorize(table.get)(ia).astype(np.uint8)
    qb = np.vectorize(table.get)(ib).astype(np.uint8)
    sa = rng.integers(127, 128, size=(K // 32, G * rows), endpoint=True).astype(np.uint8)
    sb = rng.integers(127, 128, size=(G, K // 32, N), endpoint=True).astype(np.uint8)
    layout = np.repeat(np.arange(G, dtype=np.int32), rows)
    d = _run_contig(qa, sa, qb, sb, layout, out)
    exact = o.grouped_gemm_mx_contiguous(qa, sa, qb, sb, layout)
    rnd = o.round_to_bf16 if out == "bf16" else o.round_to_f16
    want = torch.from_numpy(rnd(exact)).to(torch_dtype(out))
    assert np.array_equal(bits(d), bits(want))
