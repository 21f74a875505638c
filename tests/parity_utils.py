"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI
binding, run the oracle on the same float32 inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

import fp8_block_scaled_amd as gfg
from oracle import fp8_oracle as o

SENTINEL = -12352.0          # exactly representable in bf16 and f16

CALC_DIFF_MAX = 1e-5         # GPU vs fp64 oracle
MAX_REL_MAX = 1e-2           # row-floored max relative error
# Denominator floor of the relative error, as a fraction of the row's largest
# |output|.  gfx950's scaled FP8 MFMA does not sum a 128-wide K block in fp32:
# inside a 16-element K group it drops products 2^-14 below the group's
# largest, and on N(0,1) data one block's error reaches ~2e-4 of the sum of
# |products| (measured through the C-ABI in tests/test_gpu_mfma_precision.py).
# Outputs that cancel to near zero therefore carry an absolute error set by
# the row's scale, not their own: at a floor of 1e-3 of the row maximum a
# single K block already exceeds 1e-2; at 1e-2 of the row maximum the bound
# holds.  check_close reports both.
REL_FLOOR = 1e-2


def torch_dtype(name):
    return {"bf16": torch.bfloat16, "f16": torch.float16}[name]


def to_dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy()


def gpu_contiguous(qa, sa, qb, sb, layout, out_dtype, d=None, stream=None):
    M, N = qa.shape[0], qb.shape[1]
    if d is None:
        d = torch.full((M, N), SENTINEL, dtype=torch_dtype(out_dtype), device="cuda")
    gfg.grouped_fp8_gemm_contiguous(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb),
                                    to_dev(layout.astype(np.int32)), d, stream=stream)
    torch.cuda.synchronize()
    return d


def gpu_masked(qa, sa, qb, sb, masked_m, out_dtype, d=None):
    G, Mmax, N = qa.shape[0], qa.shape[1], qb.shape[1]
    if d is None:
        d = torch.full((G, Mmax, N), SENTINEL, dtype=torch_dtype(out_dtype), device="cuda")
    gfg.grouped_fp8_gemm_masked(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb),
                                to_dev(np.asarray(masked_m, np.int32)), d)
    torch.cuda.synchronize()
    return d


def check_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """calc_diff and row-floored max relative error, over the given valid rows."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    cd = o.calc_diff(got, ref)
    mr = o.max_rel_err_rowfloor(got, ref, floor=REL_FLOOR)
    print(f"[parity] {what}: calc_diff={cd:.3e} max_rel(floor {REL_FLOOR:g})={mr:.3e} "
          f"max_rel(floor 1e-3)={o.max_rel_err_rowfloor(got, ref, floor=1e-3):.3e}", flush=True)
    assert cd <= CALC_DIFF_MAX, f"{what}: calc_diff {cd:.3e} > {CALC_DIFF_MAX}"
    assert mr <= MAX_REL_MAX, f"{what}: max rel err {mr:.3e} > {MAX_REL_MAX}"
    return cd, mr


def sentinel_bits(out_dtype):
    return bits(torch.tensor([SENTINEL], dtype=torch_dtype(out_dtype)))[0]
