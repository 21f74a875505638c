"""Host-side arithmetic of bench.py (no GPU): the algorithmic bytes and FLOPs
the roofline is priced on, written out here from the operand shapes, and the
one-GPU guard of the command line."""
import json
import os
import subprocess
import sys

import bench
from fp8_block_scaled_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_bytes_and_flops_from_operand_sizes():
    # 4 experts x 1024 rows, N=2048, K=7168, bf16 output: every operand once
    w = wl.workload("contig_g4_m1024_n2048_k7168")
    M, N, K, G = 4096, 2048, 7168, 4
    a = M * K                                  # e4m3 activations
    sa = M * (K // 128)                        # (1,128) scale bytes
    b = G * N * K                              # e4m3 weights of the four experts
    sb = G * (N // 128) * (K // 128)           # (128,128) scale bytes
    d = M * N * 2                              # bf16 output
    assert bench.algorithmic_bytes(w) == a + sa + b + sb + d == 105_090_560
    assert w.flops == 2 * M * N * K == 120_259_084_288


def test_masked_bytes_count_valid_rows_and_whole_tiles():
    # a masked workload: A rows are the valid ones, A scales cover whole 128-row
    # tiles, only experts with rows bring their weights
    w = wl.workload("masked_g8_m1024_n2048_k7168")
    KB, NB = w.K // 128, w.N // 128
    valid = [min(max(m, 0), w.M_max) for m in w.masked_m]
    tiles = sum((m + 127) // 128 for m in valid)
    experts = sum(1 for m in valid if m > 0)
    want = sum(valid) * w.K + tiles * 128 * KB + experts * (w.N * w.K + NB * KB) + sum(valid) * w.N * 2
    assert bench.algorithmic_bytes(w) == want


def test_quant_bytes():
    # read bf16, write one code byte per element and one scale byte per 128
    assert bench.quant_bytes(1, 32768, 2304, 2) == 32768 * 2304 * 3 + 32768 * 18 == 227_082_240
    assert bench.quant_bytes(3, 70, 384, 4) == 3 * 70 * 384 * 5 + 3 * 70 * 3


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
