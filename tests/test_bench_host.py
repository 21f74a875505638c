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


def test_trace_summary_final_100(tmp_path):
    """bench.py --trace-summary: per-kernel calls, overall mean and the mean of
    the final 100 dispatches by start time, from a rocprofv3 kernel-trace csv."""
    import csv
    rows = []
    for i in range(250):                       # 250 GEMM dispatches: 1000 ns, last 100 at 500 ns
        dur = 500 if i >= 150 else 1000
        rows.append(("gemm_kernel", 10_000 * i, 10_000 * i + dur))
    rows.append(("copy", 5, 25))
    rows.reverse()                               # the file order must not matter
    d = tmp_path / "run"
    d.mkdir()
    with open(d / "x_kernel_trace.csv", "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for name, t0, t1 in rows:
            wr.writerow(["KERNEL_DISPATCH", name, t0, t1])
    out = {r["kernel"]: r for r in bench.summarize_trace(str(tmp_path))}
    g = out["gemm_kernel"]
    assert g["calls"] == 250
    assert g["final100_mean_ns"] == 500.0
    assert g["mean_ns"] == (150 * 1000 + 100 * 500) / 250
    assert out["copy"]["calls"] == 1 and out["copy"]["final100_mean_ns"] == 20.0


def test_kernel_source_hash_ignores_comments(tmp_path):
    a, b = tmp_path / "a.hip", tmp_path / "b.hip"
    a.write_text("int x; // one\n\nint y;\n")
    b.write_text("int x;   // two\nint y;\n")
    assert bench.kernel_source_hash([str(a)]) == bench.kernel_source_hash([str(b)])
    b.write_text("int x;\nint z;\n")
    assert bench.kernel_source_hash([str(a)]) != bench.kernel_source_hash([str(b)])
