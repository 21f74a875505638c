"""Benchmark: grouped FP8 block-scaled GEMM throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one call of the grouped GEMM (tile scheduling, LDS-staged scaled-MFMA
K-loop and epilogue, all inside the one kernel) over one batch of seeded
synthetic inputs already resident in HBM (for a gemm1 workload, such as
kimi_tp4_gemm1_t4096, the call with the fused silu_mul epilogue; for an mx_*
workload, the MXFP8 GEMM with one scale per 32 K elements; for mx4_*, the
MXFP4 one, priced against the FP4 peak); quantization happens before timing,
as the inputs of the op are FP8 bytes and E8M0 scales.  Several input sets
whose combined size exceeds the 256 MB Infinity Cache rotate between steps, so
each step streams its operands from HBM.

Prints one JSON line: valid-row TFLOP/s (2 * M_valid * N * K / t), the
roofline object for the kernel (HIP events on the launch stream), and the CPU
oracle timed on the host cores on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0          # MI355X dense FP8 MFMA peak
PEAK_FP4_TFLOPS = 10100.0         # MI355X dense FP4 (and FP6) MFMA peak
PEAK_HBM_GBS = 8000.0
RIDGE_FLOP_PER_BYTE = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
# The largest of the five reference workloads: 8 experts x 4096 rows, N=7168, K=2304.
DEFAULT_WORKLOAD = "contig_g8_m4096_n7168_k2304_logmag"
_CSRC = os.path.join(ROOT, "fp8_block_scaled_amd", "csrc")
KERNEL_SRC = [os.path.join(_CSRC, n) for n in ("gfg_gemm.hip", "gfg_gemm256.hip", "gfg_device.h")]
QUANT_SRC = [os.path.join(_CSRC, "gfg_quant.hip")]


def kernel_source_hash(paths=KERNEL_SRC) -> str:
    """Hash of the kernel sources' code: // comments and blank lines removed,
    so an edit to comments alone keeps stored counter results valid."""
    import re
    code = []
    for path in paths:
        with open(path) as f:
            lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in f]
        code.append("\n".join(ln for ln in lines if ln))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def algorithmic_bytes(w, layout=None) -> int:
    """Bytes the op must move at least once: A rows of non-empty tiles, B of the
    experts that have rows, both scale tensors' used parts, and D's valid rows."""
    KB, NB = w.K // 128, w.N // 128
    out_b = 2
    out_cols = w.I if w.op in ("silu_mul", "mx4_silu") else w.N
    mx = w.op in ("mx", "mx4", "mx4_silu")
    a_scale_per_row = w.K // 32 if mx else KB
    b_scale = w.N * (w.K // 32) if mx else NB * KB
    elem = 0.5 if w.op in ("mx4", "mx4_silu") else 1.0          # bytes per A/B element
    if w.layout == "masked":
        tiles_rows = sum(-(-min(max(m, 0), w.M_max) // 128) * 128 for m in w.masked_m)
        a_rows = sum(min(max(m, 0), w.M_max) for m in w.masked_m)
        groups = sum(1 for m in w.masked_m if m > 0)
    else:
        tiles_rows = w.M
        a_rows = w.M
        groups = sum(1 for m in w.m_per_group if m > 0)
    return int(a_rows * w.K * elem + tiles_rows * a_scale_per_row + groups * (w.N * w.K * elem + b_scale)
               + w.m_valid * out_cols * out_b)


def traffic_from_profile(w):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
    on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def _pmc_per_dispatch(root, counter):
    """{kernel name: average per dispatch} of one counter from a rocprofv3 --pmc csv run."""
    import collections
    import csv
    import glob
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    files = glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {root}")
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: (sum(d.values()) / len(d), len(d)) for k, d in per.items()}


def summarize_trace(root, last=100):
    """Per-kernel durations from a rocprofv3 --kernel-trace csv run: calls,
    mean over all dispatches, and the mean of the final `last` dispatches (the
    timing protocol of the second reference page, section "Performance":
    AMD_SERIALIZE_KERNEL=3 and the final 100 matching dispatches)."""
    import collections
    import csv
    import glob
    files = glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {root}")
    per = collections.defaultdict(list)
    res = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
                per[r["Kernel_Name"]].append((t0, t1 - t0))
                # kernel resources as the trace records them (first dispatch)
                res.setdefault(r["Kernel_Name"], {k: int(r[c]) for k, c in (
                    ("lds_bytes", "LDS_Block_Size"), ("scratch_bytes", "Scratch_Size"), ("vgpr", "VGPR_Count"),
                    ("agpr", "Accum_VGPR_Count"), ("sgpr", "SGPR_Count"), ("workgroup", "Workgroup_Size_X"),
                    ("grid", "Grid_Size_X")) if c in r and r[c] not in ("", None)})
    out = []
    for name, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        v.sort()
        d = np.array([x for _, x in v], dtype=np.float64)
        tail = d[-last:]
        out.append({"kernel": name, "calls": len(d), "mean_ns": round(float(d.mean()), 1),
                    f"final{last}_mean_ns": round(float(tail.mean()), 1), f"final{last}_min_ns": int(tail.min()),
                    f"final{last}_max_ns": int(tail.max()), f"final{last}_std_ns": round(float(tail.std()), 1),
                    "resources": res.get(name, {})})
    return out


def quant_traffic_path(w, in_dtype):
    return os.path.join(ROOT, "profiles", f"traffic_quant_{w.name}_{in_dtype}.json")


def summarize_traffic(workload, fetch_dir, write_dir, copy_bytes, quant_in=None):
    """HBM bytes per launch of the GEMM kernel (or, with quant_in, of the device
    quantizer on the workload's A operand in that input dtype): FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) divided by what the same counter reads per
    byte for the plain copy kernel of known size that the run also launched."""
    from fp8_block_scaled_amd import workloads as wl
    w = wl.workload(workload)
    if quant_in:
        a = wl.draw(w)["a"]
        G, M, K = (1, *a.shape) if a.ndim == 2 else a.shape
        algo, path, src, match = (quant_bytes(G, M, K, 2 if quant_in == "bf16" else 4),
                                  quant_traffic_path(w, quant_in), QUANT_SRC, "quant_act_1x128")
    else:
        algo, path, src, match = (algorithmic_bytes(w), os.path.join(ROOT, "profiles", f"traffic_{w.name}.json"),
                                  KERNEL_SRC, "grouped_fp8_gemm")
    out = {"workload": w.name if not quant_in else f"quant_act_1x128 of {w.name}.a ({quant_in})",
           "kernel_source_sha256_16": kernel_source_hash(src)}
    total = 0.0
    for counter, root in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _pmc_per_dispatch(root, counter)
        gemm = [v for k, v in per.items() if match in k]
        copy = [(k, v) for k, v in per.items() if "neg" in k.lower()]
        if not gemm or not copy:
            raise SystemExit(f"{counter}: need both the GEMM and the copy kernel in {root}: {list(per)}")
        ck, (cval, _) = copy[0]
        factor = cval * 1024.0 / copy_bytes
        gbytes = gemm[0][0] * 1024.0 / factor
        total += gbytes
        kk = "quant" if quant_in else "gemm"
        out[counter] = {f"{kk}_KiB_per_dispatch": round(gemm[0][0], 1), f"{kk}_dispatches": gemm[0][1],
                        "copy_kernel": ck, "copy_bytes": copy_bytes, "copy_KiB_per_dispatch": round(cval, 1),
                        "factor": round(factor, 4), f"{kk}_bytes_per_launch": int(gbytes)}
    out["hbm_bytes_per_launch"] = int(total)
    out["algorithmic_bytes_per_launch"] = algo
    out["traffic_over_algorithmic"] = round(total / algo, 3)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))


CPU_MIN_SECONDS = 10.0   # the oracle repeats its sample until this much host time has passed


def _repeat_timed(fn):
    """Run fn until CPU_MIN_SECONDS have passed (at least once): (seconds per run, runs)."""
    runs, t0 = 0, time.perf_counter()
    while True:
        fn()
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_MIN_SECONDS:
            return dt / runs, runs


CPU_SAMPLE_FLOPS = 2e12   # larger workloads time a bounded sample of one expert's rows


def cpu_baseline(w, x):
    """The fp64 oracle (dequantize, then matmul) on the same workload, timed on
    the host.  Its own quantizer prepares the operands outside the timing; the
    timed sample repeats until at least CPU_MIN_SECONDS of host time.  `cores`
    is the BLAS thread count the matmul ran with; `affinity_cores` the CPUs
    the process may run on."""
    from threadpoolctl import threadpool_info
    from oracle import fp8_oracle as o
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    affinity = len(os.sched_getaffinity(0))
    quant_mx = o.quantize_mx4_1x32 if w.op in ("mx4", "mx4_silu") else o.quantize_mx_1x32
    gemm_mx = {"mx4": o.grouped_gemm_mx4_contiguous, "mx4_silu": o.grouped_gemm_mx4_silu_mul_contiguous}.get(
        w.op, o.grouped_gemm_mx_contiguous)

    def result(flops, dt, runs, what, parts=None):
        r = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
             "affinity_cores": affinity, "kind": "oracle",
             "sample": f"{what}, {dt:.2f} s per run, {runs} runs; quantization untimed"}
        if parts:
            r["parts_s"] = parts
        return r

    def parts_of(xa, xb, quant_a, gemm_fn):
        """Seconds per run of the oracle's quantize (A and B), dequantize
        (A and B) and grouped GEMM (which dequantizes, then multiplies), each
        on the timed sample (one run each)."""
        t0 = time.perf_counter()
        qa, sa = quant_a(xa)
        qb, sb = o.quantize_weight_128x128(xb)
        t1 = time.perf_counter()
        o.dequantize_act(qa.reshape(-1, qa.shape[-1]), sa.reshape(-1, sa.shape[-1]))
        o.dequantize_weight(qb, sb)
        t2 = time.perf_counter()
        gemm_fn(qa, sa, qb, sb)
        t3 = time.perf_counter()
        return {"quantize": round(t1 - t0, 3), "dequantize": round(t2 - t1, 3),
                "gemm_incl_dequantize": round(t3 - t2, 3)}

    if w.op in ("silu_mul", "mx4_silu") or (w.op in ("mx", "mx4") and w.b_distinct):
        # bounded sample: the rows of the first 16 experts (all 385 weight
        # matrices would be 22 GB in float64)
        n_exp = min(16, w.G)
        layout = x["grouped_layout"]
        rows = np.nonzero((layout >= 0) & (layout < n_exp))[0]
        sel = x["b_index"][:n_exp] if "b_index" in x else np.arange(n_exp)
        if w.op == "silu_mul":
            qa, sa = o.quantize_act_1x128(x["a"][rows])
            qb_d, sb_d = o.quantize_weight_128x128(x["b"])
            fn = lambda: o.grouped_gemm_silu_mul_contiguous(qa, sa, qb_d[sel], sb_d[sel], layout[rows])
            what = "fp64 dequantize + matmul + silu_mul"
        else:
            qa, sa = quant_mx(x["a"][rows])
            qb_d, sb_d = quant_mx(x["b"])
            fn = lambda: gemm_mx(qa, sa, qb_d[sel], sb_d[sel], layout[rows])
            what = "fp64 MX dequantize + matmul" + (" + silu_mul" if w.op == "mx4_silu" else "")
        dt, runs = _repeat_timed(fn)
        return result(2 * rows.size * w.N * w.K, dt, runs,
                      f"the rows of experts 0..{n_exp - 1} of {w.name} ({rows.size} of {w.m_valid} valid rows; {what})")
    if w.op in ("mx", "mx4"):
        qa, sa = quant_mx(x["a"])
        qb, sb = quant_mx(x["b"])
        dt, runs = _repeat_timed(lambda: gemm_mx(qa, sa, qb, sb, x["grouped_layout"]))
        return result(w.flops, dt, runs, f"full steps of {w.name} (fp64 MX dequantize + matmul over all valid rows)")
    if w.layout == "masked":
        qa, sa = o.quantize_act_masked(x["a"])
        qb, sb = o.quantize_weight_128x128(x["b"])
        dt, runs = _repeat_timed(lambda: o.grouped_gemm_masked(qa, sa, qb, sb, w.masked_m))
        parts = parts_of(x["a"], x["b"], o.quantize_act_masked,
                         lambda qa, sa, qb, sb: o.grouped_gemm_masked(qa, sa, qb, sb, w.masked_m))
        return result(w.flops, dt, runs, f"full steps of {w.name} (fp64 dequantize + matmul over all valid rows)",
                      parts)
    if w.flops > CPU_SAMPLE_FLOPS:
        # bounded sample: the first rows of expert 0, against expert 0's weights
        layout = x["grouped_layout"]
        rows = np.nonzero(layout == 0)[0][:512]
        xa, xb = x["a"][rows], x["b"][:1]
        lay0 = np.zeros(rows.size, dtype=layout.dtype)
        qa, sa = o.quantize_act_1x128(xa)
        qb, sb = o.quantize_weight_128x128(xb)
        dt, runs = _repeat_timed(lambda: o.grouped_gemm_contiguous(qa, sa, qb, sb, lay0))
        parts = parts_of(xa, xb, o.quantize_act_1x128,
                         lambda qa, sa, qb, sb: o.grouped_gemm_contiguous(qa, sa, qb, sb, lay0))
        return result(2 * rows.size * w.N * w.K, dt, runs,
                      f"the first {rows.size} rows of expert 0 of {w.name} against expert 0's {w.N}x{w.K} weights "
                      f"(fp64 dequantize + matmul)", parts)
    qa, sa = o.quantize_act_1x128(x["a"])
    qb, sb = o.quantize_weight_128x128(x["b"])
    dt, runs = _repeat_timed(lambda: o.grouped_gemm_contiguous(qa, sa, qb, sb, x["grouped_layout"]))
    parts = parts_of(x["a"], x["b"], o.quantize_act_1x128,
                     lambda qa, sa, qb, sb: o.grouped_gemm_contiguous(qa, sa, qb, sb, x["grouped_layout"]))
    return result(w.flops, dt, runs, f"full steps of {w.name} (fp64 dequantize + matmul over all valid rows)", parts)


def quant_bytes(G, M, K, in_size):
    """Algorithmic HBM bytes of one device quantizer call: read x, write the
    E4M3 codes and the E8M0 scale bytes."""
    return G * M * K * (in_size + 1) + G * M * (K // 128)


def quant_traffic(w, in_dtype):
    """HBM bytes per call of the device quantizer from stored counter runs, if
    they were taken on the current quantizer source (else None)."""
    path = quant_traffic_path(w, in_dtype)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash(QUANT_SRC):
        return None
    return t.get("hbm_bytes_per_launch")


def bench_quant(args):
    """The device activation quantizer on a workload's A operand (bf16 or f32
    input), timed with HIP events on its stream; HBM-bound, priced against
    8 TB/s on algorithmic bytes."""
    import torch
    import fp8_block_scaled_amd as gfg
    from fp8_block_scaled_amd import workloads as wl
    from oracle import fp8_oracle as o

    gfg.load_library()
    w = wl.workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if args.in_dtype == "bf16" else torch.float32
    in_size = 2 if args.in_dtype == "bf16" else 4
    x0 = wl.draw(w)["a"]
    if x0.ndim == 2:
        x0 = x0[None]
    G, M, K = x0.shape
    per_set = quant_bytes(G, M, K, in_size)
    nsets = args.sets or max(2, -(-(600 << 20) // per_set))
    xs, qs, ss = [], [], []
    for s in range(nsets):
        x = x0 if s == 0 else wl.draw(w, seed_offset=s)["a"].reshape(G, M, K)
        xs.append(torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt))
        qs.append(torch.empty((G, M, K), dtype=torch.uint8, device=dev))
        ss.append(torch.empty((G, K // 128, M), dtype=torch.uint8, device=dev))
    code = gfg.IN_BF16 if dt == torch.bfloat16 else gfg.IN_F32
    handle = torch.cuda.current_stream(dev).cuda_stream
    calls = [(xs[i].data_ptr(), code, G, M, K, qs[i].data_ptr(), ss[i].data_ptr(), handle) for i in range(nsets)]

    def step(i):
        rc = gfg.raw_quantize_act_device(*calls[i % nsets])
        if rc:
            raise gfg.GfgError(rc, gfg.load_library().grouped_fp8_last_error().decode())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i)
    stop.record()
    torch.cuda.synchronize(dev)
    ms = start.elapsed_time(stop) / args.steps
    gbs = per_set / (ms * 1e-3) / 1e9
    res = {
        "metric": "device activation quantizer GB/s (algorithmic bytes), 1 MI355X",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{args.in_dtype}->e4m3", "data": "synthetic",
        "config": {"workload": f"quant_act_1x128 of {w.name}.a", "G": G, "M": M, "K": K,
                   "in": args.in_dtype, "input_sets": nsets},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": quant_traffic(w, args.in_dtype)},
        "algorithmic_bytes_per_step": per_set,
    }
    if not args.no_cpu:
        rows = min(M, 8192)
        xs0 = xs[0][0, :rows].float().cpu().numpy()
        dtc, runs = _repeat_timed(lambda: o.quantize_act_1x128(xs0))
        res["cpu_baseline"] = {"value": round(quant_bytes(1, rows, K, in_size) / dtc / 1e9, 3), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"oracle quantize_act_1x128 on the first {rows} rows of group 0 "
                                         f"({rows}x{K}), {dtc:.2f} s per run, {runs} runs"}
    print(json.dumps(res), flush=True)
    if args.copy_bytes:
        del xs, qs, ss, calls
        # the calibration kernel of the counter passes: reads and writes copy_bytes each call
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize(dev)


def graph_cross_check(args, calls, sets, w, dev):
    """The second timing of the page-3 protocol (section "Measurement"): a
    hipGraph that holds graph_launches launches (the same rotating input sets),
    replayed, timed with HIP events on the replay stream and divided by the
    launches.  The output of input set 0 after the replays must equal, bit for
    bit, that of an eager launch on the same inputs."""
    import torch
    import fp8_block_scaled_amd as gfg
    n = args.graph_launches
    s = torch.cuda.Stream(dev)
    h = s.cuda_stream
    gcalls = [(fn, a[:-1] + (h,)) for fn, a in calls]

    def launch(i):
        fn, a = gcalls[i % len(gcalls)]
        rc = fn(*a)
        if rc:
            raise gfg.GfgError(rc, gfg.load_library().grouped_fp8_last_error().decode())

    torch.cuda.synchronize(dev)
    with torch.cuda.stream(s):
        launch(0)
    torch.cuda.synchronize(dev)
    eager = sets[0]["d"].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(n):
            launch(i)
    replays = max(3, args.steps // n)
    with torch.cuda.stream(s):           # replay() launches on the current stream
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize(dev)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(s)
        for _ in range(replays):
            g.replay()
        stop.record(s)
    torch.cuda.synchronize(dev)
    ms = start.elapsed_time(stop) / (replays * n)
    same = bool(torch.equal(sets[0]["d"].view(torch.int16), eager.view(torch.int16)))
    if not same:
        raise RuntimeError("graph replay output differs from the eager launch")
    return {"launches_per_graph": n, "replays": replays, "ms_per_launch": round(ms, 6),
            "TFLOPs": round(w.flops / (ms * 1e-3) / 1e12, 3), "matches_eager_bitwise": same}


def measure_ceilings(a_bytes, dev):
    """The committed ceiling kernels, timed with HIP events on their stream:
    the two scaled MFMAs alone on real E4M3 operands (the first bytes of the
    workload's A; the faster one is the ceiling), a 1 GiB HBM copy and a
    1 GiB HBM read."""
    import torch
    import fp8_block_scaled_amd as gfg
    s = torch.cuda.Stream(dev)
    h = s.cuda_stream
    nb = gfg.ceiling_mfma_operand_bytes()
    flat = a_bytes.reshape(-1).view(torch.uint8)
    if flat.numel() < nb:
        flat = flat.repeat(-(-nb // flat.numel()))
    ops = flat[:nb].clone()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    torch.cuda.synchronize(dev)

    def timed(fn, reps):
        with torch.cuda.stream(s):
            fn()
        torch.cuda.synchronize(dev)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(s)
        for _ in range(reps):
            fn()
        stop.record(s)
        torch.cuda.synchronize(dev)
        return start.elapsed_time(stop) / reps * 1e-3

    iters = 4000
    flops = [0.0]

    def mfma():
        flops[0] = gfg.ceiling_mfma(ops.data_ptr(), nb, iters, sink.data_ptr(), sink.numel(), h)

    t_m = timed(mfma, 20)
    flops16 = [0.0]

    def mfma16():
        flops16[0] = gfg.ceiling_mfma_16x16x128(ops.data_ptr(), nb, iters, sink.data_ptr(), sink.numel(), h)

    t_m16 = timed(mfma16, 20)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    t_c = timed(lambda: gfg.ceiling_copy(src.data_ptr(), dst.data_ptr(), nbytes, h), 20)
    rsink = torch.empty(cus * 64, dtype=torch.int32, device=dev)
    t_r = timed(lambda: gfg.ceiling_read(dst.data_ptr(), nbytes, rsink.data_ptr(), rsink.numel(), h), 20)
    del src, dst
    peak = gfg.device_peak()
    return {"device_peak_TFLOPs": round(peak["fp8_tflops"], 1), "device_cus": peak["cus"],
            "device_max_sclk_MHz": peak["max_sclk_mhz"],
            "mfma_TFLOPs": round(max(flops[0] / t_m, flops16[0] / t_m16) / 1e12, 1),
            "mfma_32x32x64_TFLOPs": round(flops[0] / t_m / 1e12, 1),
            "mfma_16x16x128_TFLOPs": round(flops16[0] / t_m16 / 1e12, 1),
            "mfma_kernel": f"the faster of gfg_ceiling_mfma ({iters} x 16 v_mfma_scale_f32_32x32x64_f8f6f4 per wave) "
                           f"and gfg_ceiling_mfma_16x16x128 ({iters} x 32 v_mfma_scale_f32_16x16x128_f8f6f4 per wave), "
                           "8 waves per CU",
            "copy_GBps": round(2 * nbytes / t_c / 1e9, 1),
            "copy_kernel": "gfg_ceiling_copy, 1 GiB, read + write bytes",
            "read_GBps": round(nbytes / t_r / 1e9, 1),
            "read_kernel": "gfg_ceiling_read, 1 GiB, non-temporal 16-byte loads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # The GPU's clock needs a few hundred ms of sustained load to settle at its
    # loaded frequency; a short warmup times part of the ramp.
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = enough to exceed 256 MB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run a plain copy kernel (torch.neg) over this many bytes 5 times "
                         "(the calibration kernel of the FETCH_SIZE / WRITE_SIZE counter passes)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of "
                         "'bench.py --copy-bytes B' into profiles/traffic_<workload>.json, then exit")
    ap.add_argument("--op", choices=("gemm", "quant"), default="gemm",
                    help="gemm: the grouped GEMM (the default); quant: the device activation quantizer "
                         "on the workload's A operand")
    ap.add_argument("--in-dtype", choices=("bf16", "f32"), default="bf16", help="--op quant input dtype")
    ap.add_argument("--tile", choices=("auto", "128x256", "256x256"), default="auto",
                    help="output tile of the plain FP8 GEMM (auto: chosen per launch)")
    ap.add_argument("--num-xcd", type=int, default=8, help="XCDs the tile order is split over (1 or 8)")
    ap.add_argument("--group-m", type=int, default=0, help="grouped-M width in M tiles (0: kernel default)")
    ap.add_argument("--graph-launches", type=int, default=20,
                    help="cross-check: time a hipGraph of this many launches, replayed; 0 skips it")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured MFMA-only, copy and read ceilings")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print per-kernel durations (all dispatches and the final 100) of a rocprofv3 "
                         "--kernel-trace csv run under DIR, then exit")
    args = ap.parse_args()
    if args.trace_summary:
        for r in summarize_trace(args.trace_summary):
            print(json.dumps(r))
        return
    if args.op == "quant":
        if args.gpus != 1:
            raise SystemExit("this benchmark runs on one GPU only")
        if args.traffic_from:
            if not args.copy_bytes:
                raise SystemExit("--traffic-from needs the --copy-bytes the counter runs used")
            summarize_traffic(args.workload, *args.traffic_from, args.copy_bytes, quant_in=args.in_dtype)
            return
        bench_quant(args)
        return
    if args.traffic_from:
        if not args.copy_bytes:
            raise SystemExit("--traffic-from needs the --copy-bytes the counter runs used")
        summarize_traffic(args.workload, *args.traffic_from, args.copy_bytes)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the grouped GEMM has no "
                                   "multi-GPU path here (experts would be sharded across GPUs with "
                                   "an all-to-all token exchange around the unchanged kernel)"}))
        sys.exit(2)

    import torch
    import fp8_block_scaled_amd as gfg
    from fp8_block_scaled_amd import workloads as wl

    gfg.load_library()
    gfg.set_tile_shape({"auto": gfg.TILE_AUTO, "128x256": gfg.TILE_128x256, "256x256": gfg.TILE_256x256}[args.tile])
    gfg.set_tile_order(args.num_xcd, args.group_m)
    w = wl.workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    per_set = algorithmic_bytes(w)
    nsets = args.sets or max(2, -(-(300 << 20) // per_set))
    sets = []
    x0 = None
    for s in range(nsets):
        x = wl.draw(w, seed_offset=s)
        if s == 0:
            x0 = x
        mxq = {"mx": gfg.fp8_quantize_mx_1x32, "mx4": gfg.fp4_quantize_mx_1x32,
               "mx4_silu": gfg.fp4_quantize_mx_1x32}.get(w.op)
        if w.layout == "masked":
            qa, sa = mxq(x["a"]) if mxq else gfg.fp8_quantize_act_masked(x["a"])
            meta = torch.from_numpy(np.asarray(w.masked_m, np.int32)).to(dev)
            M_rows = w.G * w.M_max
        else:
            qa, sa = mxq(x["a"]) if mxq else gfg.fp8_quantize_act_1x128(x["a"])
            meta = torch.from_numpy(x["grouped_layout"]).to(dev)
            M_rows = w.M
        qb, sb = mxq(x["b"]) if mxq else gfg.fp8_quantize_weight_128x128(x["b"])
        b_dev, sb_dev = torch.from_numpy(qb).to(dev), torch.from_numpy(sb).to(dev)
        if w.b_distinct:      # every expert its own copy in device memory
            idx = torch.from_numpy(x["b_index"]).to(dev)
            b_dev, sb_dev = b_dev.index_select(0, idx), sb_dev.index_select(0, idx)
        out_cols = w.I if w.op in ("silu_mul", "mx4_silu") else w.N
        t = dict(a=torch.from_numpy(qa).to(dev), sa=torch.from_numpy(sa).to(dev),
                 b=b_dev, sb=sb_dev, meta=meta,
                 d=torch.empty((M_rows, out_cols), dtype=torch.bfloat16 if w.out_dtype == "bf16" else torch.float16,
                               device=dev))
        sets.append(t)
        if s:
            del x
    out_code = gfg.OUT_BF16 if w.out_dtype == "bf16" else gfg.OUT_F16
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream

    # prepared launches: pointers and sizes resolved once
    calls = []
    for t in sets:
        silu = w.op in ("silu_mul", "mx4_silu")
        n_arg = w.I if silu else w.N      # the silu_mul entry points take I (B has 2*I rows)
        fns = {"gemm": (gfg.raw_contiguous, gfg.raw_masked), "silu_mul": (gfg.raw_silu_mul_contiguous,
               gfg.raw_silu_mul_masked), "mx": (gfg.raw_mx_contiguous, gfg.raw_mx_masked),
               "mx4": (gfg.raw_mx4_contiguous, gfg.raw_mx4_masked),
               "mx4_silu": (gfg.raw_mx4_silu_mul_contiguous, gfg.raw_mx4_silu_mul_masked)}[w.op]
        if w.layout == "masked":
            a = (t["a"].data_ptr(), t["sa"].data_ptr(), t["b"].data_ptr(), t["sb"].data_ptr(),
                 t["meta"].data_ptr(), t["d"].data_ptr(), w.G, w.M_max, n_arg, w.K, out_code, handle)
            calls.append((fns[1], a))
        else:
            a = (t["a"].data_ptr(), t["sa"].data_ptr(), t["b"].data_ptr(), t["sb"].data_ptr(),
                 t["meta"].data_ptr(), t["d"].data_ptr(), w.M, n_arg, w.K, w.G, out_code, handle)
            calls.append((fns[0], a))

    def step(i):
        fn, a = calls[i % len(calls)]
        rc = fn(*a)
        if rc:
            raise gfg.GfgError(rc, gfg.load_library().grouped_fp8_last_error().decode())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / args.steps
    tflops = w.flops / (ms * 1e-3) / 1e12
    traffic = traffic_from_profile(w)
    abytes = algorithmic_bytes(w)
    gbps = abytes / (ms * 1e-3) / 1e9
    peak = PEAK_FP4_TFLOPS if w.op in ("mx4", "mx4_silu") else PEAK_FP8_TFLOPS
    if w.flops / abytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        roofline = {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": traffic}
    else:   # below the ridge the algorithmic bytes bound the step
        roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBS, 4), "traffic": traffic}

    graph = graph_cross_check(args, calls, sets, w, dev) if args.graph_launches > 0 else None
    ceilings = None if args.no_ceilings else measure_ceilings(sets[0]["a"], dev)

    res = {
        "metric": "grouped FP8 GEMM TFLOP/s (valid rows) and % of FP8 MFMA peak, 1 MI355X",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4e2m1" if w.op in ("mx4", "mx4_silu") else "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "op": w.op, "layout": w.layout, "G": w.G, "N": w.N, "K": w.K,
                   "M_rows": w.M, "M_valid": w.m_valid, "out": w.out_dtype,
                   "input_sets": nsets, "parallelism": "none (1 GPU)", "tile": args.tile,
                   "num_xcd": args.num_xcd, "group_m": args.group_m},
        "pct_of_fp8_peak": round(100.0 * tflops / PEAK_FP8_TFLOPS, 2),
        "pct_of_mfma_peak_for_dtype": round(100.0 * tflops / peak, 2),
        "roofline": roofline,
        "algorithmic_bytes_per_step": abytes,
        "algorithmic_GBps": round(gbps, 1),
        "host_wall_s_timed": round(wall, 4),
    }
    if graph:
        res["graph_cross_check"] = graph
    if ceilings:
        if w.op in ("mx4", "mx4_silu"):
            # the ceiling kernel and the device peak are FP8's; an FP4 MFMA of the
            # same shape holds the matrix pipe half as long
            ceilings["frac_of_device_peak"] = round(tflops / (2 * ceilings["device_peak_TFLOPs"]), 4)
            ceilings["frac_of_mfma_ceiling"] = None
        else:
            ceilings["frac_of_mfma_ceiling"] = round(tflops / ceilings["mfma_TFLOPs"], 4)
            ceilings["frac_of_device_peak"] = round(tflops / ceilings["device_peak_TFLOPs"], 4)
        if roofline["bound"] == "hbm":     # algorithmic bytes against the measured memory rates
            ceilings["frac_of_read_ceiling"] = round(gbps / ceilings["read_GBps"], 4)
            ceilings["frac_of_copy_ceiling"] = round(gbps / ceilings["copy_GBps"], 4)
        res["ceilings"] = ceilings
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, x0)
    print(json.dumps(res), flush=True)
    if args.copy_bytes:
        del sets, calls
        # one elementwise kernel per call that reads and writes copy_bytes each
        # (a driver memcpy may be split over several dispatches)
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize(dev)


if __name__ == "__main__":
    main()
