"""Seeded synthetic inputs for the grouped FP8 GEMM.

This module only draws float32 tensors and routing metadata; it holds none of
the method's arithmetic (no quantization, no scaling, no products), so both
the HIP path and the CPU oracle can be fed from it.

The shapes follow the coverage named on the first reference page, "Grouped
and Batched GEMM kernels with blockscaling matching DeepGEMM API" (section
"Test plan"): 1-8 groups, 100 (unaligned) to 1024 rows per group, and the
DeepSeek-V3 expert shapes N=2048/K=7168 and N=7168/K=2304, bf16 and f16 out.
No public dataset or weights are involved: every value is a seeded draw.

Recipe (numpy PCG64, seed = 1000 + workload index):
  * A, B ~ N(0, 1) float32; padding rows of a contiguous A are zero;
  * the prefill workload multiplies each row of A by 10**U(-2, 2);
  * random group sizes are integers uniform on [100, 1024] inclusive;
  * random masked_m are integers uniform on [0, 1024] inclusive, then two
    seeded distinct groups are set to 0 and 1024.

gemm1 with silu_mul (third reference page, the MoE gemm1/gemm2 pull request,
section "Results"): the Kimi-K2.5 TP=4 expert shape, 385 experts, hidden size
K = 7168, intermediate size I = 512 (so B[g] is [2*I, K]: gate rows, then up
rows), top-9 routing.  For a batch of T tokens each token picks 9 distinct
experts uniformly at random (seeded), and an expert's rows are the tokens
routed to it, padded to a multiple of 128.  The 385 weight matrices are 8
seeded N(0,1) draws repeated in turn (expert g uses draw g % 8): the kernel
reads 385 separate copies from device memory, but the host draws and
quantizes only 8 (11 GB of float32 otherwise).

MXFP8 (the third page's MX kernels, with E4M3 elements): the same data
recipes, quantized with one E8M0 scale per 32 K elements of every row --
the benchmarked 4 x 1024, N=2048, K=7168 shape and the Kimi gemm1 shape.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ALIGN = 128   # each expert's rows start on a multiple of 128 in the contiguous layout


@dataclass
class Workload:
    name: str
    layout: str                 # "contiguous" or "masked"
    G: int
    N: int
    K: int
    out_dtype: str              # "bf16" or "f16"
    seed: int
    m_per_group: list = field(default_factory=list)   # contiguous: valid rows per group
    M_max: int = 0                                    # masked: rows per group buffer
    masked_m: list = field(default_factory=list)      # masked: valid rows per group
    row_log10_range: tuple | None = None              # per-token magnitude 10**U(lo, hi)
    op: str = "gemm"                                  # "gemm", "silu_mul" (N = 2*I), "mx" / "mx4" (MXFP8 / MXFP4),
                                                      # "mx4_silu" (MXFP4 gemm1 with silu_mul, N = 2*I)
    b_distinct: int = 0                               # > 0: expert g's B is draw g % b_distinct

    @property
    def I(self) -> int:
        """silu_mul output width (half of B's rows)."""
        return self.N // 2

    @property
    def M(self) -> int:
        if self.layout == "masked":
            return self.G * self.M_max
        return sum(-(-m // ALIGN) * ALIGN for m in self.m_per_group)

    @property
    def m_valid(self) -> int:
        if self.layout == "masked":
            return int(sum(min(max(m, 0), self.M_max) for m in self.masked_m))
        return int(sum(self.m_per_group))

    @property
    def flops(self) -> int:
        """Algorithmic FLOPs over valid rows: 2 * M_valid * N * K."""
        return 2 * self.m_valid * self.N * self.K


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def standard_workloads() -> list[Workload]:
    """The five reference workloads (index i uses seed 1000 + i)."""
    ws = []
    ws.append(Workload("contig_g2_m100_n256_k256", "contiguous", 2, 256, 256, "bf16", 1000,
                       m_per_group=[100, 100]))
    ws.append(Workload("contig_g4_m1024_n2048_k7168", "contiguous", 4, 2048, 7168, "bf16", 1001,
                       m_per_group=[1024] * 4))
    r = _rng(1002)
    ws.append(Workload("contig_g8_mrand_n7168_k2304", "contiguous", 8, 7168, 2304, "f16", 1002,
                       m_per_group=[int(v) for v in r.integers(100, 1024, size=8, endpoint=True)]))
    r = _rng(1003)
    mm = [int(v) for v in r.integers(0, 1024, size=8, endpoint=True)]
    i0, i1 = (int(v) for v in r.choice(8, size=2, replace=False))
    mm[i0], mm[i1] = 0, 1024
    ws.append(Workload("masked_g8_m1024_n2048_k7168", "masked", 8, 2048, 7168, "bf16", 1003,
                       M_max=1024, masked_m=mm))
    ws.append(Workload("contig_g8_m4096_n7168_k2304_logmag", "contiguous", 8, 7168, 2304, "bf16",
                       1004, m_per_group=[4096] * 8, row_log10_range=(-2.0, 2.0)))
    return ws


def context_workloads() -> list[Workload]:
    """Shapes outside the five reference workloads, measured for context.

    ``dense_g1_m4096_n4096_k16384``: one group, a plain 4096 x 4096 x 16384
    block-scaled GEMM, the shape at which the second reference page
    ("[Kernel][MI350] cache-aware 8-wave BF16/FP16 GEMM", section "Perf", its
    first table) quotes an FP8 dense throughput (row-scaled there, on another
    power profile; block-scaled here).  A, B ~ N(0, 1), seed 1005.
    """
    return [Workload("dense_g1_m4096_n4096_k16384", "contiguous", 1, 4096, 16384, "bf16", 1005,
                     m_per_group=[4096])]


def _topk_counts(rng: np.random.Generator, tokens: int, experts: int, k: int) -> list:
    """Rows per expert when each of `tokens` tokens picks k distinct experts uniformly."""
    counts = np.zeros(experts, dtype=np.int64)
    for _ in range(tokens):
        counts[rng.choice(experts, size=k, replace=False)] += 1
    return [int(c) for c in counts]


def gemm1_workloads() -> list[Workload]:
    """gemm1 + silu_mul at the Kimi-K2.5 TP=4 expert shape (385 experts,
    K = 7168, I = 512, top 9) for a 4096-token batch, seed 1006."""
    return [Workload("kimi_tp4_gemm1_t4096", "contiguous", 385, 1024, 7168, "bf16", 1006,
                     m_per_group=_topk_counts(_rng(1006), 4096, 385, 9), op="silu_mul", b_distinct=8)]


def mx_workloads() -> list[Workload]:
    """MX GEMMs: the benchmarked contiguous shape and the Kimi-K2.5 TP=4 gemm1
    shape without its epilogue, in MXFP8 (seeds 1007, 1008) and in MXFP4, the
    page's a4w4 (seeds 1009, 1010); and the Kimi gemm1 as the page runs it,
    a4w4 with silu_mul (seed 1011, B [2I, K] with I = 512); N(0,1) data."""
    return [Workload("mx_contig_g4_m1024_n2048_k7168", "contiguous", 4, 2048, 7168, "bf16", 1007,
                     m_per_group=[1024] * 4, op="mx"),
            Workload("mx_kimi_tp4_gemm1_t4096", "contiguous", 385, 1024, 7168, "bf16", 1008,
                     m_per_group=_topk_counts(_rng(1008), 4096, 385, 9), op="mx", b_distinct=8),
            Workload("mx4_contig_g4_m1024_n2048_k7168", "contiguous", 4, 2048, 7168, "bf16", 1009,
                     m_per_group=[1024] * 4, op="mx4"),
            Workload("mx4_kimi_tp4_gemm1_t4096", "contiguous", 385, 1024, 7168, "bf16", 1010,
                     m_per_group=_topk_counts(_rng(1010), 4096, 385, 9), op="mx4", b_distinct=8),
            Workload("mx4_silu_kimi_tp4_gemm1_t4096", "contiguous", 385, 1024, 7168, "bf16", 1011,
                     m_per_group=_topk_counts(_rng(1011), 4096, 385, 9), op="mx4_silu", b_distinct=8)]


def workload(name_or_index) -> Workload:
    """A standard workload by index or name, a context workload by name, or an
    ad-hoc one named ``contig_g{G}_m{rows per group}_n{N}_k{K}`` or
    ``masked_g{G}_m{M_max}_n{N}_k{K}`` (every group full; bf16 out; seed 2000)."""
    ws = standard_workloads()
    if isinstance(name_or_index, int):
        return ws[name_or_index]
    for w in ws + context_workloads():
        if w.name == name_or_index:
            return w
    if name_or_index.startswith("kimi_"):
        for w in gemm1_workloads():
            if w.name == name_or_index:
                return w
    if name_or_index.startswith(("mx_", "mx4_")):
        for w in mx_workloads():
            if w.name == name_or_index:
                return w
    import re
    m = re.fullmatch(r"(contig|masked)_g(\d+)_m(\d+)_n(\d+)_k(\d+)", name_or_index)
    if m:
        kind, G, rows, N, K = m.group(1), *(int(v) for v in m.groups()[1:])
        if kind == "contig":
            return Workload(name_or_index, "contiguous", G, N, K, "bf16", 2000, m_per_group=[rows] * G)
        return Workload(name_or_index, "masked", G, N, K, "bf16", 2000, M_max=rows, masked_m=[rows] * G)
    raise KeyError(name_or_index)


def contiguous_layout(m_per_group, align: int = ALIGN) -> np.ndarray:
    """int32 [M]: expert id per row, each expert's run padded with -1 to a multiple of align."""
    parts = []
    for g, m in enumerate(m_per_group):
        padded = -(-m // align) * align
        parts.append(np.full(m, g, dtype=np.int32))
        parts.append(np.full(padded - m, -1, dtype=np.int32))
    if not parts:
        return np.zeros(0, dtype=np.int32)
    return np.concatenate(parts)


def draw(w: Workload, seed_offset: int = 0):
    """Draw the float32 inputs of a workload.

    Contiguous: returns dict(a [M, K], b [G, N, K], grouped_layout [M]).
    Masked:     returns dict(a [G, M_max, K], b [G, N, K], masked_m [G]).
    With ``b_distinct`` > 0, ``b`` holds only the distinct draws
    [b_distinct, N, K] and ``b_index`` [G] names the draw each expert uses.
    ``seed_offset`` gives independent input sets of the same shape.
    """
    rng = _rng(w.seed + 7919 * seed_offset)
    if w.layout == "masked":
        a = rng.standard_normal((w.G, w.M_max, w.K), dtype=np.float32)
        out = dict(a=a, masked_m=np.asarray(w.masked_m, dtype=np.int32))
    else:
        layout = contiguous_layout(w.m_per_group)
        a = rng.standard_normal((layout.size, w.K), dtype=np.float32)
        a[layout < 0] = 0.0
        out = dict(a=a, grouped_layout=layout)
    if w.row_log10_range is not None:
        lo, hi = w.row_log10_range
        mag = np.power(10.0, rng.uniform(lo, hi, size=a.shape[:-1] + (1,))).astype(np.float32)
        a *= mag
    if w.b_distinct:
        out["b"] = rng.standard_normal((w.b_distinct, w.N, w.K), dtype=np.float32)
        out["b_index"] = np.arange(w.G, dtype=np.int64) % w.b_distinct
    else:
        out["b"] = rng.standard_normal((w.G, w.N, w.K), dtype=np.float32)
    return out


def small_contiguous(seed: int, m_per_group, N: int, K: int, align: int = ALIGN):
    """A small contiguous case for parity tests (N(0,1) data, zero padding rows)."""
    rng = _rng(seed)
    layout = contiguous_layout(m_per_group, align)
    a = rng.standard_normal((layout.size, K), dtype=np.float32)
    a[layout < 0] = 0.0
    b = rng.standard_normal((len(m_per_group), N, K), dtype=np.float32)
    return dict(a=a, b=b, grouped_layout=layout)


def small_masked(seed: int, masked_m, M_max: int, N: int, K: int):
    """A small masked case for parity tests."""
    rng = _rng(seed)
    G = len(masked_m)
    a = rng.standard_normal((G, M_max, K), dtype=np.float32)
    b = rng.standard_normal((G, N, K), dtype=np.float32)
    return dict(a=a, b=b, masked_m=np.asarray(masked_m, dtype=np.int32))


def integer_case(seed: int, G: int, rows: int, N: int, K: int, vmax: int = 4):
    """Small-integer e4m3 inputs for the exact special case.

    Returns raw FP8 codes and E8M0 bytes directly (no quantizer involved):
    every element is an integer in [-vmax, vmax] (exactly representable in
    e4m3) and every scale byte is in {127, 128, 129}.  The products and all
    partial sums are then integers far below 2**24, so any fp32 summation
    order gives the exact result.
    """
    rng = _rng(seed)
    ints_a = rng.integers(-vmax, vmax, size=(G * rows, K), endpoint=True)
    ints_b = rng.integers(-vmax, vmax, size=(G, N, K), endpoint=True)
    sa = rng.integers(127, 129, size=(-(-K // 128), G * rows), endpoint=True).astype(np.uint8)
    sb = rng.integers(127, 129, size=(G, -(-N // 128), -(-K // 128)), endpoint=True).astype(np.uint8)
    return dict(ints_a=ints_a, ints_b=ints_b, scale_a=sa, scale_b=sb,
                grouped_layout=np.repeat(np.arange(G, dtype=np.int32), rows))
