"""The measured-ceiling kernels the benchmark reports against: the copy
kernel copies, and the MFMA kernel runs and reports its FLOPs."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as gfg

pytestmark = pytest.mark.gpu


def test_ceiling_copy_copies():
    dev = torch.device("cuda:0")
    n = (1 << 20) + 48
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev)
    dst = torch.zeros_like(src)
    gfg.ceiling_copy(src.data_ptr(), dst.data_ptr(), n)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_ceiling_read_reads_every_word():
    """The XOR of the per-wave sinks is the XOR of every 32-bit word read."""
    dev = torch.device("cuda:0")
    n = (3 << 20) + 16 * 5                     # a ragged tail past the unrolled loop
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.full((cus * 64,), -1, dtype=torch.int32, device=dev)
    gfg.ceiling_read(src.data_ptr(), n, sink.data_ptr(), sink.numel())
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


def test_ceiling_mfma_runs_and_counts():
    dev = torch.device("cuda:0")
    nb = gfg.ceiling_mfma_operand_bytes()
    ops = torch.full((nb,), 0x38, dtype=torch.uint8, device=dev)     # E4M3 1.0
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    flops = gfg.ceiling_mfma(ops.data_ptr(), nb, 3, sink.data_ptr(), sink.numel())
    torch.cuda.synchronize()
    assert flops == cus * 8 * 3 * 16 * 2 * 32 * 32 * 64
    # every product is 1 * 1 with unit scales: each accumulator element sums
    # 3 iterations x 2 K halves x 64 products, and a lane holds 8 x 16 of them
    assert torch.all(sink == 3 * 2 * 64 * 128).item()



def test_device_peak_matches_device_properties():
    """CUs x 8192 FP8 FLOP per clock at the device's maximum shader clock."""
    props = torch.cuda.get_device_properties(0)
    p = gfg.device_peak()
    assert p["cus"] == props.multi_processor_count
    assert 1000 <= p["max_sclk_mhz"] <= 3000
    assert p["fp8_tflops"] == pytest.approx(p["cus"] * 8192 * p["max_sclk_mhz"] * 1e6 / 1e12, rel=1e-3)


def test_ceiling_mfma_16x16x128_runs_and_counts():
    dev = torch.device("cuda:0")
    nb = gfg.ceiling_mfma_operand_bytes()
    ops = torch.full((nb,), 0x38, dtype=torch.uint8, device=dev)     # E4M3 1.0
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    flops = gfg.ceiling_mfma_16x16x128(ops.data_ptr(), nb, 3, sink.data_ptr(), sink.numel())
    torch.cuda.synchronize()
    assert flops == cus * 8 * 3 * 32 * 2 * 16 * 16 * 128
    # each accumulator element sums 3 iterations x 128 products of 1 * 1, and
    # a lane holds 32 x 4 of them
    assert torch.all(sink == 3 * 128 * 128).item()
