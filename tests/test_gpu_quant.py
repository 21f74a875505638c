"""GPU parity of the device activation quantizer against the CPU oracle.

The quantizer's outputs are integers (E4M3 codes, E8M0 bytes), so the bar is
bit-exact equality with ``oracle.quantize_act_1x128`` on the same inputs
(bfloat16 inputs are widened to float32 exactly before the oracle sees them).
The two documented departures from the host quantizer, which cannot return
an error from the device, are checked on their own: a block holding a NaN or
an infinity gets scale byte 255 and E4M3 NaN codes, and a block whose scale
would fall below 2^-127 gets 2^-127.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as gfg
from fp8_block_scaled_amd import workloads as wl
from oracle import fp8_oracle as o

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _draw(shape, seed, logmag=True):
    """N(0,1) rows, each scaled by 10^U(-2, 2) (per-token magnitudes)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if logmag:
        mag = np.power(10.0, rng.uniform(-2.0, 2.0, size=shape[:-1] + (1,))).astype(np.float32)
        x = x * mag
    return x


def _device_quant(x_host, dtype):
    x = torch.from_numpy(np.ascontiguousarray(x_host)).to(DEV).to(dtype)
    q, s = gfg.fp8_quantize_act_1x128_device(x)
    torch.cuda.synchronize(DEV)
    widened = x.float().cpu().numpy()          # the values the device saw, exactly
    return q.cpu().numpy(), s.cpu().numpy(), widened


def _oracle(x):
    if x.ndim == 2:
        return o.quantize_act_1x128(x)
    return o.quantize_act_masked(x)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 128), (7, 256), (65, 384), (130, 1152), (257, 2304), (3, 70, 384),
                                   (2, 20001, 1152)])
def test_device_quant_bit_exact(shape, dtype):
    print(f"[quant] shape={shape} dtype={dtype}", flush=True)
    x = _draw(shape, seed=sum(shape))
    q, s, xw = _device_quant(x, dtype)
    oq, os_ = _oracle(xw)
    assert np.array_equal(s, os_), "scale bytes differ"
    assert np.array_equal(q, oq), "e4m3 codes differ"


@pytest.mark.parametrize("idx,dtype", [(1, torch.float32), (4, torch.bfloat16)], ids=["contig_4x1024_f32", "contig_8x4096_bf16"])
def test_device_quant_workload_activations(idx, dtype):
    """The A operand of two benchmark workloads: every scale byte, and the codes
    of sampled rows (the oracle works row by row, so a sample is exact)."""
    w = wl.workload(idx)
    x = wl.draw(w)["a"]
    print(f"[quant] workload {w.name} A {x.shape} {dtype}", flush=True)
    q, s, xw = _device_quant(x, dtype)
    rows = np.sort(np.random.default_rng(7).choice(x.shape[0], size=384, replace=False))
    oq, os_ = o.quantize_act_1x128(xw[rows])
    assert np.array_equal(s[:, rows], os_)
    assert np.array_equal(q[rows], oq)
    # every scale byte: amax per block against the ceil rule, through the oracle's exponent
    t = o.e8m0_ceil_exponent(np.abs(xw.reshape(xw.shape[0], -1, 128)).max(axis=2))
    assert np.array_equal(s, (t + 127).astype(np.uint8).T)


def test_device_quant_boundaries():
    """Blocks built at the rounding boundaries: amax exactly 448 * 2^t and one
    ulp above, E4M3 midpoints (ties to even), values that land in the E4M3
    subnormal range, zeros, negative zero and an all-zero block."""
    blocks = []
    rng = np.random.default_rng(3)
    for t in (-20, -1, 0, 3, 40):
        b = rng.uniform(-1.0, 1.0, 128).astype(np.float32) * np.float32(448.0 * 2.0 ** t)
        b[5] = np.float32(448.0 * 2.0 ** t)
        blocks.append(b)
        b2 = b.copy()
        b2[5] = np.nextafter(np.float32(448.0 * 2.0 ** t), np.float32(np.inf))
        blocks.append(b2)
    codes = np.arange(0, 127, dtype=np.uint8)
    vals = o.decode_e4m3(codes)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)    # every positive midpoint (exact in f32)
    b = np.zeros(128, np.float32)
    b[: mids.size] = mids[:128]
    b[-1] = 448.0                                               # scale 2^0 for this block
    blocks.append(b)
    b = -b
    blocks.append(b)
    b = np.zeros(128, np.float32)
    b[0], b[1], b[2] = 448.0, 2.0 ** -10, 3 * 2.0 ** -10        # ties around the smallest subnormal
    b[3], b[4] = -0.0, 2.0 ** -9 * 1.5
    blocks.append(b)
    blocks.append(np.zeros(128, np.float32))
    x = np.stack(blocks).reshape(1, -1)
    x = np.concatenate([x, x[:, ::-1]], axis=0).copy()          # two rows, blocks in both orders
    q, s, xw = _device_quant(x, torch.float32)
    oq, os_ = o.quantize_act_1x128(xw)
    assert np.array_equal(s, os_)
    assert np.array_equal(q, oq)


def test_device_quant_nonfinite_and_tiny_blocks():
    x = _draw((4, 512), seed=11)
    x[1, 130] = np.nan            # row 1, block 1
    x[2, 300] = np.inf            # row 2, block 2
    x[3, 384:512] = np.float32(1e-37)     # row 3, block 3: t would be < -127
    x[3, 400] = np.float32(-3e-37)
    q, s, xw = _device_quant(x, torch.float32)
    assert s[1, 1] == 255 and np.all(q[1, 128:256] == 0x7F)
    assert s[2, 2] == 255 and np.all(q[2, 256:384] == 0x7F)
    assert s[3, 3] == 0
    assert np.array_equal(q[3, 384:512], o.encode_e4m3_rne(xw[3, 384:512].astype(np.float64) * 2.0 ** 127))
    # every other block matches the oracle
    clean = xw.copy()
    clean[1, 128:256] = 0.0
    clean[2, 256:384] = 0.0
    clean[3, 384:512] = 0.0
    oq, os_ = o.quantize_act_1x128(clean)
    keep = np.ones_like(s, dtype=bool)
    keep[1, 1] = keep[2, 2] = keep[3, 3] = False
    assert np.array_equal(s[keep], os_[keep])
    qb = q.reshape(4, 4, 128)
    oqb = oq.reshape(4, 4, 128)
    assert np.array_equal(qb.transpose(1, 0, 2)[keep], oqb.transpose(1, 0, 2)[keep])


def test_device_quant_matches_host_quantizer():
    """On the small contiguous workload (padding rows of zeros included) the
    device quantizer's bytes equal the host quantizer's, so either can feed
    the GEMM."""
    w = wl.workload(0)
    x = wl.draw(w)
    qa_h, sa_h = gfg.fp8_quantize_act_1x128(x["a"])
    xa = torch.from_numpy(x["a"]).to(DEV)
    qa_d, sa_d = gfg.fp8_quantize_act_1x128_device(xa)
    torch.cuda.synchronize(DEV)
    assert np.array_equal(qa_d.cpu().numpy(), qa_h)
    assert np.array_equal(sa_d.cpu().numpy(), sa_h)


def test_device_quant_repeatable_and_stream():
    x = torch.from_numpy(_draw((300, 1024), seed=5)).to(DEV)
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        q1, s1 = gfg.fp8_quantize_act_1x128_device(x, stream=s)
    s.synchronize()
    q2, s2 = gfg.fp8_quantize_act_1x128_device(x)
    torch.cuda.synchronize(DEV)
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
