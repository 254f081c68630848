"""The matrix-core rate probe (moe_q4_probe_mfma): each MFMA shape runs,
leaves finite checksums, reports the operation count of its launch, and the
measured rate lies between a tenth of the published dense peak and the peak
itself (a rate above the peak would mean a wrong count)."""
import sys

import pytest
import torch

import bit_quantized_moe_q4_amd as mq

pytestmark = pytest.mark.gpu

PEAK = {mq.PROBE_BF16: 2500.0, mq.PROBE_I8: 5000.0, mq.PROBE_F32_K1: 157.3}   # TFLOP/s, TOPS
OPS_PER_MFMA = {mq.PROBE_BF16: 32 * 32 * 16 * 2, mq.PROBE_I8: 32 * 32 * 32 * 2, mq.PROBE_F32_K1: 2 * 32 * 32 * 2}
CHAINS = {mq.PROBE_BF16: 8, mq.PROBE_I8: 8, mq.PROBE_F32_K1: 4}


@pytest.mark.parametrize("kind", [mq.PROBE_BF16, mq.PROBE_I8, mq.PROBE_F32_K1])
def test_probe_mfma(kind):
    assert torch.cuda.is_available()
    blocks, iters = 512, 4000
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    ops = mq.moe_q4_probe_mfma(kind, blocks, iters, out)
    assert ops == blocks * 4 * CHAINS[kind] * iters * OPS_PER_MFMA[kind]
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    mq.moe_q4_probe_mfma(kind, blocks, iters, out)
    e1.record()
    e1.synchronize()
    rate = ops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print("probe kind %d: %.1f (peak %.1f)" % (kind, rate, PEAK[kind]), flush=True)
    sys.stdout.flush()
    assert 0.1 * PEAK[kind] < rate <= 1.05 * PEAK[kind]
