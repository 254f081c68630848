"""moe_q4_decode_noalloc: the one-token decode with the library's fixed
per-GPU scratch array, against moe_q4_decode with a caller workspace.

Both run the same pinned W4A8 program, so y must agree bit for bit.  Two
calls in a row on one GPU, the second on a smaller layer, check that the
shared array carries nothing from one call into the next.
"""
import sys

import numpy as np
import pytest
import torch

import moe_synth
import oracle
import bit_quantized_moe_q4_amd as mq
from layers import both_layers

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _one(cfg, step):
    ol, gl = both_layers(cfg)
    x = torch.from_numpy(moe_synth.tokens(cfg, step=step, T=1)[0]).cuda()
    y_ref = mq.moe_q4_decode(gl, x)
    y = torch.full((cfg.H,), float("nan"), dtype=torch.float32, device="cuda")
    mq.moe_q4_decode_noalloc(gl, x, y)
    torch.cuda.synchronize()
    return ol, gl, x, y, y_ref


def test_noalloc_matches_decode_twice_then_smaller():
    assert torch.cuda.is_available()
    big = moe_synth.CONFIGS["decode"]
    small = moe_synth.CONFIGS["tiny"].with_(name="noalloc_small", H=256, E=8, I=128, k=2, shared=True)
    say("noalloc: decode layer", big.H, big.E, big.I, big.k)
    ol, gl, x, y, y_ref = _one(big, 7)
    assert torch.equal(y, y_ref)
    yo = oracle.decode(ol, x.cpu().numpy())
    assert np.array_equal(y.cpu().numpy(), yo)
    # second call in a row on the same GPU, smaller layer and input
    say("noalloc: small layer", small.H, small.E, small.I, small.k)
    ol2, gl2, x2, y2, y2_ref = _one(small, 11)
    assert torch.equal(y2, y2_ref)
    assert np.array_equal(y2.cpu().numpy(), oracle.decode(ol2, x2.cpu().numpy()))
    # and the big layer again, after the small one
    y3 = torch.empty_like(y)
    mq.moe_q4_decode_noalloc(gl, x, y3)
    torch.cuda.synchronize()
    assert torch.equal(y3, y_ref)


def test_noalloc_rejects_a_layer_beyond_the_array():
    cfg = moe_synth.CONFIGS["tiny"].with_(name="noalloc_big", H=8192, E=1024, I=64, k=2, shared=False)
    gl = mq.MoELayer(torch.zeros((cfg.H, cfg.E), device="cuda"),
                     torch.zeros((cfg.E, cfg.I, cfg.H // 32 * 18), dtype=torch.uint8, device="cuda"),
                     torch.zeros((cfg.E, cfg.I, cfg.H // 32 * 18), dtype=torch.uint8, device="cuda"),
                     torch.zeros((cfg.E, cfg.H, cfg.I // 32 * 18), dtype=torch.uint8, device="cuda"),
                     cfg.k, tiles=False)
    assert mq.moe_q4_decode_workspace_bytes(gl) > (1 << 20)
    x = torch.zeros(cfg.H, device="cuda")
    y = torch.zeros(cfg.H, device="cuda")
    with pytest.raises(RuntimeError, match="fixed array"):
        mq.moe_q4_decode_noalloc(gl, x, y)
