"""GPU parity of the stacked decode step (moe_q4_decode_stack).

The stack runs each layer's decode with the RMSNorm between layers taken
inside the next layer's first kernel.  Bars: y bit-identical to the chain of
moe_q4_decode and moe_q4_rmsnorm calls, and to the oracle's chain of decode
and rmsnorm (both are the same fp32 programs), on a 6-layer stack of small
layers (Q4_0 and Q8_0, each row-major and in tile order), a 4-layer
stack at the decode layer's shape (both Q4_0 layouts) and a 45-layer stack
(two stacked launches).  Layers in tile order run as one stacked launch
(every layer in one kernel, y handed from layer to layer by tagged words);
its bounded waits are forced to give up once to check their reporting.
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

EPS = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _chain(gls, x):
    xd = x
    for L in gls:
        y = mq.moe_q4_decode(L, xd)
        xd, _ = mq.moe_q4_rmsnorm(y[None], EPS, f32=True)
        xd = xd[0]
    return y


def _oracle_chain(ols, x):
    xo = x
    for L in ols:
        y = oracle.decode(L, xo)
        xo = oracle.rmsnorm(y[None], EPS)[0]
    return y


@pytest.mark.parametrize("wfmt,tiles", [("q4", False), ("q4", True), ("q8", False), ("q8", True)],
                         ids=["q4-rowmajor", "q4-tiled", "q8-rowmajor", "q8-tiled"])
def test_stack_small_layers(wfmt, tiles):
    cfg = moe_synth.CONFIGS["tiny"].with_(name="stack_small", H=256, E=8, I=128, k=2, shared=True)
    pairs = [both_layers(cfg, layer=l, tiles=tiles, wfmt=wfmt) for l in range(6)]
    ols, gls = [p[0] for p in pairs], [p[1] for p in pairs]
    stack = mq.LayerStack(gls)
    for step in range(3):
        x = moe_synth.tokens(cfg, step=600 + step, T=1)[0]
        xd = torch.from_numpy(x).cuda()
        ys = mq.moe_q4_decode_stack(stack, xd, EPS).cpu().numpy()
        yc = _chain(gls, xd).cpu().numpy()
        assert np.array_equal(ys.view(np.uint32), yc.view(np.uint32)), step
        yo = _oracle_chain(ols, x)
        err = np.max(np.abs(ys.astype(np.float64) - yo)) / np.max(np.abs(yo))
        assert err <= 1e-5, (step, err)


@pytest.mark.parametrize("tiles", [False, True], ids=["rowmajor", "tiled"])
def test_stack_decode_layers(tiles):
    cfg = moe_synth.CONFIGS["decode"]
    say("building 4 decode-size layers")
    from bit_quantized_moe_q4_amd.synth_layer import device_layer
    gls = [device_layer(cfg, layer=l, tiles=tiles) for l in range(4)]
    stack = mq.LayerStack(gls)
    ws = mq.stack_workspace(stack)
    for step in range(3):
        xd = torch.from_numpy(moe_synth.tokens(cfg, step=700 + step, T=1)[0]).cuda()
        ys = mq.moe_q4_decode_stack(stack, xd, EPS, ws=ws).cpu().numpy()
        yc = _chain(gls, xd).cpu().numpy()
        assert np.array_equal(ys.view(np.uint32), yc.view(np.uint32)), step


def test_stack_longer_than_one_launch():
    # 45 small layers: one launch runs at most 40 layers, so the second launch
    # takes the first one's y through the RMSNorm, as every later layer does
    cfg = moe_synth.CONFIGS["tiny"].with_(name="stack_long", H=256, E=8, I=128, k=2, shared=True)
    pairs = [both_layers(cfg, layer=l % 7, tiles=True) for l in range(45)]
    gls = [p[1] for p in pairs]
    stack = mq.LayerStack(gls)
    ws = mq.stack_workspace(stack)
    for step in range(2):
        xd = torch.from_numpy(moe_synth.tokens(cfg, step=800 + step, T=1)[0]).cuda()
        ys = mq.moe_q4_decode_stack(stack, xd, EPS, ws=ws).cpu().numpy()
        yc = _chain(gls, xd).cpu().numpy()
        assert np.array_equal(ys.view(np.uint32), yc.view(np.uint32)), step


def test_stack_wait_failure_is_reported():
    """The stacked launch's bounded waits, forced to give up (every wait looks
    for a tag no word carries, 16 polls): the launch ends, the failures are
    counted, and the next normal call on the same workspace is exact again."""
    cfg = moe_synth.CONFIGS["tiny"].with_(name="stack_fail", H=256, E=8, I=128, k=2, shared=True)
    gls = [both_layers(cfg, layer=l, tiles=True)[1] for l in range(3)]
    stack = mq.LayerStack(gls)
    ws = mq.stack_workspace(stack)
    xd = torch.from_numpy(moe_synth.tokens(cfg, step=900, T=1)[0]).cuda()
    y0 = mq.moe_q4_decode_stack(stack, xd, EPS, ws=ws)
    assert mq.moe_q4_decode_status(gls[0], ws) == 0
    lib = mq._lib.lib()
    try:
        lib.moe_q4_test_decode_wait_fail(1)
        mq.moe_q4_decode_stack(stack, xd, EPS, ws=ws)
        torch.cuda.synchronize()
    finally:
        lib.moe_q4_test_decode_wait_fail(0)
    failed = mq.moe_q4_decode_status(gls[0], ws)
    say("forced stack give-ups:", failed)
    assert failed > 0
    assert mq.moe_q4_decode_status(gls[0], ws) == 0
    y1 = mq.moe_q4_decode_stack(stack, xd, EPS, ws=ws)
    assert torch.equal(y0, y1)
    assert torch.equal(y1, _chain(gls, xd))


def test_stack_of_one_is_decode():
    cfg = moe_synth.CONFIGS["tiny"].with_(name="stack_one", H=256, E=8, I=128, k=2, shared=False)
    ol, gl = both_layers(cfg, tiles=False)
    x = torch.from_numpy(moe_synth.tokens(cfg, step=5, T=1)[0]).cuda()
    ys = mq.moe_q4_decode_stack(mq.LayerStack([gl]), x, EPS)
    assert torch.equal(ys, mq.moe_q4_decode(gl, x))
