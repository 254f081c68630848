"""Layers that keep one resident copy of their weights: the tile order only.

MoELayer(tiles=True) releases the row-major matrices when the library covers
the shape without them (moe_q4_check_layer).  Every entry point then reads
the tile order; its results must equal, bit for bit, those of the same
layer holding both copies (the same kernels for prefill and the one-token
decode) and of the row-major batched decode.
"""
import sys

import numpy as np
import pytest
import torch

import moe_synth
import bit_quantized_moe_q4_amd as mq
from layers import tokens
from bit_quantized_moe_q4_amd.synth_layer import device_layer

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.fixture(scope="module")
def three_layouts():
    cfg = moe_synth.CONFIGS["decode"]
    W = moe_synth.expert_weights(cfg, threads=16)
    only = device_layer(cfg, weights=W)
    both = device_layer(cfg, weights=W, rowmajor=True)
    rows = device_layer(cfg, weights=W, tiles=False)
    return cfg, only, both, rows


def test_tile_only_is_the_default_and_holds_one_copy(three_layouts):
    cfg, only, both, rows = three_layouts
    assert not only.rowmajor and only.tiles is not None
    assert both.rowmajor and rows.rowmajor and rows.tiles is None
    per = (cfg.E + 1) * 3 * cfg.I * (cfg.H // 32) * 18 + cfg.H * cfg.E * 4
    assert only.resident_bytes() == per == 229_310_464
    assert both.resident_bytes() == 2 * per - cfg.H * cfg.E * 4
    say("one layer: %.1f MB resident" % (only.resident_bytes() / 1e6))


def test_tile_only_decode_and_batch(three_layouts):
    cfg, only, both, rows = three_layouts
    X = torch.from_numpy(moe_synth.tokens(cfg, step=300, T=9)).cuda()
    ws_o, ws_b = mq.decode_workspace(only), mq.decode_workspace(both)
    for t in range(3):
        yo = mq.moe_q4_decode(only, X[t], ws=ws_o)
        yb = mq.moe_q4_decode(both, X[t], ws=ws_b)
        assert np.array_equal(_bits(yo), _bits(yb)), t
        yn = torch.empty_like(yb)
        mq.moe_q4_decode_noalloc(only, X[t], yn)
        assert np.array_equal(_bits(yn), _bits(yb)), t
    for M in (3, 9):
        y_only = mq.moe_q4_decode_batch(only, X[:M])
        y_rows = mq.moe_q4_decode_batch(rows, X[:M])
        assert np.array_equal(_bits(y_only), _bits(y_rows)), M


def test_tile_only_stack(three_layouts):
    cfg, only, both, rows = three_layouts
    c1 = only.clone()
    assert not c1.rowmajor
    stack = mq.LayerStack([only, c1, only])
    x = torch.from_numpy(moe_synth.tokens(cfg, step=500, T=1)[0]).cuda()
    ys = mq.moe_q4_decode_stack(stack, x, 1e-6)
    ws = mq.decode_workspace(both)
    h = x
    for i in range(3):
        y = mq.moe_q4_decode(both, h, ws=ws)
        if i < 2:
            h, _ = mq.moe_q4_rmsnorm(y[None], 1e-6, f32=True)
            h = h[0]
    assert np.array_equal(_bits(ys), _bits(y))


def test_tile_only_prefill_both_forms(three_layouts):
    cfg, only, both, rows = three_layouts
    pcfg = cfg.with_(T=300)
    x, bits, xw, xd, xbd = tokens(pcfg, T=300, step=4)
    r = mq.moe_q4_route(only, xbd)
    for fn in (mq.moe_q4_prefill, mq.moe_q4_prefill_w4a8):
        yo = fn(only, xbd, r)
        yb = fn(both, xbd, r)
        assert np.array_equal(_bits(yo), _bits(yb)), fn.__name__


def test_uncovered_shape_keeps_its_rows():
    # the tile-order down kernel of the three-launch decode stops at I = 2048:
    # such a layer keeps its row-major matrices, or refuses when asked not to
    cfg = moe_synth.CONFIGS["tiny"].with_(name="wide_i", H=256, E=4, I=4096, k=2, shared=False)
    W = moe_synth.expert_weights(cfg)
    gl = device_layer(cfg, weights=W)
    assert gl.rowmajor and gl.tiles is not None
    with pytest.raises(RuntimeError, match="row-major"):
        device_layer(cfg, weights=W, rowmajor=False)
