"""GPU parity of the batched decode (moe_q4_decode_batch, up to 32 tokens;
batches of 1 or 2 tokens run the one-token program token by token).

Each token of a batch follows the one-token decode program, so the bar is
bit-exactness twice over: every row of y, and the routing ids and weights,
equal those of moe_q4_decode of that token alone, and sampled tokens equal
the oracle's decode (max|dy| / max|y_ref| <= 1e-5; 0 is expected).  Shapes:
the full decode layer at several batch sizes, and small layers that take the
halfword-load row program, the largest expert count and top-k, a shared
expert or none, a router bias, and all-tied logits.
"""
import sys

import numpy as np
import pytest
import torch

import moe_synth
import oracle
import bit_quantized_moe_q4_amd as mq
from layers import both_layers
from bit_quantized_moe_q4_amd.synth_layer import device_layer

pytestmark = pytest.mark.gpu

DECODE_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _batch_tokens(cfg, M, step0):
    return np.stack([moe_synth.tokens(cfg, step=step0 + t, T=1)[0] for t in range(M)])


def _check_against_single(gl, X):
    """y, ids, w of the batch call vs one moe_q4_decode per token (bit for bit)."""
    xd = torch.from_numpy(X).cuda()
    yb, ids, w = mq.moe_q4_decode_batch(gl, xd, routing=True)
    ws = mq.decode_workspace(gl)
    for t in range(X.shape[0]):
        y1, tr = mq.moe_q4_decode(gl, xd[t].contiguous(), ws=ws, trace=True)
        assert np.array_equal(yb[t].cpu().numpy().view(np.uint32), y1.cpu().numpy().view(np.uint32)), t
        assert np.array_equal(ids[t].cpu().numpy(), tr["ids"].cpu().numpy()), t
        assert np.array_equal(w[t].cpu().numpy().view(np.uint32), tr["w"].cpu().numpy().view(np.uint32)), t
    return yb.cpu().numpy()


def _check_against_oracle(ol, X, Y, sample):
    worst = 0.0
    for t in sample:
        yo = oracle.decode(ol, X[t])
        err = np.max(np.abs(Y[t].astype(np.float64) - yo)) / np.max(np.abs(yo))
        worst = max(worst, err)
        assert err <= DECODE_TOL, (t, err)
    return worst


@pytest.fixture(scope="module")
def decode_layers():
    cfg = moe_synth.CONFIGS["decode"]
    say("building decode-size layer")
    ol, gl = both_layers(cfg, tiles=False)
    return cfg, ol, gl


@pytest.fixture(scope="module")
def decode_layers_tiled(decode_layers):
    # the same packed matrices with their tile-order copies: the batched
    # kernels then read the tile order
    cfg, ol, gl = decode_layers
    return cfg, ol, mq.MoELayer(gl.w_router, gl.gate, gl.up, gl.down, gl.top_k, gl.router_bias,
                                gl.s_gate, gl.s_up, gl.s_down, tiles=True)


@pytest.mark.parametrize("M", [1, 2, 5, 8, 17, 32])
@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
def test_decode_batch_full_layer(decode_layers, decode_layers_tiled, M, layout):
    cfg, ol, gl = decode_layers_tiled if layout == "tiled" else decode_layers
    if layout == "tiled":
        assert gl.tiles is not None
    X = _batch_tokens(cfg, M, 2000 + 40 * M)
    Y = _check_against_single(gl, X)
    worst = _check_against_oracle(ol, X, Y, sorted({0, M // 2, M - 1}))
    say("decode batch M=%d: bit-identical to single-token decode; oracle max-rel %.2e" % (M, worst))


def test_decode_batch_repeated_token(decode_layers):
    # 32 copies of one token: one expert list holds every token
    cfg, ol, gl = decode_layers
    x = moe_synth.tokens(cfg, step=77, T=1)[0]
    X = np.repeat(x[None], 32, axis=0)
    Y = _check_against_single(gl, X)
    assert np.array_equal(Y, np.repeat(Y[:1], 32, axis=0))
    _check_against_oracle(ol, X, Y, [0])


@pytest.mark.parametrize("name,H,E,I,k,shared,bias,M", [
    ("tiny", 256, 8, 128, 2, False, None, 7),
    ("tiny_shared", 256, 8, 128, 2, True, None, 32),
    # K = 96: 3 blocks per row, the halfword-load row program
    ("odd_chunks", 96, 5, 96, 3, True, None, 9),
    ("zipf_bias", 512, 64, 256, 8, True, "zipf", 24),
    # the largest expert count and top-k the library accepts
    ("many_experts", 256, 1024, 64, 32, True, "zipf", 32),
    # every expert chosen by every token (k = E)
    ("k_equals_E", 256, 16, 128, 16, True, None, 32),
    # H = 16384: x codes staged a few tokens at a time; 16 lanes per row
    ("wide_hidden", 16384, 8, 64, 2, True, None, 32),
    # I = 8192: q8(h) staged a few pairs at a time; 16 lanes per down row
    ("wide_inter", 256, 16, 8192, 8, True, None, 32),
    # H = I = 64: one tile piece per row (two blocks per lane span)
    ("smallest_tiled", 64, 4, 64, 2, True, None, 5),
    # H = 192, I = 320: 6 and 10 blocks per row, lane spans past the row
    ("ragged_tiled", 192, 6, 320, 3, True, None, 11),
])
@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
def test_decode_batch_small(name, H, E, I, k, shared, bias, M, layout):
    say("decode batch", name, "M=%d" % M, layout)
    cfg = moe_synth.CONFIGS["tiny"].with_(name=name, H=H, E=E, I=I, k=k, shared=shared, bias=bias)
    ol, gl = both_layers(cfg, tiles=(layout == "tiled"))
    assert (gl.tiles is not None) == (layout == "tiled" and H % 64 == 0 and I % 64 == 0)
    X = _batch_tokens(cfg, M, 500)
    Y = _check_against_single(gl, X)
    _check_against_oracle(ol, X, Y, range(min(M, 4)))


def test_decode_batch_tied_logits():
    # W_r = 0: every logit is +0, so the top-k is experts 0..k-1 for every token
    cfg = moe_synth.CONFIGS["tiny"].with_(name="tied", H=256, E=16, I=128, k=4, shared=True)
    W = moe_synth.expert_weights(cfg)
    gl = device_layer(cfg, weights=W, tiles=False)
    gl0 = mq.MoELayer(torch.zeros_like(gl.w_router), gl.gate, gl.up, gl.down, gl.top_k, None,
                      gl.s_gate, gl.s_up, gl.s_down, tiles=False)
    X = _batch_tokens(cfg, 12, 900)
    _check_against_single(gl0, X)
    _, ids, _ = mq.moe_q4_decode_batch(gl0, torch.from_numpy(X).cuda(), routing=True)
    assert np.array_equal(ids.cpu().numpy(), np.tile(np.arange(4, dtype=np.int32), (12, 1)))


def test_decode_batch_empty_and_workspace(decode_layers):
    cfg, ol, gl = decode_layers
    x0 = torch.empty((0, cfg.H), dtype=torch.float32, device="cuda")
    y0 = mq.moe_q4_decode_batch(gl, x0)
    assert y0.shape == (0, cfg.H)
    assert mq.moe_q4_decode_batch_workspace_bytes(gl, 33) == 0
    # one workspace reused across batch sizes: calls on one stream are ordered
    ws = mq.batch_workspace(gl, 32)
    for M in (32, 3, 32):
        X = _batch_tokens(cfg, M, 3000 + M)
        yb = mq.moe_q4_decode_batch(gl, torch.from_numpy(X).cuda(), ws=ws)
        yr = np.stack([mq.moe_q4_decode(gl, torch.from_numpy(X[t]).cuda()).cpu().numpy() for t in range(M)])
        assert np.array_equal(yb.cpu().numpy(), yr)


def test_decode_batch_one_or_two_tokens_use_the_one_token_program(decode_layers):
    # M <= 2: the one-token program per token, in the one-token workspace;
    # a workspace sized for 32 tokens serves them too
    cfg, ol, gl = decode_layers
    one = mq.decode_workspace(gl).numel()
    assert mq.moe_q4_decode_batch_workspace_bytes(gl, 1) == one
    assert mq.moe_q4_decode_batch_workspace_bytes(gl, 2) == one
    assert mq.moe_q4_decode_batch_workspace_bytes(gl, 3) > one
    big = mq.batch_workspace(gl, 32)
    for M in (1, 2):
        X = _batch_tokens(cfg, M, 5000 + M)
        xd = torch.from_numpy(X).cuda()
        exact = mq.batch_workspace(gl, M)
        for ws in (exact, big):
            yb, ids, w = mq.moe_q4_decode_batch(gl, xd, ws=ws, routing=True)
            for t in range(M):
                y1, tr = mq.moe_q4_decode(gl, xd[t].contiguous(), trace=True)
                assert np.array_equal(yb[t].cpu().numpy().view(np.uint32), y1.cpu().numpy().view(np.uint32))
                assert np.array_equal(ids[t].cpu().numpy(), tr["ids"].cpu().numpy())
                assert np.array_equal(w[t].cpu().numpy().view(np.uint32), tr["w"].cpu().numpy().view(np.uint32))
