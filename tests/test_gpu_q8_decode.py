"""GPU parity of the Q8_0 weight path (8-bit weights, W8A8 decode).

Bars: q8w_pack bytes bit-exact against the oracle's packing (and its
hand-worked blocks); decode with Q8_0 layers bit-exact in every traced value
(logits, ids, weights, q8(x), q8(h)) and y within max|dy|/max|y_ref| <= 1e-5
(0 expected) against the oracle's W8A8 program; the batched decode on Q8_0
layers bit-identical to one-token decode; q8w_tile bytes against the tile
order's byte permutation, and decode over the tile-order copies (the default
for H, I multiples of 64) bit-identical to the row-major kernels.  Shapes:
the full decode layer, small layers on the halfword row program, H = 16384,
I = 8192, ragged and minimal tiled shapes.
"""
import sys

import numpy as np
import pytest
import torch

import moe_synth
import oracle
import bit_quantized_moe_q4_amd as mq
from conftest import read_golden
from layers import both_layers

pytestmark = pytest.mark.gpu

DECODE_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("rows,K", [(1, 32), (7, 96), (300, 256), (513, 2048), (64, 16384)])
def test_q8w_pack_bytes(rows, K):
    rng = np.random.default_rng(rows * 7 + K)
    w = (rng.standard_normal((rows, K)) * rng.choice([1e-3, 0.02, 3.0], size=(rows, 1))).astype(np.float32)
    w[0, :32] = 0.0                                   # an all-zero block
    got = mq.q8w_pack(torch.from_numpy(w).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.q8w_pack(w))


def test_q8w_pack_golden_blocks():
    g = read_golden("q8w_blocks.txt")
    for tag in "ABCDE":
        if tag + "_w_dec" in g:
            w = np.array([float(u) for u in g[tag + "_w_dec"]], dtype=np.float32)
        else:
            unit = 2.0 ** int(g[tag + "_unit_log2"][0])
            w = np.array([float(u) * unit for u in g[tag + "_w_units"]], dtype=np.float32)
        exp = bytes(int(b, 16) for b in g[tag + "_bytes"])
        got = mq.q8w_pack(torch.from_numpy(w.reshape(1, 32)).cuda()).cpu().numpy().tobytes()
        assert got == exp, tag


def _decode_steps(ol, gl, cfg, steps):
    ws = mq.decode_workspace(gl)
    worst = 0.0
    for step in steps:
        x = moe_synth.tokens(cfg, step=step, T=1)[0]
        y, tr = mq.moe_q4_decode(gl, torch.from_numpy(x).cuda(), ws=ws, trace=True)
        yo, to = oracle.decode(ol, x, trace=True)
        for key in ("logits", "w", "dx", "dh"):
            assert np.array_equal(tr[key].cpu().numpy().view(np.uint32), to[key].view(np.uint32)), key
        for key in ("ids", "qx", "qh"):
            assert np.array_equal(tr[key].cpu().numpy(), to[key]), key
        err = np.max(np.abs(y.cpu().numpy().astype(np.float64) - yo)) / np.max(np.abs(yo))
        worst = max(worst, err)
        assert err <= DECODE_TOL, (step, err)
    return worst


def _q8_tile_reference(packed: np.ndarray, K: int) -> np.ndarray:
    """The tile order of moe_q4.h (q8w_tile) as a byte permutation of
    row-major Q8_0 blocks [rows][K/32][34]."""
    rows = packed.shape[0]
    nb, ns = K // 32, K // 64
    blk = packed.reshape(rows // 32, 32, ns, 2, 34)          # group, row, step, block-of-step, byte
    out = np.empty((rows // 32, ns, 2176), dtype=np.uint8)
    lanes = blk.transpose(0, 2, 3, 1, 4).reshape(rows // 32, ns, 64, 34)   # lane = 32 * g + n
    out[:, :, :2048] = lanes[:, :, :, 2:].reshape(rows // 32, ns, 2048)
    out[:, :, 2048:] = lanes[:, :, :, :2].reshape(rows // 32, ns, 128)
    return out.reshape(rows, nb * 34)


@pytest.mark.parametrize("rows,K", [(32, 64), (96, 128), (512, 2048), (2048, 512)])
def test_q8w_tile_bytes(rows, K):
    rng = np.random.default_rng(rows + 3 * K)
    w = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32)).cuda()
    packed = mq.q8w_pack(w)
    tiled = mq.q8w_tile(packed)
    assert np.array_equal(tiled.cpu().numpy(), _q8_tile_reference(packed.cpu().numpy(), K))
    # spot check: row 37 (group 1, n = 5), block 3 (step 1, g = 1) -> lane 37 of piece (1, 1)
    if rows >= 64 and K >= 256:
        pk, tl = packed.cpu().numpy(), tiled.cpu().numpy().reshape(-1)
        piece = 32 * (K // 32 * 34) + 2176
        blk = pk[37, 3 * 34:4 * 34]
        assert bytes(tl[piece + 32 * 37: piece + 32 * 38]) == bytes(blk[2:])
        assert bytes(tl[piece + 2048 + 2 * 37: piece + 2048 + 2 * 38]) == bytes(blk[:2])


@pytest.mark.parametrize("name,H,E,I,k,shared", [
    ("tiny_shared", 256, 8, 128, 2, True),
    ("minimal", 64, 4, 64, 2, True),
    ("ragged_pieces", 192, 16, 128, 4, True),
    ("wide_hidden", 16384, 8, 64, 2, True),
    ("ragged_inter", 256, 8, 192, 3, False),
    ("wide_inter", 128, 8, 2048, 4, True),
])
def test_q8_decode_tiled_matches_rowmajor(name, H, E, I, k, shared):
    # the Q8_0 tile-order decode kernels realise the row-major programs' trees
    say("q8 decode tiled vs row-major", name)
    from bit_quantized_moe_q4_amd.synth_layer import device_layer
    cfg = moe_synth.CONFIGS["tiny"].with_(name=name, H=H, E=E, I=I, k=k, shared=shared, bias="zipf")
    W = moe_synth.expert_weights(cfg, 0, threads=16)
    gt = device_layer(cfg, weights=W, tiles=True, wfmt="q8")
    gr = device_layer(cfg, weights=W, tiles=False, wfmt="q8")
    assert gt.tiles is not None and gr.tiles is None
    for step in range(3):
        x = torch.from_numpy(moe_synth.tokens(cfg, step=step, T=1)[0]).cuda()
        yt, tt = mq.moe_q4_decode(gt, x, trace=True)
        yr, trr = mq.moe_q4_decode(gr, x, trace=True)
        assert np.array_equal(yt.cpu().numpy().view(np.uint32), yr.cpu().numpy().view(np.uint32)), step
        for key in ("ids", "w", "qh", "dh", "logits"):
            assert np.array_equal(tt[key].cpu().numpy(), trr[key].cpu().numpy()), (step, key)


@pytest.mark.parametrize("name,H,E,I,k,shared,bias", [
    ("tiny", 256, 8, 128, 2, False, None),
    ("tiny_shared", 256, 8, 128, 2, True, None),
    ("odd_chunks", 96, 5, 96, 3, True, None),
    ("zipf_bias", 512, 64, 256, 8, True, "zipf"),
    ("wide_hidden", 16384, 8, 64, 2, True, None),
    ("wide_inter", 256, 16, 8192, 8, True, None),
])
def test_q8_decode_small(name, H, E, I, k, shared, bias):
    say("q8 decode", name)
    cfg = moe_synth.CONFIGS["tiny"].with_(name=name, H=H, E=E, I=I, k=k, shared=shared, bias=bias)
    ol, gl = both_layers(cfg, wfmt="q8")
    _decode_steps(ol, gl, cfg, range(4))


@pytest.fixture(scope="module")
def q8_layers():
    cfg = moe_synth.CONFIGS["decode"]
    say("building decode-size Q8_0 layer")
    ol, gl = both_layers(cfg, wfmt="q8")
    return cfg, ol, gl


def test_q8_decode_full_layer(q8_layers):
    cfg, ol, gl = q8_layers
    worst = _decode_steps(ol, gl, cfg, range(3))
    say("q8 decode full layer: max-rel %.2e" % worst)


@pytest.mark.parametrize("M", [1, 8, 32])
def test_q8_decode_batch_matches_single(q8_layers, M):
    cfg, ol, gl = q8_layers
    X = np.stack([moe_synth.tokens(cfg, step=4000 + 50 * M + t, T=1)[0] for t in range(M)])
    xd = torch.from_numpy(X).cuda()
    yb = mq.moe_q4_decode_batch(gl, xd).cpu().numpy()
    ws = mq.decode_workspace(gl)
    for t in range(M):
        y1 = mq.moe_q4_decode(gl, xd[t].contiguous(), ws=ws).cpu().numpy()
        assert np.array_equal(yb[t].view(np.uint32), y1.view(np.uint32)), t
    yo = oracle.decode(ol, X[0])
    assert np.max(np.abs(yb[0].astype(np.float64) - yo)) / np.max(np.abs(yo)) <= DECODE_TOL


def test_q8_layer_refuses_prefill(q8_layers):
    cfg, ol, gl = q8_layers
    xb = torch.zeros((4, cfg.H), dtype=torch.bfloat16, device="cuda")
    r = mq.moe_q4_route(gl, xb)
    with pytest.raises(RuntimeError, match="Q4_0"):
        mq.moe_q4_prefill(gl, xb, r)
