"""Pins of the oracle's layer functions (CPU only).

- prefill_ref (binary64) against a dense torch float64 SwiGLU FFN built from
  the weights the packing is lossless for, and from dequantised weights;
- the W4A8 program against integer codes chosen by the test (so every block
  dot is known without the oracle) and against a binary64 evaluation of the
  same quantised operands;
- invariants: zero input, one-hot expert, token and expert relabelling.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from test_oracle_formats import _grid_weights


def _dense_ffn64(x, g, u, d):
    """torch float64 SwiGLU expert: x [n,H]; g,u [I,H]; d [H,I]."""
    x, g, u, d = (torch.as_tensor(np.asarray(a, np.float64)) for a in (x, g, u, d))
    return (torch.nn.functional.silu(x @ g.T) * (x @ u.T)) @ d.T


def _dense_layer64(x, ids, w64, W, shared):
    y = torch.zeros((x.shape[0], x.shape[1]), dtype=torch.float64)
    for t in range(x.shape[0]):
        for s in range(ids.shape[1]):
            e = ids[t, s]
            y[t] += float(w64[t, s]) * _dense_ffn64(x[t:t + 1], W["gate"][e], W["up"][e], W["down"][e])[0]
        if shared:
            y[t] += _dense_ffn64(x[t:t + 1], W["s_gate"], W["s_up"], W["s_down"])[0]
    return y.numpy()


def _grid_layer(rng, H, I, E, shared):
    def g(rows, K):
        return _grid_weights(rng, rows, K, -8, -5)[0]
    W = dict(gate=np.stack([g(I, H) for _ in range(E)]), up=np.stack([g(I, H) for _ in range(E)]),
             down=np.stack([g(H, I) for _ in range(E)]))
    W.update(s_gate=g(I, H) if shared else None, s_up=g(I, H) if shared else None,
             s_down=g(H, I) if shared else None)
    return W


@pytest.mark.parametrize("shared", [False, True])
def test_prefill_ref_vs_dense_float64(shared):
    rng = np.random.default_rng(21)
    H, I, E, k, T = 64, 64, 4, 2, 6
    W = _grid_layer(rng, H, I, E, shared)
    Wr = (rng.standard_normal((H, E)) * 0.1).astype(np.float32)
    L = oracle.PackedLayer.from_float(Wr, None, W["gate"], W["up"], W["down"],
                                      W["s_gate"], W["s_up"], W["s_down"], k=k)
    # packing is lossless on the grid, so the dense fp32 weights are the truth
    assert np.array_equal(oracle.q4_dequant(L.gate, H), W["gate"])
    x = rng.standard_normal((T, H)).astype(np.float32)
    r = oracle.route(L, x)
    y = oracle.prefill_ref(L, x, r["ids"], r["w64"])
    ref = _dense_layer64(x, r["ids"], r["w64"], W, shared)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_prefill_ref_random_weights_and_token_subset():
    cfg = moe_synth.CONFIGS["tiny"]
    W = moe_synth.expert_weights(cfg)
    Wr = moe_synth.router(cfg)
    L = oracle.PackedLayer.from_float(Wr, None, W["gate"], W["up"], W["down"], k=cfg.k)
    x = moe_synth.tokens(cfg)
    r = oracle.route(L, x)
    Wd = dict(gate=oracle.q4_dequant(L.gate, cfg.H), up=oracle.q4_dequant(L.up, cfg.H),
              down=oracle.q4_dequant(L.down, cfg.I))
    ref = _dense_layer64(x, r["ids"], r["w64"], Wd, False)
    y = oracle.prefill_ref(L, x, r["ids"], r["w64"])
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)
    sub = np.array([5, 0, 11])
    ys = oracle.prefill_ref(L, x, r["ids"], r["w64"], tokens=sub)
    assert np.array_equal(ys, y[sub])


def test_prefill_ref_one_hot_expert_is_dense_ffn():
    rng = np.random.default_rng(8)
    H, I = 128, 64
    W = _grid_layer(rng, H, I, 1, True)
    Wr = np.zeros((H, 1), np.float32)
    L = oracle.PackedLayer.from_float(Wr, None, W["gate"], W["up"], W["down"],
                                      W["s_gate"], W["s_up"], W["s_down"], k=1)
    x = rng.standard_normal((4, H)).astype(np.float32)
    r = oracle.route(L, x)
    assert np.all(r["ids"] == 0) and np.all(r["w64"] == 1.0)
    y = oracle.prefill_ref(L, x, r["ids"], r["w64"])
    ref = (_dense_ffn64(x, W["gate"][0], W["up"][0], W["down"][0])
           + _dense_ffn64(x, W["s_gate"], W["s_up"], W["s_down"])).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)


def test_prefill_ref_zero_input_and_relabelling():
    cfg = moe_synth.CONFIGS["tiny"].with_(E=6, k=3)
    W = moe_synth.expert_weights(cfg)
    Wr = moe_synth.router(cfg)
    x = moe_synth.tokens(cfg)
    L = oracle.PackedLayer.from_float(Wr, None, W["gate"], W["up"], W["down"], k=cfg.k)
    r = oracle.route(L, x)
    y = oracle.prefill_ref(L, x, r["ids"], r["w64"])
    z = oracle.prefill_ref(L, np.zeros_like(x), r["ids"], r["w64"])
    assert np.all(z == 0.0)
    # permuting the experts (router columns together with weights) changes nothing
    p = np.array([3, 0, 5, 1, 4, 2])
    L2 = oracle.PackedLayer(Wr[:, p], None, L.gate[p], L.up[p], L.down[p], k=cfg.k)
    r2 = oracle.route(L2, x)
    assert np.array_equal(p[r2["ids"]], r["ids"])
    assert np.allclose(oracle.prefill_ref(L2, x, r2["ids"], r2["w64"]), y, rtol=1e-13, atol=1e-16)
    # permuting tokens permutes outputs
    q = np.random.default_rng(0).permutation(cfg.T)
    r3 = oracle.route(L, x[q])
    assert np.array_equal(oracle.prefill_ref(L, x[q], r3["ids"], r3["w64"]), y[q])


# ---------------------------------------------------------------- W4A8
def _int_activation(rng, K, log2_d=-5):
    """x whose q8 codes are known: x = qa * 2^log2_d with |qa| = 127 in every
    block, so amax/127 = 2^log2_d exactly and x/d = qa exactly."""
    qa = rng.integers(-127, 128, size=K)
    qa[::32] = rng.choice([-127, 127], size=K // 32)
    return (qa * 2.0 ** log2_d).astype(np.float32), qa


@pytest.mark.parametrize("N,K", [(16, 256), (33, 2048), (8, 32), (5, 96)])
def test_w4a8_block_dots_are_integer_dots(N, K):
    rng = np.random.default_rng(N + K)
    w, q, d = _grid_weights(rng, N, K, -10, -4)
    W = oracle.q4_pack(w)
    x, qa = _int_activation(rng, K)
    qx, dx = oracle.q8_quantize(x.reshape(1, K))
    assert np.array_equal(qx[0], qa) and np.all(dx == 2.0 ** -5)
    dots, out = oracle.w4a8_gemv(W, K, qx[0], dx[0])
    prod = ((q - 8) * qa).reshape(N, K // 32, 32)
    assert np.array_equal(dots, prod.sum(axis=2))
    # the pmaddubsw form: sum q*a - 8*sum a (unsigned codes, one correction)
    alt = (q * qa).reshape(N, K // 32, 32).sum(2) - 8 * qa.reshape(K // 32, 32).sum(1)
    assert np.array_equal(dots, alt)
    assert np.abs(dots).max() <= 32512
    # fp32 row program vs the same operands in binary64
    ideal = (d * 2.0 ** -5 * dots).sum(axis=1)
    mag = np.abs(d * 2.0 ** -5 * dots).sum(axis=1)
    assert np.all(np.abs(out.astype(np.float64) - ideal) <= 1e-6 * mag + 1e-30)


def _tiny_decode_layer(shared=True, E=8, k=2, H=256, I=128, bias=None):
    cfg = moe_synth.CONFIGS["tiny"].with_(E=E, k=k, H=H, I=I, shared=shared)
    W = moe_synth.expert_weights(cfg)
    Wr = moe_synth.router(cfg)
    return cfg, oracle.PackedLayer.from_float(Wr, bias, W["gate"], W["up"], W["down"],
                                              W["s_gate"], W["s_up"], W["s_down"], k=k)


@pytest.mark.parametrize("shared", [False, True])
def test_decode_trace_vs_binary64(shared):
    cfg, L = _tiny_decode_layer(shared)
    H, I, k = cfg.H, cfg.I, cfg.k
    x = moe_synth.tokens(cfg, step=3, T=1)[0]
    y, tr = oracle.decode(L, x, trace=True)
    r = oracle.route(L, x[None])
    assert np.array_equal(tr["ids"], r["ids"][0]) and np.array_equal(tr["w"], r["w32"][0])
    qx, dx = oracle.q8_quantize(x[None])
    assert np.array_equal(tr["qx"], qx[0]) and np.array_equal(tr["dx"], dx[0])
    experts = list(tr["ids"]) + (["s"] if shared else [])
    y64 = np.zeros(H)
    for s, e in enumerate(experts):
        G = L.s_gate if e == "s" else L.gate[e]
        Um = L.s_up if e == "s" else L.up[e]
        D = L.s_down if e == "s" else L.down[e]
        Gd, Ud, Dd = (oracle.q4_dequant(M, K).astype(np.float64) for M, K in ((G, H), (Um, H), (D, I)))
        xq = (tr["qx"].astype(np.float64).reshape(-1, 32) * tr["dx"][:, None]).ravel()
        g64, u64 = Gd @ xq, Ud @ xq
        mag = np.abs(Gd) @ np.abs(xq)
        assert np.all(np.abs(tr["gate"][s] - g64) <= 1e-6 * mag + 1e-30)
        assert np.all(np.abs(tr["up"][s] - u64) <= 1e-6 * (np.abs(Ud) @ np.abs(xq)) + 1e-30)
        # q8(h) codes: nearest integers to h/d (h in binary64 from the fp32 g, u)
        h64 = tr["gate"][s] / (1 + np.exp(-tr["gate"][s].astype(np.float64))) * tr["up"][s]
        ratio = h64.reshape(-1, 32) / tr["dh"][s][:, None]
        assert np.all(np.abs(ratio - tr["qh"][s].reshape(-1, 32)) <= 0.5 + 1e-4)
        hq = (tr["qh"][s].astype(np.float64).reshape(-1, 32) * tr["dh"][s][:, None]).ravel()
        o64 = Dd @ hq
        assert np.all(np.abs(tr["o"][s] - o64) <= 1e-6 * (np.abs(Dd) @ np.abs(hq)) + 1e-30)
        y64 += (float(tr["w"][s]) if e != "s" else 1.0) * tr["o"][s].astype(np.float64)
    assert np.max(np.abs(y - y64)) <= 1e-6 * np.max(np.abs(y64))


def test_decode_close_to_float_layer():
    # W4A8 only adds int8 rounding of x and h to the float layer
    cfg, L = _tiny_decode_layer(True)
    errs = []
    for step in range(4):
        x = moe_synth.tokens(cfg, step=step, T=1)
        y = oracle.decode(L, x[0])
        r = oracle.route(L, x)
        ref = oracle.prefill_ref(L, x, r["ids"], r["w64"])[0]
        errs.append(np.linalg.norm(y - ref) / np.linalg.norm(ref))
    assert max(errs) < 3e-2, errs


def test_decode_zero_input_and_scaling():
    cfg, L = _tiny_decode_layer(True)
    y = oracle.decode(L, np.zeros(cfg.H, np.float32))
    assert np.all(y == 0.0)
    x = moe_synth.tokens(cfg, step=1, T=1)[0]
    _, a = oracle.decode(L, x, trace=True)
    _, b = oracle.decode(L, x * np.float32(4.0), trace=True)
    assert np.array_equal(a["qx"], b["qx"]) and np.array_equal(a["ids"], b["ids"])
    assert np.array_equal(a["logits"] * np.float32(4.0), b["logits"])


def test_decode_one_hot_expert():
    # one routed expert (k=1, weight exactly 1) and no shared expert: the layer
    # is a single W4A8 SwiGLU FFN; check y against the trace's own rows
    cfg, L = _tiny_decode_layer(False, E=1, k=1)
    x = moe_synth.tokens(cfg, step=2, T=1)[0]
    y, tr = oracle.decode(L, x, trace=True)
    assert tr["w"][0] == 1.0 and tr["ids"][0] == 0
    assert np.array_equal(y, tr["o"][0])


def test_rmsnorm_vs_binary64():
    rng = np.random.default_rng(9)
    y = (rng.standard_normal((7, 2048)) * rng.uniform(0.01, 100, (7, 1))).astype(np.float32)
    out = oracle.rmsnorm(y, 1e-6).astype(np.float64)
    yd = y.astype(np.float64)
    ref = yd / np.sqrt((yd ** 2).mean(1, keepdims=True) + 1e-6)
    assert np.allclose(out, ref, rtol=2e-6, atol=0)
    c = np.full((1, 64), 3.0, np.float32)
    assert np.allclose(oracle.rmsnorm(c, 0.0), 1.0, rtol=1e-7)


# ---------------------------------------------------------------- Q8_0 weights (W8A8 decode)
@pytest.mark.parametrize("N,K", [(7, 64), (33, 512)])
def test_w8a8_block_dots_are_integer_dots(N, K):
    rng = np.random.default_rng(N * K)
    nb = K // 32
    q = rng.integers(-127, 128, size=(N, nb, 32))
    q[:, :, 0] = 127
    d = 2.0 ** rng.integers(-10, -4, size=(N, nb, 1))
    W = oracle.q8w_pack((q * d).reshape(N, K).astype(np.float32))
    x, qa = _int_activation(rng, K)
    qx, dx = oracle.q8_quantize(x.reshape(1, K))
    dots, out = oracle.w8a8_gemv(W, K, qx[0], dx[0])
    assert np.array_equal(dots, (q * qa.reshape(nb, 32)).sum(axis=2))
    ideal = (d[:, :, 0] * 2.0 ** -5 * dots).sum(axis=1)
    mag = np.abs(d[:, :, 0] * 2.0 ** -5 * dots).sum(axis=1)
    assert np.all(np.abs(out.astype(np.float64) - ideal) <= 1e-6 * mag + 1e-30)


def _tiny_q8_layer(shared=True, E=8, k=2, H=256, I=128):
    cfg = moe_synth.CONFIGS["tiny"].with_(E=E, k=k, H=H, I=I, shared=shared)
    W = moe_synth.expert_weights(cfg)
    Wr = moe_synth.router(cfg)
    return cfg, oracle.PackedLayer.from_float(Wr, None, W["gate"], W["up"], W["down"],
                                              W["s_gate"], W["s_up"], W["s_down"], k=k,
                                              wfmt=oracle.Q8_0), W


@pytest.mark.parametrize("shared", [False, True])
def test_decode_q8w_trace_vs_binary64(shared):
    cfg, L, _ = _tiny_q8_layer(shared)
    H, I = cfg.H, cfg.I
    x = moe_synth.tokens(cfg, step=4, T=1)[0]
    y, tr = oracle.decode(L, x, trace=True)
    experts = list(tr["ids"]) + (["s"] if shared else [])
    xq = (tr["qx"].astype(np.float64).reshape(-1, 32) * tr["dx"][:, None]).ravel()
    y64 = np.zeros(H)
    ybound = np.zeros(H)
    w = list(tr["w"]) + ([1.0] if shared else [])
    for s, e in enumerate(experts):
        G = L.s_gate if e == "s" else L.gate[e]
        Um = L.s_up if e == "s" else L.up[e]
        D = L.s_down if e == "s" else L.down[e]
        Gd, Ud, Dd = (oracle.q8w_dequant(M, K).astype(np.float64) for M, K in ((G, H), (Um, H), (D, I)))
        assert np.all(np.abs(tr["gate"][s] - Gd @ xq) <= 1e-6 * (np.abs(Gd) @ np.abs(xq)) + 1e-30)
        assert np.all(np.abs(tr["up"][s] - Ud @ xq) <= 1e-6 * (np.abs(Ud) @ np.abs(xq)) + 1e-30)
        hq = (tr["qh"][s].astype(np.float64).reshape(-1, 32) * tr["dh"][s][:, None]).ravel()
        o64 = Dd @ hq
        assert np.all(np.abs(tr["o"][s] - o64) <= 1e-6 * (np.abs(Dd) @ np.abs(hq)) + 1e-30)
        y64 += w[s] * o64
        ybound += abs(w[s]) * (np.abs(Dd) @ np.abs(hq))
    assert np.all(np.abs(y - y64) <= 1e-5 * ybound + 1e-30)


def test_decode_q8w_closer_to_float_than_q4():
    # 8-bit weights: the decode output sits closer to the unquantised layer's
    # binary64 FFN than the 4-bit decode does (same int8 activations)
    cfg, L8, W = _tiny_q8_layer(True)
    L4 = oracle.PackedLayer.from_float(L8.w_router, None, W["gate"], W["up"], W["down"],
                                       W["s_gate"], W["s_up"], W["s_down"], k=cfg.k)
    e4, e8 = [], []
    for step in range(4):
        x = moe_synth.tokens(cfg, step=20 + step, T=1)[0]
        r = oracle.route(L8, x[None])
        ref = np.zeros(cfg.H)
        xd = x.astype(np.float64)
        experts = [(W["gate"][e], W["up"][e], W["down"][e], float(wv)) for e, wv in zip(r["ids"][0], r["w64"][0])]
        experts.append((W["s_gate"], W["s_up"], W["s_down"], 1.0))
        for G, U, D, wv in experts:
            g, u = G.astype(np.float64) @ xd, U.astype(np.float64) @ xd
            ref += wv * (D.astype(np.float64) @ (g / (1 + np.exp(-g)) * u))
        e4.append(np.linalg.norm(oracle.decode(L4, x) - ref) / np.linalg.norm(ref))
        e8.append(np.linalg.norm(oracle.decode(L8, x) - ref) / np.linalg.norm(ref))
    assert max(e8) < min(e4), (e8, e4)
