"""Pins of the oracle's bf16 prefill program (CPU only).

The program (orc_prefill_bf16) states the rounding points of the grouped
GEMM: weights (q - 8) * d rounded once to bf16, h = bf16(silu(g) * u), a
routed expert's output rounded to bf16, the shared expert's to float32, and
the float32 combine y = ((o_shared + w_0 o_0) + w_1 o_1) + ...  It is pinned
here by
- its bf16 rounding against torch's float32 -> bfloat16 conversion (ties to
  even, overflow, subnormals, zeros, infinities) on every kind of bit
  pattern;
- closed forms of special layers where each rounding point can be evaluated
  by hand: weights on the Q4 grid (exact in bf16), a down matrix 0.875 * I
  (so o = bf16(0.875 h) exactly), integer-valued tokens (exact sums), a
  one-hot token (one product per output), chosen routing weights;
- its distance from the binary64 reference (rounding points present, and
  bf16-sized).
"""
import numpy as np
import torch

import moe_synth
import oracle
from test_oracle_formats import _grid_weights


def _torch_bf16(a):
    """torch's float32 -> bfloat16 conversion, widened back to float32."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    # ties in both parities, values just off the ties, overflow, subnormals
    base = rng.integers(0, 2 ** 16, size=20000, dtype=np.uint64).astype(np.uint32) << 16
    special = np.concatenate([
        base | 0x8000, base | 0x7fff, base | 0x8001, base | 0xffff,
        np.array([0x7f7fffff, 0x7f7f8000, 0x7f7f7fff, 0xff7fffff, 0x00000001, 0x00008000,
                  0x00018000, 0x80008000, 0x007fffff, 0x00000000, 0x80000000, 0x7f800000,
                  0xff800000, 0x3f808000, 0x3f818000], dtype=np.uint32),
    ]).astype(np.uint32)
    u = np.concatenate([bits, special])
    x = u.view(np.float32)
    nan = np.isnan(x)
    got = oracle.bf16_round(x)
    want = _torch_bf16(x)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    assert np.all(np.isnan(got[nan]))
    # the result is always a bfloat16 (low 16 bits zero)
    assert np.all(got[~nan].view(np.uint32) & 0xffff == 0)


def _scaled_identity_down(H, I, c=0.875):
    """c * I as Q4_0: each row one entry c = 7 * (c/7), the scale c/7 exact."""
    d = np.zeros((H, I), np.float32)
    d[np.arange(H), np.arange(H) % I] = c
    return d


def _grid_tokens(rng, T, H):
    """bf16-exact tokens: integers in [-16, 16] times 2^-4."""
    return (rng.integers(-16, 17, size=(T, H)) / 16.0).astype(np.float32)


def _layer(gates, ups, downs, s=None, k=1):
    E, I, H = gates.shape
    Wr = np.zeros((H, E), np.float32)
    return oracle.PackedLayer.from_float(Wr, None, gates, ups, downs,
                                         None if s is None else s[0], None if s is None else s[1],
                                         None if s is None else s[2], k=k)


def _expert_closed_form(g, u, x, round_o, c=0.875):
    """o of one expert whose down matrix is c * I, from exact g = G x, u = U x
    (float64 sums that are exact for these operands): h = bf16(f32(silu(g) u)),
    then o = f32(c h), rounded on to bf16 for a routed expert."""
    gg = g.astype(np.float64) @ x.astype(np.float64)
    uu = u.astype(np.float64) @ x.astype(np.float64)
    h = _torch_bf16((gg / (1.0 + np.exp(-gg)) * uu).astype(np.float32)).astype(np.float64)
    o = (c * h).astype(np.float32)
    return _torch_bf16(o) if round_o else o


def test_prefill_bf16_h_and_o_rounding_closed_form():
    rng = np.random.default_rng(11)
    H = I = 32
    g = _grid_weights(rng, I, H, -4, -2)[0][None]
    u = _grid_weights(rng, I, H, -4, -2)[0][None]
    dn = _scaled_identity_down(H, I)[None]
    L = _layer(g, u, dn)
    assert np.array_equal(oracle.q4_dequant(L.down[0], I), dn[0])      # lossless: 0.875 = 7 * 0.125
    T = 6
    x = _grid_tokens(rng, T, H)
    ids = np.zeros((T, 1), np.int32)
    w32 = np.ones((T, 1), np.float32)
    y = oracle.prefill_bf16(L, x, ids, w32)
    want = np.stack([_expert_closed_form(g[0], u[0], x[t], True) for t in range(T)])
    assert np.array_equal(y, want)          # (values: the sign of an exact zero depends on sum order)
    # the rounding points matter on these inputs: without them the values differ
    assert not np.array_equal(want, np.stack([
        (0.875 * (lambda gg, uu: gg / (1 + np.exp(-gg)) * uu)(g[0] @ x[t].astype(np.float64),
                                                             u[0] @ x[t].astype(np.float64))).astype(np.float32)
        for t in range(T)]))


def test_prefill_bf16_weights_rounded_once_closed_form():
    # off-grid weights: (q - 8) * d carries more than bf16's 8 significant
    # bits; a one-hot token makes g and u single dequantised weights
    rng = np.random.default_rng(12)
    H = I = 32
    g = (rng.standard_normal((1, I, H)) * 0.3).astype(np.float32)
    u = (rng.standard_normal((1, I, H)) * 0.3).astype(np.float32)
    dn = _scaled_identity_down(H, I)[None]
    L = _layer(g, u, dn)
    gq = oracle.q4_dequant(L.gate[0], H)
    uq = oracle.q4_dequant(L.up[0], H)
    assert not np.array_equal(_torch_bf16(gq), gq)          # the rounding is not a no-op here
    x = np.eye(H, dtype=np.float32)[[0, 5, 17, 31]]
    T = x.shape[0]
    y = oracle.prefill_bf16(L, x, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32))
    want = np.stack([_expert_closed_form(_torch_bf16(gq), _torch_bf16(uq), x[t], True) for t in range(T)])
    assert np.array_equal(y, want)


def test_prefill_bf16_combine_order_closed_form():
    rng = np.random.default_rng(13)
    H = I = 32
    E, k = 3, 2
    gs = np.stack([_grid_weights(rng, I, H, -4, -2)[0] for _ in range(E)])
    us = np.stack([_grid_weights(rng, I, H, -4, -2)[0] for _ in range(E)])
    dn = np.stack([_scaled_identity_down(H, I)] * E)
    sg, su = _grid_weights(rng, I, H, -4, -2)[0], _grid_weights(rng, I, H, -4, -2)[0]
    L = _layer(gs, us, dn, s=(sg, su, _scaled_identity_down(H, I)), k=k)
    T = 5
    x = _grid_tokens(rng, T, H)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    w32 = rng.uniform(0.05, 0.95, size=(T, k)).astype(np.float32)
    y = oracle.prefill_bf16(L, x, ids, w32)
    for t in range(T):
        acc = _expert_closed_form(sg, su, x[t], False)            # shared: float32, not bf16
        for s in range(k):
            o = _expert_closed_form(gs[ids[t, s]], us[ids[t, s]], x[t], True)
            acc = (acc + (w32[t, s] * o).astype(np.float32)).astype(np.float32)
        assert np.array_equal(y[t], acc), t


def test_prefill_bf16_against_binary64_reference():
    # the program sits a bf16-sized distance from the exact layer: rounding
    # points present (far above binary32 noise) and no larger than bf16's
    cfg = moe_synth.CONFIGS["tiny"].with_(name="bf16prog", H=256, E=8, I=128, k=2, shared=True)
    W = moe_synth.expert_weights(cfg, 0, threads=4)
    L = oracle.PackedLayer.from_float(moe_synth.router(cfg, 0), moe_synth.router_bias(cfg, 0), W["gate"],
                                      W["up"], W["down"], W["s_gate"], W["s_up"], W["s_down"], k=cfg.k,
                                      threads=4)
    bits = moe_synth.to_bf16_bits(moe_synth.tokens(cfg, T=24))
    x = moe_synth.bf16_bits_to_f32(bits)
    r = oracle.route(L, x)
    y = oracle.prefill_bf16(L, x, r["ids"], r["w32"]).astype(np.float64)
    ref = oracle.prefill_ref(L, x, r["ids"], r["w64"])
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert 1e-4 < rel < 1e-2, rel
