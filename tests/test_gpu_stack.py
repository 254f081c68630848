"""The 40-layer stack workload: 40 layers of 256 routed experts + 1 shared
(hidden 2048, intermediate 512, top-8), all resident on the device (18.3 GB
of Q4_0), an 8192-token prefill and then 256 one-token decode steps, with
RMSNorm (unit gain, eps 1e-6) between layers: bf16 into the next prefill
layer, fp32 into the next decode layer.

Parity is teacher-forced at sampled layers and steps: the oracle runs each
checked layer on the GPU's own input to that layer.  Bars: routing of the
sampled tokens bit-exact (ids and fp32 weights), prefill rows
rel-L2 <= 1e-2 against the binary64 reference and <= 2e-4 against the
oracle's bf16 program (orc_prefill_bf16), the RMSNorm glue bit-exact,
decode max|dy|/max|y_ref| <= 1e-5.  Drift over the 40 layers is not bounded
(every checked decode layer is exact, so there is none to report there)."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
import bit_quantized_moe_q4_amd as mq
from bit_quantized_moe_q4_amd.synth_layer import device_layer

pytestmark = pytest.mark.gpu

CHECK_LAYERS = (0, 19, 39)
CHECK_STEPS = (0, 127, 255)
N_TOKENS = 24                 # sampled prefill tokens per checked layer
DECODE_STEP0 = 1000           # decode inputs: token streams disjoint from the prefill batch
EPS = 1e-6


def say(*a):
    print("[stack]", *a, flush=True)


def _bits(t_bf16):
    return t_bf16.view(torch.int16).cpu().numpy().view(np.uint16)


def test_stack_teacher_forced():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cfg = moe_synth.CONFIGS["stack"]
    layers = []
    for l in range(cfg.layers):
        layers.append(device_layer(cfg, layer=l, threads=16))
        if l % 5 == 4:
            say("packed layers 0..%d on the device" % l)
    # one resident copy of the weights: 40 x (257 experts x 3 matrices of
    # Q4_0 + the fp32 router) = 18.27 GB, the tile order only
    assert all(not L.rowmajor for L in layers)
    per = (cfg.E + 1) * 3 * cfg.I * (cfg.H // 32) * 18 + cfg.H * cfg.E * 4
    assert sum(L.resident_bytes() for L in layers) == cfg.layers * per
    say("resident: %.2f GB" % (cfg.layers * per / 1e9))

    # ---------------------------------------------------------------- prefill
    T = cfg.T
    sample = np.sort(np.random.default_rng(7).choice(T, N_TOKENS, replace=False))
    sample_d = torch.from_numpy(sample).cuda()
    x0 = moe_synth.tokens(cfg)
    xb = torch.from_numpy(moe_synth.to_bf16_bits(x0).view(np.int16)).cuda().view(torch.bfloat16)
    rws = torch.empty(mq.moe_q4_route_workspace_bytes(layers[0], T), dtype=torch.uint8, device="cuda")
    pws = torch.empty(mq.moe_q4_prefill_workspace_bytes(layers[0], T), dtype=torch.uint8, device="cuda")
    routing = mq.Routing.empty(T, cfg.k, cfg.E, xb.device)
    y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    saved = {}
    for l, L in enumerate(layers):
        mq.moe_q4_route(L, xb, out=routing, ws=rws)
        mq.moe_q4_prefill(L, xb, routing, y=y, ws=pws)
        _, xn = mq.moe_q4_rmsnorm(y, EPS, f32=False, bf16=True)
        off = routing.expert_offsets.cpu().numpy()
        assert off[0] == 0 and off[-1] == T * cfg.k and np.all(np.diff(off) >= 0), l
        if l in CHECK_LAYERS:
            saved[l] = dict(x=_bits(xb[sample_d]), ids=routing.topk_ids[sample_d].cpu().numpy(),
                            w=routing.topk_w[sample_d].cpu().numpy(), y=y[sample_d].cpu().numpy(),
                            xn=_bits(xn[sample_d]))
        assert torch.isfinite(y).all().item(), l
        xb = xn
    say("prefill through %d layers done" % cfg.layers)

    # ---------------------------------------------------------------- decode
    ws = mq.decode_workspace(layers[0])
    dec = {}
    for s in range(cfg.steps):
        xd = torch.from_numpy(moe_synth.tokens(cfg, step=DECODE_STEP0 + s, T=1)).cuda()
        for l, L in enumerate(layers):
            yd = mq.moe_q4_decode(L, xd[0], ws=ws)
            if s in CHECK_STEPS and l in CHECK_LAYERS:
                dec[(s, l)] = (xd[0].cpu().numpy(), yd.cpu().numpy())
            xd, _ = mq.moe_q4_rmsnorm(yd[None], EPS, f32=True)
        if s % 64 == 63:
            say("decode step %d through %d layers done" % (s, cfg.layers))
    del layers, rws, pws, routing, y, ws, xb
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- oracle
    for l in CHECK_LAYERS:
        W = moe_synth.expert_weights(cfg, l, threads=16)
        ol = oracle.PackedLayer.from_float(moe_synth.router(cfg, l), moe_synth.router_bias(cfg, l),
                                           W["gate"], W["up"], W["down"], W["s_gate"], W["s_up"],
                                           W["s_down"], k=cfg.k, threads=16)
        del W
        sv = saved[l]
        xs = moe_synth.bf16_bits_to_f32(sv["x"])
        rr = oracle.route(ol, xs)
        assert np.array_equal(sv["ids"], rr["ids"]), l
        assert np.array_equal(sv["w"].view(np.uint32), rr["w32"].view(np.uint32)), l
        yref = oracle.prefill_ref(ol, xs, rr["ids"], rr["w64"])
        rel = np.linalg.norm(sv["y"].astype(np.float64) - yref) / np.linalg.norm(yref)
        say("layer %d: prefill rel-L2 %.3e over %d tokens" % (l, rel, N_TOKENS))
        assert rel <= 1e-2, (l, rel)
        # and against the oracle's bf16 program (the kernels' rounding points)
        yp = oracle.prefill_bf16(ol, xs, rr["ids"], rr["w32"], threads=16).astype(np.float64)
        relp = np.linalg.norm(sv["y"].astype(np.float64) - yp) / np.linalg.norm(yp)
        say("layer %d: vs the bf16 program rel-L2 %.3e" % (l, relp))
        assert relp <= 2e-4, (l, relp)
        assert np.array_equal(sv["xn"], moe_synth.to_bf16_bits(oracle.rmsnorm(sv["y"], EPS))), l
        for s in CHECK_STEPS:
            xin, yg = dec[(s, l)]
            yo = oracle.decode(ol, xin)
            err = np.max(np.abs(yg.astype(np.float64) - yo)) / np.max(np.abs(yo))
            say("layer %d step %d: decode max-rel %.3e" % (l, s, err))
            assert err <= 1e-5, (l, s, err)
