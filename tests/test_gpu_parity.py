"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars (the library's stated contract):
  - bit-exact: Q4 packing bytes, int8 activation codes and scales, router
    logits, top-k ids and weights, expert offsets / perm / inv_perm, every
    per-block int32 W4A8 dot, decode q8(h) codes and scales;
  - decode y: max|y - y_ref| / max|y_ref| <= 1e-5 (the fp32 program is the
    same on both sides, so 0 is expected);
  - prefill y (bf16 MFMA path): ||y - y_ref||_2 / ||y_ref||_2 <= 1e-2 against
    the oracle's binary64 reference; and against the oracle's bf16 program
    (orc_prefill_bf16: weights, h and routed outputs rounded to bf16, the
    float32 combine in slot order) rel-L2 <= 2e-4 over the checked tokens and
    <= 2e-3 per token.  The kernels and the program differ only in the order
    of the fp32 sums and in the exponential; a value that lands within that
    difference of a bf16 rounding boundary moves by one bf16 step (2^-8
    relative), which put the measured distance at 0 .. 1.1e-4 rel-L2 (worst
    token 7e-4).  Leaving out any one rounding point moves it to 6e-4
    (routed outputs) .. 4e-3 (weights), so the rel-L2 bar tells them apart.
Sizes: small shapes that span several tiles with ragged tails, plus the full
workload shapes (decode 2048x128x512 top-8 + shared; prefill 2048 tokens;
skewed 10240 tokens) on sampled tokens.
"""
import sys

import numpy as np
import pytest
import torch

import moe_synth
import oracle
import bit_quantized_moe_q4_amd as mq
from layers import both_layers, tokens
from bit_quantized_moe_q4_amd.synth_layer import device_layer

pytestmark = pytest.mark.gpu

PREFILL_TOL = 1e-2
PROGRAM_TOL = 2e-4
PROGRAM_TOK_TOL = 2e-3
DECODE_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    say("library:", mq.library_path())
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- packing
@pytest.mark.parametrize("rows,K", [(1, 32), (7, 96), (300, 256), (513, 2048), (64, 16384)])
def test_q4_pack_bytes(rows, K):
    say("q4_pack", rows, K)
    rng = np.random.default_rng(rows * 7 + K)
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    w[0, :32] = 0.0                                    # zero block
    if rows > 2:
        w[1, :32] *= 1e-6                             # fp16-subnormal scale
        w[2, :32] = np.round(w[2, :32] * 64) / 64     # many exact halves
    got = mq.q4_pack(torch.from_numpy(w).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.q4_pack(w))


def test_q4_pack_golden_blocks():
    from conftest import read_golden
    g = read_golden("q4_blocks.txt")
    for tag in "ABCD":
        unit = 2.0 ** int(g[tag + "_unit_log2"][0])
        w = np.array([float(u) * unit for u in g[tag + "_w_units"]], dtype=np.float32)
        exp = bytes(int(b, 16) for b in g[tag + "_bytes"])
        got = mq.q4_pack(torch.from_numpy(w.reshape(1, 32)).cuda()).cpu().numpy().tobytes()
        assert got == exp, tag


def _tile_order_reference(packed: np.ndarray, K: int) -> np.ndarray:
    """The tile order of moe_q4.h (q4_tile) as a byte permutation of row-major
    Q4_0 blocks [rows][K/32][18]."""
    rows = packed.shape[0]
    nb, ns = K // 32, K // 64
    blk = packed.reshape(rows // 32, 32, ns, 2, 18)          # group, row, step, block-of-step, byte
    out = np.empty((rows // 32, ns, 1152), dtype=np.uint8)
    lanes = blk.transpose(0, 2, 3, 1, 4).reshape(rows // 32, ns, 64, 18)   # lane = 32 * g + n
    out[:, :, :1024] = lanes[:, :, :, 2:].reshape(rows // 32, ns, 1024)
    out[:, :, 1024:] = lanes[:, :, :, :2].reshape(rows // 32, ns, 128)
    return out.reshape(rows, nb * 18)


@pytest.mark.parametrize("rows,K", [(32, 64), (96, 128), (512, 2048), (2048, 512)])
def test_q4_tile_bytes(rows, K):
    rng = np.random.default_rng(rows + K)
    w = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32)).cuda()
    packed = mq.q4_pack(w)
    tiled = mq.q4_tile(packed)
    ref = _tile_order_reference(packed.cpu().numpy(), K)
    assert np.array_equal(tiled.cpu().numpy(), ref)
    # group G keeps its byte range: the multiset of bytes of each 32-row group is unchanged
    a = np.sort(packed.cpu().numpy().reshape(rows // 32, -1), axis=1)
    b = np.sort(tiled.cpu().numpy().reshape(rows // 32, -1), axis=1)
    assert np.array_equal(a, b)


def test_q4_tile_lane_map_spot_checks():
    # row 37 (group 1, n = 5), block 3 (step 1, g = 1) -> lane 37 of piece (1, 1)
    rows, K = 64, 256
    w = torch.from_numpy(np.random.default_rng(3).standard_normal((rows, K)).astype(np.float32)).cuda()
    packed = mq.q4_pack(w).cpu().numpy()
    tiled = mq.q4_tile(torch.from_numpy(packed).cuda()).cpu().numpy().reshape(-1)
    rb = K // 32 * 18
    piece = 1 * 32 * rb + 1 * 1152
    blk = packed[37, 3 * 18:4 * 18]
    assert bytes(tiled[piece + 16 * 37: piece + 16 * 38]) == bytes(blk[2:])
    assert bytes(tiled[piece + 1024 + 2 * 37: piece + 1024 + 2 * 38]) == bytes(blk[:2])


@pytest.mark.parametrize("rows,K", [(1, 32), (5, 2048), (33, 512)])
def test_q8_quantize(rows, K):
    say("q8", rows, K)
    rng = np.random.default_rng(rows + K)
    x = (rng.standard_normal((rows, K)) * 3).astype(np.float32)
    x[0, :32] = 0.0
    x[-1, 32:64] = np.round(x[-1, 32:64] * 2) / 2
    q, d = mq.q8_quantize(torch.from_numpy(x).cuda())
    qo, do = oracle.q8_quantize(x)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), do.view(np.uint32))


# ---------------------------------------------------------------- W4A8 row
@pytest.mark.parametrize("N,K", [(512, 2048), (2048, 512), (37, 256), (5, 128), (3, 96),
                                 (64, 4096), (9, 16384)])
def test_w4a8_gemv_dots_bit_exact(N, K):
    say("w4a8_gemv", N, K)
    rng = np.random.default_rng(N * 3 + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W = oracle.q4_pack(w)
    x = rng.standard_normal(K).astype(np.float32)
    qa, da = oracle.q8_quantize(x[None])
    dots_o, out_o = oracle.w4a8_gemv(W, K, qa[0], da[0])
    dots, out = mq.moe_q4_w4a8_gemv(torch.from_numpy(W).cuda(), N, K, torch.from_numpy(qa[0]).cuda(),
                                    torch.from_numpy(da[0]).cuda())
    assert np.array_equal(dots.cpu().numpy(), dots_o)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), out_o.view(np.uint32))


# ---------------------------------------------------------------- routing
def _route_case(cfg, T, step=0, tie_cols=False):
    ol, gl = both_layers(cfg)
    if tie_cols:
        # duplicate router columns: exactly equal logits, lower index must win
        wr = ol.w_router.copy()
        wr[:, 1] = wr[:, 0]
        wr[:, cfg.E - 1] = wr[:, cfg.E // 2]
        ol.w_router = np.ascontiguousarray(wr)
        gl = mq.MoELayer(torch.from_numpy(wr).cuda(), gl.gate, gl.up, gl.down, cfg.k,
                         gl.router_bias, gl.s_gate, gl.s_up, gl.s_down)
    x, bits, xw, xd, xbd = tokens(cfg, step=step, T=T)
    return ol, gl, xw, xbd


def _check_route(ol, r, xw):
    ref = oracle.route(ol, xw)
    assert np.array_equal(r.logits.cpu().numpy().view(np.uint32), ref["logits"].view(np.uint32))
    assert np.array_equal(r.topk_ids.cpu().numpy(), ref["ids"])
    assert np.array_equal(r.topk_w.cpu().numpy().view(np.uint32), ref["w32"].view(np.uint32))
    assert np.array_equal(r.expert_offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(r.perm.cpu().numpy(), ref["perm"])
    assert np.array_equal(r.inv_perm.cpu().numpy(), ref["inv_perm"])
    return ref


@pytest.mark.parametrize("name,T,E,k,H,bias", [
    ("tiny", 16, 8, 2, 256, None),
    ("ragged", 1, 16, 4, 256, None),
    ("ragged", 65, 16, 4, 256, None),
    ("ragged", 200, 128, 8, 512, "zipf"),
    ("odd_chunks", 70, 24, 3, 96, None),
    ("wide", 130, 256, 8, 2048, None),
    ("k_equals_e", 33, 4, 4, 128, None),
    ("one_expert", 40, 1, 1, 64, None),
    ("one_chunk", 40, 8, 2, 32, None),
    ("e_not_mult_64", 100, 37, 6, 1024, None),
    ("e256_long", 700, 256, 8, 2048, "zipf"),
])
def test_route_bit_exact(name, T, E, k, H, bias):
    say("route", name, T, E, k, H, bias)
    cfg = moe_synth.CONFIGS["tiny"].with_(name=name, E=E, k=k, H=H, I=64, shared=False, bias=bias)
    ol, gl, xw, xbd = _route_case(cfg, T)
    r = mq.moe_q4_route(gl, xbd, logits=True)
    _check_route(ol, r, xw)
    # fp32 input path
    r32 = mq.moe_q4_route(gl, torch.from_numpy(xw).cuda(), logits=True)
    _check_route(ol, r32, xw)


def test_route_ties_lower_index():
    cfg = moe_synth.CONFIGS["tiny"].with_(name="ties", E=16, k=4, H=256, I=64, shared=False)
    ol, gl, xw, xbd = _route_case(cfg, 96, tie_cols=True)
    r = mq.moe_q4_route(gl, xbd, logits=True)
    ref = _check_route(ol, r, xw)
    ids = ref["ids"]
    both = (ids == 0).any(1) & (ids == 1).any(1)
    assert both.any()
    for t in np.nonzero(both)[0]:
        assert list(ids[t]).index(0) + 1 == list(ids[t]).index(1)


def test_route_all_tied_tokens():
    # zero tokens tie every logit at +0 (no bias): the picks are experts 0..k-1
    # in order, each weighted 1/k; mixed with ordinary tokens in one batch
    cfg = moe_synth.CONFIGS["tiny"].with_(name="zero_tok", E=64, k=8, H=256, I=64, shared=False)
    ol, gl = both_layers(cfg)
    x, bits, xw, xd, xbd = tokens(cfg, T=48)
    xw = xw.copy()
    xw[::3] = 0.0
    xbd = torch.from_numpy(moe_synth.to_bf16_bits(xw).view(np.int16)).cuda().view(torch.bfloat16)
    r = mq.moe_q4_route(gl, xbd, logits=True)
    ref = _check_route(ol, r, xw)
    assert np.array_equal(ref["ids"][::3], np.tile(np.arange(cfg.k, dtype=np.int32), (16, 1)))
    assert np.all(ref["w32"][::3] == np.float32(1.0 / cfg.k))


def test_route_deterministic_and_empty():
    cfg = moe_synth.CONFIGS["tiny"]
    ol, gl = both_layers(cfg)
    _, _, xw, _, xbd = tokens(cfg)
    a = mq.moe_q4_route(gl, xbd)
    b = mq.moe_q4_route(gl, xbd)
    for f in ("topk_ids", "expert_offsets", "perm", "inv_perm"):
        assert torch.equal(getattr(a, f), getattr(b, f))
    e = mq.moe_q4_route(gl, xbd[:0])
    assert torch.count_nonzero(e.expert_offsets).item() == 0
    y = mq.moe_q4_prefill(gl, xbd[:0], e)
    assert y.shape == (0, cfg.H)


# ---------------------------------------------------------------- prefill
def _prefill_err(ol, gl, cfg, T, sample=None, step=0):
    x, bits, xw, xd, xbd = tokens(cfg, step=step, T=T)
    r = mq.moe_q4_route(gl, xbd)
    y = mq.moe_q4_prefill(gl, xbd, r).cpu().numpy().astype(np.float64)
    ref_route = oracle.route(ol, xw)
    assert np.array_equal(r.topk_ids.cpu().numpy(), ref_route["ids"])
    if callable(sample):
        sample = sample(ref_route)
    toks = np.arange(T) if sample is None else np.asarray(sample)
    yref = oracle.prefill_ref(ol, xw, ref_route["ids"], ref_route["w64"], tokens=toks, threads=8)
    ys = y[toks]
    assert np.all(np.isfinite(ys))
    rel = np.linalg.norm(ys - yref) / np.linalg.norm(yref)
    per_tok = np.linalg.norm(ys - yref, axis=1) / np.linalg.norm(yref, axis=1)
    say("prefill rel-L2 %.3e  worst token %.3e" % (rel, per_tok.max()))
    return rel, per_tok, y, ref_route


def _check_program(ol, xw, rr, y, toks, label):
    """y rows of the listed tokens against the oracle's bf16 program."""
    yp = oracle.prefill_bf16(ol, xw, rr["ids"], rr["w32"], tokens=toks, threads=16).astype(np.float64)
    ys = y[toks]
    rel = np.linalg.norm(ys - yp) / np.linalg.norm(yp)
    per_tok = np.linalg.norm(ys - yp, axis=1) / np.maximum(np.linalg.norm(yp, axis=1), 1e-30)
    say("%s: vs the bf16 program rel-L2 %.3e, worst token %.3e over %d tokens" %
        (label, rel, per_tok.max(), len(toks)))
    assert rel <= PROGRAM_TOL
    assert per_tok.max() <= PROGRAM_TOK_TOL


@pytest.mark.parametrize("name,T,H,E,I,k,shared", [
    ("tiny", 16, 256, 8, 128, 2, False),
    ("multi_tile", 300, 512, 16, 256, 4, True),
    ("ragged_k_tail", 77, 96, 5, 96, 2, True),
    ("one_expert_dense", 150, 256, 1, 128, 1, False),
    # more than 8 slots per token (the combine's wide path), and k = E
    ("wide_topk", 96, 256, 64, 128, 16, True),
    ("every_expert", 64, 256, 32, 64, 32, True),
])
@pytest.mark.parametrize("tiles", [True, False], ids=["tiled", "rowmajor"])
def test_prefill_small(name, T, H, E, I, k, shared, tiles):
    say("prefill", name, T, H, E, I, k, shared, "tiles" if tiles else "row-major")
    cfg = moe_synth.CONFIGS["tiny"].with_(name=name, H=H, E=E, I=I, k=k, shared=shared)
    ol, gl = both_layers(cfg, tiles=tiles)
    assert (gl.tiles is not None) == (tiles and H % 64 == 0 and I % 64 == 0)
    rel, per_tok, y, rr = _prefill_err(ol, gl, cfg, T)
    assert rel <= PREFILL_TOL
    assert per_tok.max() <= 3 * PREFILL_TOL
    x, bits, xw, xd, xbd = tokens(cfg, T=T)
    _check_program(ol, xw, rr, y, np.arange(T), name)


@pytest.fixture(scope="module")
def prefill_layer():
    cfg = moe_synth.CONFIGS["prefill"]
    say("building prefill-size layer")
    return cfg, both_layers(cfg)


def _cover_sample(rr, T, k, extra=0, seed=0):
    """Tokens such that every 32-row subtile of every expert segment (the
    grouped GEMM's unit of rows) and of the shared expert's rows holds at
    least one sampled row: segment positions 0, 32, 64, ... and the last of
    each non-empty segment, mapped to their tokens through the oracle's perm,
    plus tokens 0, 32, ..., T-1 (the shared expert's rows are in token order)
    and `extra` random tokens."""
    off, perm = rr["offsets"], rr["perm"]
    pos = []
    for e in range(len(off) - 1):
        if off[e + 1] > off[e]:
            pos.extend(range(off[e], off[e + 1], 32))
            pos.append(off[e + 1] - 1)
    toks = [perm[np.asarray(pos)] // k, np.arange(0, T, 32), [T - 1]]
    if extra:
        toks.append(np.random.default_rng(seed).choice(T, extra, replace=False))
    return np.unique(np.concatenate(toks))


def test_prefill_2k_sampled(prefill_layer):
    cfg, (ol, gl) = prefill_layer
    rel, per_tok, y, rr = _prefill_err(ol, gl, cfg, cfg.T,
                                       sample=lambda rr: _cover_sample(rr, cfg.T, cfg.k, extra=45, seed=1))
    say("sampled %d tokens" % per_tok.size)
    assert rel <= PREFILL_TOL
    assert per_tok.max() <= 3 * PREFILL_TOL
    # every expert segment is non-empty at this size; the y rows exist for all tokens
    assert np.all(np.diff(rr["offsets"]) > 0)
    assert np.all(np.isfinite(y))
    x, bits, xw, xd, xbd = tokens(cfg, T=cfg.T)
    _check_program(ol, xw, rr, y, _cover_sample(rr, cfg.T, cfg.k, extra=45, seed=1), "2k")


def test_prefill_2k_sampled_generic_kernels(prefill_layer):
    # the same packed layer without tile-order copies: the generic grouped GEMM
    cfg, (ol, gl) = prefill_layer
    g2 = mq.MoELayer(gl.w_router, gl.gate, gl.up, gl.down, gl.top_k, gl.router_bias,
                     gl.s_gate, gl.s_up, gl.s_down, tiles=False)
    sample = np.array([0, 7, 1000, cfg.T - 1])
    rel, _, y, rr = _prefill_err(ol, g2, cfg, cfg.T, sample=sample)
    assert rel <= PREFILL_TOL
    x, bits, xw, xd, xbd = tokens(cfg, T=cfg.T)
    _check_program(ol, xw, rr, y, sample, "2k generic kernels")


def _fused_vs_stages(gl, xbd):
    """moe_q4_prefill (all stages in one call) against the stages run apart
    (gate/up + down, then the combine)."""
    T = xbd.shape[0]
    r = mq.moe_q4_route(gl, xbd)
    y_all = mq.moe_q4_prefill(gl, xbd, r)
    ws = torch.empty(mq.moe_q4_prefill_workspace_bytes(gl, T), dtype=torch.uint8, device="cuda")
    y_st = torch.empty_like(y_all)
    S = mq._lib
    mq.moe_q4_prefill_stage(gl, xbd, r, y_st, ws, S.STAGE_GATEUP | S.STAGE_DOWN)
    mq.moe_q4_prefill_stage(gl, xbd, r, y_st, ws, S.STAGE_COMBINE)
    return y_all, y_st


@pytest.mark.parametrize("k", [3, 4])
def test_prefill_stores_stay_inside_tile_rows(k):
    """The grouped GEMM stores through buffer descriptors bounded by each
    tile's row count, so a partial tile's padding rows are never stored.
    With 77 tokens the shared expert's last tile and the last expert's
    segment end inside a 32-row group: y sits at the start of a larger
    buffer whose tail holds a sentinel, and the workspace is filled with a
    sentinel byte first.  After gate/up + down, the tail past y and the
    alignment padding after h (k = 4) or after the expert outputs (k = 3)
    are unchanged, and after the combine y equals a one-call prefill's bit
    for bit."""
    cfg = moe_synth.CONFIGS["tiny"].with_(name="pad_rows", T=77, H=320, E=16, I=64, k=k, shared=True)
    ol, gl = both_layers(cfg)
    assert gl.tiles is not None
    x, bits, xw, xd, xbd = tokens(cfg, T=cfg.T)
    T, H, I = cfg.T, cfg.H, cfg.I
    r = mq.moe_q4_route(gl, xbd)
    say("padding rows: T=%d k=%d H=%d I=%d" % (T, k, H, I))
    sentinel = -12345.0
    big = torch.full(((T + 64) * H,), sentinel, dtype=torch.float32, device="cuda")
    y = big[:T * H].view(T, H)
    ws = torch.full((mq.moe_q4_prefill_workspace_bytes(gl, T),), 0xA5, dtype=torch.uint8, device="cuda")
    S = mq._lib
    mq.moe_q4_prefill_stage(gl, xbd, r, y, ws, S.STAGE_GATEUP | S.STAGE_DOWN)
    torch.cuda.synchronize()
    assert torch.all(big[T * H:] == sentinel)
    # workspace: h [(T*k + T) rows][I] bf16, then the expert outputs [T*k][H]
    # bf16, each region rounded up to 256 bytes
    up256 = lambda n: (n + 255) // 256 * 256
    h_end = (T * k + T) * I * 2
    o0 = up256(h_end)
    o_end = o0 + T * k * H * 2
    pads = [(h_end, o0), (o_end, up256(o_end))]
    pads = [(a, b) for a, b in pads if b > a]
    assert pads, "the shape leaves no padding to check"
    wsc = ws.cpu().numpy()
    for a, b in pads:
        assert np.all(wsc[a:b] == 0xA5), (a, b)
    mq.moe_q4_prefill_stage(gl, xbd, r, y, ws, S.STAGE_COMBINE)
    y_one = mq.moe_q4_prefill(gl, xbd, r)
    assert torch.equal(y, y_one)
    assert torch.all(big[T * H:] == sentinel)


def test_prefill_all_stages_match_stages_apart(prefill_layer):
    # the same y bit for bit, whichever way the call is split
    cfg, (ol, gl) = prefill_layer
    x, bits, xw, xd, xbd = tokens(cfg, T=cfg.T, step=11)
    y_all, y_st = _fused_vs_stages(gl, xbd)
    assert torch.equal(y_all, y_st)


@pytest.mark.parametrize("name,T,H,E,I,k,shared", [
    ("no_shared", 300, 512, 16, 256, 4, False),
    ("ragged_cols", 77, 192, 5, 64, 2, True),
    ("k8_many_tiles", 700, 256, 64, 128, 8, True),
])
def test_prefill_all_stages_small(name, T, H, E, I, k, shared):
    cfg = moe_synth.CONFIGS["tiny"].with_(name=name, H=H, E=E, I=I, k=k, shared=shared)
    ol, gl = both_layers(cfg)
    x, bits, xw, xd, xbd = tokens(cfg, T=T)
    y_all, y_st = _fused_vs_stages(gl, xbd)
    assert torch.equal(y_all, y_st)
    # and against the binary64 reference
    ref_route = oracle.route(ol, xw)
    yref = oracle.prefill_ref(ol, xw, ref_route["ids"], ref_route["w64"], threads=8)
    rel = np.linalg.norm(y_all.cpu().numpy().astype(np.float64) - yref) / np.linalg.norm(yref)
    assert rel <= PREFILL_TOL, rel


def test_prefill_2k_token_permutation_equivariance(prefill_layer):
    cfg, (ol, gl) = prefill_layer
    x, bits, xw, xd, xbd = tokens(cfg, T=512, step=5)
    r = mq.moe_q4_route(gl, xbd)
    y = mq.moe_q4_prefill(gl, xbd, r)
    p = torch.randperm(512, generator=torch.Generator().manual_seed(0)).cuda()
    xp = xbd[p].contiguous()
    r2 = mq.moe_q4_route(gl, xp)
    y2 = mq.moe_q4_prefill(gl, xp, r2)
    # a token's rows are independent of its batch position (same tiles -> same sums
    # is not guaranteed, the value is); compare within the bf16 path tolerance
    rel = (torch.linalg.norm(y2 - y[p]) / torch.linalg.norm(y)).item()
    assert rel <= 1e-3, rel


def test_prefill_skewed_10k_sampled():
    cfg = moe_synth.CONFIGS["skew"]
    say("building skewed layer")
    ol, gl = both_layers(cfg)
    x, bits, xw, xd, xbd = tokens(cfg)
    r = mq.moe_q4_route(gl, xbd)
    ref = oracle.route(ol, xw)
    assert np.array_equal(r.topk_ids.cpu().numpy(), ref["ids"])
    assert np.array_equal(r.perm.cpu().numpy(), ref["perm"])
    counts = np.diff(ref["offsets"])
    say("skew: hottest expert %d rows, empty experts %d" % (counts.max(), (counts == 0).sum()))
    y = mq.moe_q4_prefill(gl, xbd, r).cpu().numpy().astype(np.float64)
    # every 32-row subtile of every non-empty segment (the hot expert's 10k
    # rows included) and of the shared expert contributes a sampled token
    sample = _cover_sample(ref, cfg.T, cfg.k, extra=30, seed=3)
    yref = oracle.prefill_ref(ol, xw, ref["ids"], ref["w64"], tokens=sample, threads=16)
    rel = np.linalg.norm(y[sample] - yref) / np.linalg.norm(yref)
    per_tok = np.linalg.norm(y[sample] - yref, axis=1) / np.linalg.norm(yref, axis=1)
    say("skew prefill rel-L2 %.3e over %d tokens, worst token %.3e" % (rel, sample.size, per_tok.max()))
    assert rel <= PREFILL_TOL
    assert per_tok.max() <= 3 * PREFILL_TOL
    assert np.all(np.isfinite(y))
    # every fourth sampled token against the bf16 program
    _check_program(ol, xw, ref, y, sample[::4], "skew")


def test_prefill_wait_failure_is_reported():
    """The fused launch's bounded wait: forced to give up from the host (a
    tile count that is never reached, a 16-poll bound), every down unit
    stores nothing and is counted, and the kernels still end; the next normal
    call on the same workspace reports 0 and is correct again."""
    cfg = moe_synth.CONFIGS["tiny"].with_(name="waitfail", T=300, H=256, E=16, I=128, k=4, shared=True)
    ol, gl = both_layers(cfg)
    assert gl.tiles is not None
    x, bits, xw, xd, xbd = tokens(cfg, T=cfg.T)
    r = mq.moe_q4_route(gl, xbd)
    ws = torch.empty(mq.moe_q4_prefill_workspace_bytes(gl, cfg.T), dtype=torch.uint8, device="cuda")
    y = torch.zeros((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    S = mq._lib
    mq.moe_q4_prefill_stage(gl, xbd, r, y, ws, S.STAGE_GATEUP | S.STAGE_DOWN | S.STAGE_TEST_WAIT_FAIL)
    torch.cuda.synchronize()
    failed = mq.moe_q4_prefill_status(gl, cfg.T, ws)
    say("forced give-ups:", failed)
    # every down unit gave up once: ceil(H / 256) per tile, the tiles being
    # the shared expert's ceil(T / 160) and ceil(c_e / 160) per expert
    c = np.diff(r.expert_offsets.cpu().numpy())
    n_tiles = -(-cfg.T // 160) + int(np.sum(-(-c // 160)))
    assert failed == n_tiles * -(-cfg.H // 256)
    # down units that gave up stored nothing: the shared expert's rows of y stay 0
    assert torch.count_nonzero(y).item() == 0
    y = mq.moe_q4_prefill(gl, xbd, r, ws=ws)
    assert mq.moe_q4_prefill_status(gl, cfg.T, ws) == 0
    ref = oracle.route(ol, xw)
    yref = oracle.prefill_ref(ol, xw, ref["ids"], ref["w64"])
    yy = y.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(yy - yref) / np.linalg.norm(yref) <= PREFILL_TOL


# ---------------------------------------------------------------- decode
def _decode_steps(ol, gl, cfg, steps):
    ws = mq.decode_workspace(gl)
    worst = 0.0
    for step in steps:
        x = moe_synth.tokens(cfg, step=step, T=1)[0]
        y, tr = mq.moe_q4_decode(gl, torch.from_numpy(x).cuda(), ws=ws, trace=True)
        yo, to = oracle.decode(ol, x, trace=True)
        assert np.array_equal(tr["logits"].cpu().numpy().view(np.uint32), to["logits"].view(np.uint32))
        assert np.array_equal(tr["ids"].cpu().numpy(), to["ids"])
        assert np.array_equal(tr["w"].cpu().numpy().view(np.uint32), to["w"].view(np.uint32))
        assert np.array_equal(tr["qx"].cpu().numpy(), to["qx"])
        assert np.array_equal(tr["dx"].cpu().numpy().view(np.uint32), to["dx"].view(np.uint32))
        assert np.array_equal(tr["qh"].cpu().numpy(), to["qh"])
        assert np.array_equal(tr["dh"].cpu().numpy().view(np.uint32), to["dh"].view(np.uint32))
        yg = y.cpu().numpy()
        err = np.max(np.abs(yg.astype(np.float64) - yo)) / np.max(np.abs(yo))
        worst = max(worst, err)
        assert err <= DECODE_TOL, (step, err)
    return worst


@pytest.mark.parametrize("name,H,E,I,k,shared,bias", [
    ("tiny", 256, 8, 128, 2, False, None),
    ("tiny_shared", 256, 8, 128, 2, True, None),
    ("odd_chunks", 96, 5, 96, 3, True, None),
    ("zipf_bias", 512, 64, 256, 8, True, "zipf"),
    # H = 16384: 32 blocks per lane, 16 lanes per row (1024-thread gate/up blocks)
    ("wide_hidden", 16384, 8, 64, 2, True, None),
    # 9 slots x I = 8192: q8(h) of every slot exceeds the down kernel's LDS
    # budget, so its activation blocks are read from memory
    ("wide_inter", 256, 16, 8192, 8, True, None),
    # the largest expert count and top-k the library accepts
    ("many_experts", 256, 1024, 64, 32, True, "zipf"),
    # the largest top-k on the fast row programs (33 slots; 264 gate/up
    # blocks and 33 rows per down block)
    ("many_slots", 512, 128, 256, 32, True, "zipf"),
    # past 128 experts the one-launch step takes its top-k by wave rounds:
    # 256 experts, a count that is not a power of two, and the 1024 limit
    ("e256", 512, 256, 128, 8, True, None),
    ("e200", 256, 200, 64, 6, False, "zipf"),
    ("e1024_k4", 256, 1024, 64, 4, True, "zipf"),
])
def test_decode_small(name, H, E, I, k, shared, bias):
    say("decode", name)
    cfg = moe_synth.CONFIGS["tiny"].with_(name=name, H=H, E=E, I=I, k=k, shared=shared, bias=bias)
    ol, gl = both_layers(cfg)
    _decode_steps(ol, gl, cfg, range(6))


@pytest.mark.parametrize("name,H,E,I,k,shared", [
    ("tiny_shared", 256, 8, 128, 2, True),
    # the smallest tiled shape: H = I = 64, one piece per row, one wave
    ("minimal", 64, 4, 64, 2, True),
    # H = 192 and 320: 3 and 5 tile pieces per row, padded to 4 and 8 waves
    # of one piece, the last waves holding only +0 leaves
    ("ragged_pieces", 192, 16, 128, 4, True),
    ("ragged_pieces5", 320, 8, 64, 3, False),
    # H = 16384: 16 pieces per wave in 4 chunks
    ("wide_hidden", 16384, 8, 64, 2, True),
    ("many_experts", 256, 1024, 64, 32, True),
    # down rows of I = 192 (3 pieces, one +0 piece), 2048 (32 pieces in 4
    # chunks) and 4096 (past the tiled down kernel's 32 pieces: row-major)
    ("ragged_inter", 256, 8, 192, 3, True),
    ("wide_inter", 128, 8, 2048, 4, True),
    ("wider_inter", 128, 8, 4096, 2, True),
])
def test_decode_tiled_matches_rowmajor(name, H, E, I, k, shared):
    # the gate/up and down launches over the tile-order copies realise the
    # same pinned trees as the row-major ones: every traced value and y are
    # bit-identical
    say("decode tiled vs row-major", name)
    cfg = moe_synth.CONFIGS["tiny"].with_(name=name, H=H, E=E, I=I, k=k, shared=shared, bias="zipf")
    W = moe_synth.expert_weights(cfg, 0, threads=16)
    gt = device_layer(cfg, weights=W, tiles=True)
    gr = device_layer(cfg, weights=W, tiles=False)
    assert gt.tiles is not None and gr.tiles is None
    for step in range(4):
        x = torch.from_numpy(moe_synth.tokens(cfg, step=step, T=1)[0]).cuda()
        yt, tt = mq.moe_q4_decode(gt, x, trace=True)
        yr, trr = mq.moe_q4_decode(gr, x, trace=True)
        assert np.array_equal(yt.cpu().numpy().view(np.uint32), yr.cpu().numpy().view(np.uint32)), step
        for key in ("ids", "w", "qh", "dh", "logits"):
            assert np.array_equal(tt[key].cpu().numpy(), trr[key].cpu().numpy()), (step, key)


@pytest.mark.parametrize("cfgname", ["tiny_shared", "decode"])
def test_decode_wait_failure_is_reported(cfgname):
    """The one-launch decode's bounded waits: with the test switch every wait
    looks for a tag no word carries and gives up after 16 polls; the kernel
    ends, moe_q4_decode_status counts the failures (the three-launch path has
    no waits, so a count > 0 also shows the one-launch kernel ran), and the
    next normal step on the same workspace is exact again."""
    cfg = (moe_synth.CONFIGS["tiny"].with_(name="tiny_shared", shared=True) if cfgname == "tiny_shared"
           else moe_synth.CONFIGS["decode"])
    ol, gl = both_layers(cfg)
    ws = mq.decode_workspace(gl)
    x = moe_synth.tokens(cfg, step=3, T=1)[0]
    xd = torch.from_numpy(x).cuda()
    y0 = mq.moe_q4_decode(gl, xd, ws=ws)
    assert mq.moe_q4_decode_status(gl, ws) == 0
    lib = mq._lib.lib()
    try:
        lib.moe_q4_test_decode_wait_fail(1)
        mq.moe_q4_decode(gl, xd, ws=ws)
        torch.cuda.synchronize()
    finally:
        lib.moe_q4_test_decode_wait_fail(0)
    failed = mq.moe_q4_decode_status(gl, ws)
    say("forced decode give-ups:", failed)
    assert failed > 0
    assert mq.moe_q4_decode_status(gl, ws) == 0          # the query resets the count
    y1 = mq.moe_q4_decode(gl, xd, ws=ws)
    assert torch.equal(y0, y1)
    assert np.array_equal(y1.cpu().numpy(), oracle.decode(ol, x))
    assert mq.moe_q4_decode_status(gl, ws) == 0


def test_decode_tied_logits():
    # experts 2j and 2j+1 share a router column, so every logit ties with its
    # pair: the choice takes the lower index first (k rounds of "first maximum
    # among the rest").  An all-zero x ties every logit at zero.
    cfg = moe_synth.CONFIGS["tiny"].with_(name="ties", H=256, E=16, I=64, k=5, shared=True, bias=None)
    W = moe_synth.expert_weights(cfg, 0, threads=16)
    Wr = moe_synth.router(cfg, 0).copy()
    Wr[:, 1::2] = Wr[:, 0::2]
    ol = oracle.PackedLayer.from_float(Wr, None, W["gate"], W["up"], W["down"], W["s_gate"], W["s_up"],
                                       W["s_down"], k=cfg.k, threads=16)
    g0 = device_layer(cfg, weights=W, rowmajor=True)
    gl = mq.MoELayer(torch.from_numpy(Wr).cuda(), g0.gate, g0.up, g0.down, cfg.k, router_bias=None,
                     s_gate=g0.s_gate, s_up=g0.s_up, s_down=g0.s_down)
    _decode_steps(ol, gl, cfg, range(4))
    for step in range(4):
        x = moe_synth.tokens(cfg, step=step, T=1)[0]
        _, tr = mq.moe_q4_decode(gl, torch.from_numpy(x).cuda(), trace=True)
        ids = tr["ids"].cpu().numpy()
        assert np.all(ids[0::2] % 2 == 0) and np.all(ids[1::2] == ids[0:4:2] + 1), ids
    x0 = np.zeros(cfg.H, dtype=np.float32)
    y, tr = mq.moe_q4_decode(gl, torch.from_numpy(x0).cuda(), trace=True)
    yo, to = oracle.decode(ol, x0, trace=True)
    assert np.array_equal(tr["ids"].cpu().numpy(), to["ids"])
    assert np.array_equal(to["ids"], np.arange(cfg.k))
    assert np.array_equal(y.cpu().numpy().view(np.uint32), yo.astype(np.float32).view(np.uint32))


def test_decode_full_layer():
    cfg = moe_synth.CONFIGS["decode"]
    say("building decode-size layer")
    ol, gl = both_layers(cfg)
    worst = _decode_steps(ol, gl, cfg, range(12))
    say("decode worst max-rel %.3e" % worst)


def test_w4a8_dots_of_decode_layer_rows():
    # per-block int32 dots of real layer rows (gate rows of one expert) are exact
    cfg = moe_synth.CONFIGS["tiny"].with_(name="dots", H=2048, E=2, I=512, k=1, shared=False)
    ol, gl = both_layers(cfg)
    x = moe_synth.tokens(cfg, step=0, T=1)[0]
    qa, da = oracle.q8_quantize(x[None])
    W = ol.gate[1]
    dots_o, out_o = oracle.w4a8_gemv(W, cfg.H, qa[0], da[0])
    dots, out = mq.moe_q4_w4a8_gemv(gl.gate[1].contiguous(), cfg.I, cfg.H, torch.from_numpy(qa[0]).cuda(),
                                    torch.from_numpy(da[0]).cuda())
    assert np.array_equal(dots.cpu().numpy(), dots_o)
    assert np.array_equal(out.cpu().numpy(), out_o)


# K/32 blocks per row: 2 and 4 (a single group of 2 or 4 leaves), 6 (one
# group of 8 with +0 leaves), 20 and 34 (groups of 8 taken four blocks at a
# time, then a ragged group and groups of +0 leaves), 64 and 128
@pytest.mark.parametrize("M,N,K", [(1, 32, 64), (5, 32, 128), (37, 96, 192), (31, 160, 640), (70, 96, 1088),
                                   (64, 128, 2048), (130, 512, 2048), (33, 64, 4096)])
def test_w4a8_gemm_is_the_row_program(M, N, K):
    # int8 MFMA block dots bit-exact against the oracle's, and every output
    # row bit-identical to the one-token GEMV of the same token
    rng = np.random.default_rng(M * 131 + N + K)
    w = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).cuda()
    W = mq.q4_pack(w)
    Wt = mq.q4_tile(W)
    x = (rng.standard_normal((M, K)) * rng.choice([0.1, 1.0, 30.0], size=(M, 1))).astype(np.float32)
    x[0, :32] = 0.0                                   # an all-zero activation block
    qa, da = oracle.q8_quantize(x)
    qad, dad = torch.from_numpy(qa).cuda(), torch.from_numpy(da).cuda()
    dots, out = mq.moe_q4_w4a8_gemm(Wt, N, K, qad, dad, with_dots=True)
    dots, out = dots.cpu().numpy(), out.cpu().numpy()
    _, out_nd = mq.moe_q4_w4a8_gemm(Wt, N, K, qad, dad, with_dots=False)
    assert np.array_equal(out_nd.cpu().numpy().view(np.uint32), out.view(np.uint32))   # the kernel without the export
    Wn = W.cpu().numpy()
    for m in sorted({0, M // 2, M - 1}):
        dots_o, out_o = oracle.w4a8_gemv(Wn, K, qa[m], da[m])
        assert np.array_equal(dots[m], dots_o), m
        assert np.array_equal(out[m].view(np.uint32), out_o.astype(np.float32).view(np.uint32)), m
    for m in range(M):
        _, o1 = mq.moe_q4_w4a8_gemv(W, N, K, qad[m].contiguous(), dad[m].contiguous(), with_dots=False)
        assert np.array_equal(out[m].view(np.uint32), o1.cpu().numpy().view(np.uint32)), m


# ---------------------------------------------------------------- glue
@pytest.mark.parametrize("T,H", [(1, 2048), (9, 96), (64, 256)])
def test_rmsnorm_bit_exact(T, H):
    rng = np.random.default_rng(T + H)
    y = (rng.standard_normal((T, H)) * 3).astype(np.float32)
    o32, o16 = mq.moe_q4_rmsnorm(torch.from_numpy(y).cuda(), 1e-6, f32=True, bf16=True)
    ref = oracle.rmsnorm(y, 1e-6)
    assert np.array_equal(o32.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(o16.view(torch.int16).cpu().numpy().view(np.uint16), moe_synth.to_bf16_bits(ref))
