"""Pins of the oracle's number formats (CPU only).

Each check compares the oracle with something other than itself: numpy's
IEEE binary16 conversion, hand-worked fixtures under tests/golden/, exact
round-trips and error bounds that follow from the format's definition.
"""
import numpy as np
import pytest

import oracle
from conftest import read_golden

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- binary16
def test_f16_to_f32_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    got = np.array([orc.orc_f16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f16_edge_values():
    v = [0.0, -0.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e30, -1e30,
         2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26,
         2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -11), 2.0 ** -14 * (1 - 2 ** -12),
         1.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 1.0 + 2 ** -11 + 2 ** -20,
         0.1, 0.2, 1 / 3, 1e-8, 6e-8, 5.9604645e-08, 2.9802322e-08, 2.98023259e-08]
    return np.array(v + [-a for a in v], dtype=np.float32)


def test_f32_to_f16_matches_numpy(orc):
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    # dense coverage of the binary16 range, including subnormals and overflow
    y = (rng.standard_normal(100_000) * 10.0 ** rng.uniform(-9, 5.5, 100_000)).astype(np.float32)
    x = np.concatenate([x, y, _f16_edge_values()])
    x = x[np.isfinite(x)]
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([orc.orc_f32_to_f16(float(v)) for v in x], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


# ---------------------------------------------------------------- Q4_0
def _golden_q4_block(g, tag):
    unit = 2.0 ** int(g[tag + "_unit_log2"][0])
    w = np.array([float(u) * unit for u in g[tag + "_w_units"]], dtype=np.float32)
    assert w.size == 32
    exp = bytes(int(b, 16) for b in g[tag + "_bytes"])
    assert len(exp) == 18
    return w, exp


@pytest.mark.parametrize("tag", ["A", "B", "C", "D"])
def test_q4_golden_blocks(tag):
    w, exp = _golden_q4_block(read_golden("q4_blocks.txt"), tag)
    got = oracle.q4_pack(w.reshape(1, 32)).tobytes()
    assert got == exp, (got.hex(), exp.hex())


def _grid_weights(rng, rows, K, log2_lo=-12, log2_hi=-4):
    """Weights exactly on the Q4 grid: w = (q-8)*d, d a power of two (exact in
    fp16), every block with amax = 7d, so packing is lossless."""
    nb = K // 32
    q = rng.integers(1, 16, size=(rows, nb, 32))
    q[:, :, 0] = rng.choice([1, 15], size=(rows, nb))          # |q-8| = 7 present
    d = 2.0 ** rng.integers(log2_lo, log2_hi + 1, size=(rows, nb, 1))
    w = ((q - 8) * d).reshape(rows, K).astype(np.float32)
    return w, q.reshape(rows, K), d.reshape(rows, nb)


def test_q4_grid_roundtrip_lossless():
    rng = np.random.default_rng(7)
    w, q, d = _grid_weights(rng, 64, 256)
    packed = oracle.q4_pack(w)
    assert packed.shape == (64, 8 * 18)
    dq = oracle.q4_dequant(packed, 256)
    assert np.array_equal(dq, w)
    # scales are the powers of two we chose, stored as binary16
    blocks = packed.reshape(64, 8, 18)
    scale = blocks[:, :, 0].astype(np.uint16) | (blocks[:, :, 1].astype(np.uint16) << 8)
    assert np.array_equal(scale.view(np.float16).astype(np.float64), d)
    # nibble layout: byte 2+j = q_j | q_{j+16} << 4
    qb = q.reshape(64, 8, 32)
    assert np.array_equal(blocks[:, :, 2:] & 0xF, qb[:, :, :16])
    assert np.array_equal(blocks[:, :, 2:] >> 4, qb[:, :, 16:])


def test_q4_nibble_positions():
    # one non-zero element per block: exactly one nibble differs from 8
    w = np.zeros((32, 32), dtype=np.float32)
    for j in range(32):
        w[j, j] = 0.25 * (1 if j % 2 else -1)
    blocks = oracle.q4_pack(w)
    for j in range(32):
        nib = np.concatenate([blocks[j, 2:] & 0xF, blocks[j, 2:] >> 4])  # element order
        # nib[i] is element i for i<16 (low) and element i for i>=16 (high)
        assert np.count_nonzero(nib != 8) == 1
        assert nib[j] == (15 if j % 2 else 1)


def test_q4_pack_random_properties():
    rng = np.random.default_rng(11)
    rows, K = 96, 512
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    w[3, :32] = 0.0                                             # a zero block
    packed = oracle.q4_pack(w)
    dq = oracle.q4_dequant(packed, K)
    # idempotence: the dequantised matrix packs to the same bytes
    assert np.array_equal(oracle.q4_pack(dq), packed)
    blocks = packed.reshape(rows, K // 32, 18)
    df = (blocks[:, :, 0].astype(np.uint16) | (blocks[:, :, 1].astype(np.uint16) << 8)).view(np.float16)
    # the scale is binary16(amax/7) with the fp32 division (numpy's conversion)
    amax = np.abs(w.reshape(rows, K // 32, 32)).max(axis=2).astype(np.float32)
    assert np.array_equal(df, (amax / np.float32(7.0)).astype(np.float16))
    df = df.astype(np.float64)[:, :, None]
    wb = w.reshape(rows, K // 32, 32).astype(np.float64)
    err = np.abs(wb - dq.reshape(rows, K // 32, 32))
    assert np.all(err <= df / 2 + 1e-30)                        # nearest grid point
    codes = np.concatenate([blocks[:, :, 2:] & 0xF, blocks[:, :, 2:] >> 4], axis=2)
    assert codes.min() >= 1                                     # -8 needs a subnormal scale
    assert np.all(blocks[3, 0, 2:] == 0x88)


def test_q4_dequant_is_exact():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((8, 128)) * 0.05).astype(np.float32)
    packed = oracle.q4_pack(w)
    b = packed.reshape(8, 4, 18)
    d = (b[:, :, 0].astype(np.uint16) | (b[:, :, 1].astype(np.uint16) << 8)).view(np.float16).astype(np.float64)
    codes = np.concatenate([b[:, :, 2:] & 0xF, b[:, :, 2:] >> 4], axis=2).astype(np.float64)
    ref = ((codes - 8) * d[:, :, None]).reshape(8, 128)          # binary64, exact
    assert np.array_equal(oracle.q4_dequant(packed, 128).astype(np.float64), ref)


# ---------------------------------------------------------------- Q8
def test_q8_golden_blocks():
    g = read_golden("q8_blocks.txt")
    x = np.concatenate([np.array(g["x%d" % i], dtype=np.float32) for i in range(3)])
    assert x.size == 96
    q, d = oracle.q8_quantize(x.reshape(1, 96))
    for i in range(3):
        assert d[0, i] == np.float32(g["d%d" % i][0])
        assert np.array_equal(q[0, 32 * i:32 * (i + 1)], np.array(g["q%d" % i], dtype=np.int8))


def test_q8_properties():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 2048)) * rng.uniform(1e-3, 10, (64, 1))).astype(np.float32)
    q, d = oracle.q8_quantize(x)
    xb = x.reshape(64, 64, 32).astype(np.float64)
    qb = q.reshape(64, 64, 32).astype(np.float64)
    amax = np.abs(xb).max(axis=2)
    assert np.array_equal(d, (amax.astype(np.float32) / np.float32(127.0)))
    # the amax element maps to +-127
    idx = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(qb, idx[..., None], axis=2)[..., 0]
    assert np.all(np.abs(top) == 127)
    # each code is the nearest integer to x/d (x/d in fp32, as the definition)
    ratio = (x.reshape(64, 64, 32) / d[..., None]).astype(np.float64)
    assert np.all(np.abs(ratio - qb) <= 0.5)
    assert np.all(np.abs(qb) <= 127)
    # scaling by a power of two leaves every code unchanged
    q2, d2 = oracle.q8_quantize(x * np.float32(2.0 ** -7))
    assert np.array_equal(q2, q) and np.array_equal(d2, d * np.float32(2.0 ** -7))


def test_q8_round_half_away():
    # x/d exactly k + 1/2 for d = 1: rounding goes away from zero
    x = np.zeros(32, np.float32)
    x[0] = 127.0
    x[1:9] = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5]
    q, d = oracle.q8_quantize(x.reshape(1, 32))
    assert d[0, 0] == 1.0
    assert list(q[0, 1:9]) == [1, 2, 3, 4, -1, -2, -3, -4]


# ---------------------------------------------------------------- Q8_0 weights
def _golden_q8w_block(g, tag):
    if tag + "_w_dec" in g:
        w = np.array([float(u) for u in g[tag + "_w_dec"]], dtype=np.float32)
    else:
        unit = 2.0 ** int(g[tag + "_unit_log2"][0])
        w = np.array([float(u) * unit for u in g[tag + "_w_units"]], dtype=np.float32)
    assert w.size == 32
    exp = bytes(int(b, 16) for b in g[tag + "_bytes"])
    assert len(exp) == 34
    return w, exp


@pytest.mark.parametrize("tag", ["A", "B", "C", "D", "E"])
def test_q8w_golden_blocks(tag):
    w, exp = _golden_q8w_block(read_golden("q8w_blocks.txt"), tag)
    got = oracle.q8w_pack(w.reshape(1, 32)).tobytes()
    assert got == exp, (got.hex(), exp.hex())


def test_q8w_grid_roundtrip_lossless():
    # w = q*d with d a power of two (exact in fp16) and |q| = 127 in every
    # block: packing returns q and d, dequantising returns w exactly
    rng = np.random.default_rng(11)
    rows, K = 48, 256
    nb = K // 32
    q = rng.integers(-127, 128, size=(rows, nb, 32))
    q[:, :, 5] = rng.choice([-127, 127], size=(rows, nb))
    d = 2.0 ** rng.integers(-14, -2, size=(rows, nb, 1))
    w = (q * d).reshape(rows, K).astype(np.float32)
    packed = oracle.q8w_pack(w).reshape(rows, nb, 34)
    codes = packed[:, :, 2:].view(np.int8)
    scale = packed[:, :, :2].copy().view(np.float16).astype(np.float64)[:, :, 0]
    assert np.array_equal(codes, q)
    assert np.array_equal(scale, d[:, :, 0])
    assert np.array_equal(oracle.q8w_dequant(packed.reshape(rows, -1), K), w)


def test_q8w_rounding_error_bound():
    # normal-range d: |w - q d| <= d / 2, and the block's largest |w| maps to
    # +-127 (|w/d| <= 127 (1 + 2^-11) < 127.5, so the clamp never acts)
    rng = np.random.default_rng(12)
    rows, K = 64, 512
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    packed = oracle.q8w_pack(w).reshape(rows, K // 32, 34)
    d = packed[:, :, :2].copy().view(np.float16).astype(np.float64)[:, :, :1]
    q = packed[:, :, 2:].view(np.int8).astype(np.float64)
    wb = w.astype(np.float64).reshape(rows, K // 32, 32)
    assert np.all(np.abs(wb - q * d) <= d / 2 * (1 + 1e-6))
    top = np.argmax(np.abs(wb), axis=2)
    qt = np.take_along_axis(q, top[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(qt) == 127)
