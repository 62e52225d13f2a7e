"""Pins for the oracle's MXFP8 quantisation and the native-MX layer (no GPU)."""
import math

import numpy as np
import pytest

from oracle import experts, mx
from workload import gen


def _e4m3_table():
    """All finite E4M3 values, from the bit fields written out."""
    vals = set()
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 0xF, c & 7
        if e == 15 and m == 7:
            continue
        mag = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals.add(-mag if s else mag)
    return np.array(sorted(vals))


def test_e4m3_fields():
    t = _e4m3_table()
    assert t.max() == 448.0 and t.min() == -448.0
    assert np.min(t[t > 0]) == 2.0 ** -9                      # smallest subnormal
    assert len(t) == 253                                      # 254 finite codes, +-0 equal
    for c in (0x00, 0x01, 0x08, 0x38, 0x7E, 0xFE, 0x3F):
        v = mx.e4m3_value(c)
        assert v in set(t) or v == 0.0
    assert mx.e4m3_value(0x38) == 1.0 and mx.e4m3_value(0x7E) == 448.0
    assert math.isnan(mx.e4m3_value(0x7F)) and math.isnan(mx.e4m3_value(0xFF))


def test_round_e4m3_is_nearest_with_ties_to_even():
    t = _e4m3_table()
    pos = t[t >= 0]
    # every representable value maps to itself
    assert np.array_equal(mx.round_e4m3(t), t)
    # midpoints go to the neighbour with the even mantissa code
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = (lo + hi) / 2
        got = mx.round_e4m3(np.array([mid]))[0]
        lo_code = int(np.searchsorted(pos, lo))   # consecutive codes of the grid
        want = lo if lo_code % 2 == 0 else hi
        assert got == want, (lo, hi, got)
    # brute force: nearest element of the table (ties to even) on random values
    rng = np.random.default_rng(4)
    v = rng.uniform(-460, 460, 20000) * np.exp2(rng.integers(-12, 1, 20000))
    got = mx.round_e4m3(v)
    for x, q in zip(v[:3000], got[:3000]):
        c = min(abs(x), 448.0)
        d = np.abs(pos - c)
        best = pos[d == d.min()]
        if len(best) > 1:
            best = [b for b in best if int(np.searchsorted(pos, b)) % 2 == 0]
        assert abs(q) == best[0] and (q == 0 or np.sign(q) == np.sign(x))
    # saturation
    assert np.array_equal(mx.round_e4m3(np.array([449.0, 470.0, 1e6, -500.0])),
                          [448.0, 448.0, 448.0, -448.0])


def test_block_scale_rule():
    # amax in [2^k, 2^(k+1)) -> exponent k - 8; every block element / 2^e < 512
    rng = np.random.default_rng(6)
    v = rng.standard_normal((7, 96)) * np.exp2(rng.integers(-30, 30, (7, 1)))
    e = mx.block_exponents(v)
    amax = np.abs(v.reshape(7, 3, 32)).max(-1)
    assert np.array_equal(e, np.floor(np.log2(amax)).astype(int) - 8)
    assert np.all(amax / np.exp2(e) >= 256) and np.all(amax / np.exp2(e) < 512)
    assert mx.block_exponents(np.zeros((1, 32)))[0, 0] == -127
    assert mx.block_exponents(np.full((1, 32), 2.0 ** 200))[0, 0] == 127   # clamped


def test_quantize_closed_forms():
    # values already on a block's grid are unchanged; a constant block is exact
    blk = mx.round_e4m3(np.linspace(-448, 448, 32)) * 2.0 ** -20
    assert np.array_equal(mx.quantize_mxfp8(blk[None])[0], blk)
    assert np.all(mx.quantize_mxfp8(np.full((2, 64), 0.3))[0] == mx.round_e4m3(np.array([0.3 * 2 ** 10]))[0] * 2.0 ** -10)
    # an element in E4M3's normal range and below the clamp errs by at most
    # half a step (2^-4 of its value); above 448 x 2^e it is clamped
    rng = np.random.default_rng(8)
    v = rng.standard_normal((64, 256))
    q = mx.quantize_mxfp8(v)
    X = np.exp2(np.repeat(mx.block_exponents(v), 32, axis=-1))
    t = np.abs(v) / X
    normal = (t >= 2.0 ** -6) & (t <= 448)
    assert np.all(np.abs(q - v)[normal] <= np.abs(v)[normal] * 2.0 ** -4)
    clamped = t > 464
    assert np.all(np.abs(q)[clamped] == 448 * X[clamped])
    assert np.array_equal(mx.quantize_mxfp8(np.zeros((1, 32))), np.zeros((1, 32)))


def test_mx_layer_equals_plain_layer_on_representable_inputs():
    """Where x and every h are already MXFP8 values, the native-MX layer is the
    plain layer.  Built with W_g = 0 (h = silu(0) * b = 0, exactly
    representable) plus the shared expert's path checked against a hand
    quantisation of h."""
    sh = gen.Shape(H=64, I=64, E=4, k=2, shared=True)
    rng = np.random.default_rng(2)
    x = mx.quantize_mxfp8(rng.standard_normal((3, 64)))      # representable x
    zero = np.zeros((64, 64), np.float32)
    mats = [(zero,) + experts.dequant_expert(gen.expert_weights(sh, 0, e, 2))[1:] for e in range(4)]
    ids = np.array([[0, 1], [2, 3], [1, 2]])
    g = np.array([[0.75, 0.25], [0.5, 0.5], [0.125, 0.875]])
    y0 = mx.moe_layer_mx(x, ids, g, lambda e: mats[e])
    assert np.all(y0 == 0)                                   # h = 0 everywhere
    sw = experts.dequant_expert(gen.expert_weights(sh, 0, -1, 2))
    y = mx.moe_layer_mx(x, ids, g, lambda e: mats[e], shared=sw)
    for t in range(3):
        a = sw[0].astype(np.float64) @ x[t]
        b = sw[1].astype(np.float64) @ x[t]
        h = a / (1 + np.exp(-a)) * b
        want = sw[2].astype(np.float64) @ mx.quantize_mxfp8(h[None])[0]
        assert np.allclose(y[t], want, rtol=1e-12, atol=1e-12)


def test_mx_layer_near_plain_layer():
    """On N(0,1) activations the MXFP8 layer stays close to the plain one: the
    relative rms difference is a few per cent (3 mantissa bits)."""
    sh = gen.Shape(H=256, I=512, E=8, k=2, shared=True)
    x = gen.bf16_bits_to_f32(gen.tokens(sh, 0, 0, 16, 3))
    mats = [experts.dequant_expert(gen.expert_weights(sh, 0, e, 3)) for e in range(8)]
    sw = experts.dequant_expert(gen.expert_weights(sh, 0, -1, 3))
    rng = np.random.default_rng(3)
    ids = np.stack([rng.choice(8, 2, replace=False) for _ in range(16)])
    g = rng.dirichlet([1, 1], 16)
    yp = experts.moe_layer(x, ids, g, lambda e: mats[e], shared=sw)
    yq = mx.moe_layer_mx(x, ids, g, lambda e: mats[e], shared=sw)
    rel = np.sqrt(np.mean((yq - yp) ** 2) / np.mean(yp ** 2))
    assert 1e-3 < rel < 0.06, rel
