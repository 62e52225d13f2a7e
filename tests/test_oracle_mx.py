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


# ------------------------------------------------ the decision-aware bound
def _bound_case(H, I, seed):
    rng = np.random.default_rng(seed)
    wg = rng.standard_normal((I, H)) / np.sqrt(H)
    wu = rng.standard_normal((I, H)) / np.sqrt(H)
    wd = rng.standard_normal((H, I)) / np.sqrt(I)
    x = mx.quantize_mxfp8(rng.standard_normal(H))
    return x, wg, wu, wd


def _lin_err(c):
    """An allowance of c times the sum of the terms' magnitudes."""
    return lambda ax, aw: c * (ax @ aw.T)


def _simulated_kernel(x, wg, wu, wd, dot_err, h_rel, rng, ends):
    """A native-MX computation whose gate and up sums and whose h evaluation
    err by amounts inside the allowances (random, or at the interval ends),
    with h then quantised by the stated rule; the down product in fp64."""
    I = wg.shape[0]
    a, b = wg @ x, wu @ x
    da = dot_err(np.abs(x)[None], np.abs(wg))[0]
    db = dot_err(np.abs(x)[None], np.abs(wu))[0]
    r = (lambda: rng.choice([-1.0, 1.0], I)) if ends else (lambda: rng.uniform(-1.0, 1.0, I))
    a2, b2 = a + r() * da, b + r() * db
    h2 = a2 / (1.0 + np.exp(-a2)) * b2 * (1.0 + r() * h_rel)
    hq2 = mx.quantize_mxfp8(h2)
    return wd @ hq2, hq2


def test_bound_with_zero_allowance_is_the_mx_layer():
    x, wg, wu, wd = _bound_case(256, 128, 1)
    y, flip, arith = mx.expert_ffn_mx_bound(x, wg, wu, wd, h_rel=0.0, dot_err=_lin_err(0.0))
    assert np.array_equal(y, mx.expert_ffn_mx(x, wg, wu, wd))
    assert np.all(flip == 0) and np.all(arith == 0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bound_covers_every_kernel_inside_the_allowance(seed):
    """Large allowances (1e-3 of the terms' magnitudes per dot product, 1e-3
    on h) so that many h
    elements can round either way: every simulated kernel inside them stays
    within flip of the oracle, and the simulations do flip decisions."""
    x, wg, wu, wd = _bound_case(256, 256, seed)
    dot_err = _lin_err(1e-3)
    y, flip, _ = mx.expert_ffn_mx_bound(x, wg, wu, wd, h_rel=1e-3, dot_err=dot_err)
    hq = mx.quantize_mxfp8(wg @ x / (1 + np.exp(-(wg @ x))) * (wu @ x))
    rng = np.random.default_rng(100 + seed)
    flips = 0
    slack = 1e-12 * (np.abs(wd) @ np.abs(hq))
    for trial in range(60):
        y2, hq2 = _simulated_kernel(x, wg, wu, wd, dot_err, 1e-3, rng, ends=trial % 2 == 0)
        flips += int(np.sum(hq2 != hq))
        assert np.all(np.abs(y2 - y) <= flip + slack), f"trial {trial}"
    assert flips > 60


def test_bound_covers_the_up_error_when_the_gate_sum_does_not_cancel():
    """Gate rows aligned with the signs of x, so that a = sum |w||x| carries
    no cancellation and its allowance is small next to silu(a) times the up
    allowance: kernels that err on the up sums alone (at the interval ends)
    stay within flip, which must therefore carry the up term."""
    x, wg, wu, wd = _bound_case(256, 256, 7)
    wg = np.abs(wg) * np.sign(x)[None, :]
    y, flip, _ = mx.expert_ffn_mx_bound(x, wg, wu, wd, h_rel=0.0, dot_err=_lin_err(1e-3))
    a, b = wg @ x, wu @ x
    hq = mx.quantize_mxfp8(a / (1 + np.exp(-a)) * b)
    db = 1e-3 * (np.abs(wu) @ np.abs(x))
    rng = np.random.default_rng(70)
    slack = 1e-12 * (np.abs(wd) @ np.abs(hq))
    flips = 0
    for trial in range(40):
        b2 = b + rng.choice([-1.0, 1.0], 256) * db
        hq2 = mx.quantize_mxfp8(a / (1 + np.exp(-a)) * b2)
        flips += int(np.sum(hq2 != hq))
        assert np.all(np.abs(wd @ hq2 - y) <= flip + slack), f"trial {trial}"
    assert flips > 40


def test_h_deviation_brute_force_on_small_blocks():
    """Every value reachable by sampling each element's interval (ends and
    random points, amax crossing a power of two included) lies within the
    stated deviation of the oracle's quantised block."""
    rng = np.random.default_rng(9)
    for trial in range(40):
        h = rng.standard_normal(64) * 2.0 ** rng.integers(-4, 5)
        if trial % 4 == 0:                    # amax right at a power of two
            h[np.argmax(np.abs(h[:32]))] = np.sign(h[0]) * 2.0 ** 3
        dh = np.abs(h) * rng.uniform(0, 0.05, 64)
        dev = mx.mx_h_deviation(h[None], dh[None])[0]
        q0 = mx.quantize_mxfp8(h[None])[0]
        for _ in range(200):
            pick = rng.integers(0, 3, 64)
            h2 = np.where(pick == 0, h - dh, np.where(pick == 1, h + dh, h + rng.uniform(-1, 1, 64) * dh))
            q2 = mx.quantize_mxfp8(h2[None])[0]
            assert np.all(np.abs(q2 - q0) <= dev), trial


@pytest.mark.parametrize("H,I", [(256, 256), (2048, 512)])
def test_decision_allowance_rejects_sloppy_kernels(H, I):
    """At the kernel's arithmetic model (mfma_dot_err, h within 2^-16): a
    computation with errors of the measured instruction's size (each 128-term
    instruction off by up to 2^-11.3 of its largest product) keeps every h
    decision inside mx_h_deviation's allowance, while one that differs from
    the mode -- h rounded to bf16 before quantisation, or the block exponent
    one too high -- takes decisions outside it.  The y-level allowance, a
    worst case summed over every h element near a boundary, is much looser
    (tens of per cent of y's rms at H = 2048): the decisions are where a
    kernel of this mode is checked sharply."""
    rng = np.random.default_rng(H)
    n = 64
    wg = rng.standard_normal((I, H)) / np.sqrt(H)
    wu = rng.standard_normal((I, H)) / np.sqrt(H)
    wd = rng.standard_normal((H, I)) / np.sqrt(I)
    x = mx.quantize_mxfp8(rng.standard_normal((n, H)))
    h, dh = mx.expert_h_mx(x, wg, wu)
    dev = mx.mx_h_deviation(h, dh)
    q = mx.quantize_mxfp8(h)

    def noise(w):
        err = np.zeros((n, I))
        for c in range(0, H, 128):
            big = np.max(np.abs(x[:, None, c:c + 128] * w[None, :, c:c + 128]), axis=-1)
            err += rng.uniform(-1, 1, (n, I)) * 2.0 ** -11.3 * big
        return err
    a, b = x @ wg.T + noise(wg), x @ wu.T + noise(wu)
    q_hw = mx.quantize_mxfp8(a / (1 + np.exp(-a)) * b)
    assert np.any(q_hw != q) and np.all(np.abs(q_hw - q) <= dev)
    h_bf16 = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(h.astype(np.float32))).astype(np.float64)
    assert np.any(np.abs(mx.quantize_mxfp8(h_bf16) - q) > dev)
    s = np.repeat(np.ldexp(1.0, mx.block_exponents(h) + 1), 32, axis=-1)
    assert np.any(np.abs(mx.round_e4m3(h / s) * s - q) > dev)
    y, flip, arith = mx.expert_ffn_mx_bound(x, wg, wu, wd, h_rel=2.0 ** -16)
    assert np.max(flip + arith) < 0.5 * np.sqrt(np.mean(y ** 2))


def test_layer_bound_sums_the_experts():
    """moe_layer_mx_bound: y is moe_layer_mx's, and the allowances are the
    gate-weighted sums of the per-expert ones (hand-summed here for one
    token)."""
    sh = gen.Shape(H=128, I=128, E=4, k=2, shared=True)
    mats = [experts.dequant_expert(gen.expert_weights(sh, 0, e, 5)) for e in range(4)]
    sw = experts.dequant_expert(gen.expert_weights(sh, 0, -1, 5))
    x = gen.bf16_bits_to_f32(gen.tokens(sh, 0, 0, 3, 5))
    ids = np.array([[0, 3], [1, 2], [2, 0]])
    g = np.array([[0.6, 0.4], [0.3, 0.7], [0.5, 0.5]])
    y, flip, arith = mx.moe_layer_mx_bound(x, ids, g, lambda e: mats[e], shared=sw)
    assert np.array_equal(y, mx.moe_layer_mx(x, ids, g, lambda e: mats[e], shared=sw))
    xq = mx.quantize_mxfp8(x.astype(np.float64))
    t = 1
    f_sum = sum(g[t, j] * mx.expert_ffn_mx_bound(xq[t], *mats[ids[t, j]], h_rel=2.0 ** -16)[1]
                for j in range(2)) + mx.expert_ffn_mx_bound(xq[t], *sw, h_rel=2.0 ** -16)[1]
    assert np.allclose(flip[t], f_sum, rtol=1e-12, atol=0)
    assert np.all(arith[t] > 0)


def test_mfma_dot_err_closed_form():
    """Per 128-term chunk the largest product magnitude times 2^-10, plus 2u
    per chunk of the sum of magnitudes: on a hand-built pair of rows."""
    K = 256
    ax = np.ones((1, K))
    aw = np.full((2, K), 0.5)
    aw[0, 3] = 8.0          # chunk 0 of row 0 peaks at 8
    aw[0, 200] = 2.0        # chunk 1 of row 0 peaks at 2
    got = mx.mfma_dot_err(ax, aw)
    s0 = 0.5 * (K - 2) + 8.0 + 2.0
    assert got[0, 0] == 2.0 ** -10 * (8.0 + 2.0) + 2 * 2.0 ** -24 * 2 * s0
    assert got[0, 1] == 2.0 ** -10 * (0.5 + 0.5) + 2 * 2.0 ** -24 * 2 * (0.5 * K)
    # a ragged last chunk counts as one more instruction
    got = mx.mfma_dot_err(np.ones((1, 130)), np.ones((1, 130)))
    assert got[0, 0] == 2.0 ** -10 * 2 + 2 * 2.0 ** -24 * 2 * 130


def test_dequant_mxfp8_from_fields():
    """Codes and scale bytes written by hand from the E4M3 and E8M0 fields:
    0x38 = 1.0, 0x7E = 448, 0x01 = 2^-9, 0xC4 = -3.0 (sign, exponent 8,
    mantissa 4); scale byte 127 + e multiplies by 2^e."""
    codes = np.zeros((2, 64), np.uint8)
    codes[0, :4] = [0x38, 0x7E, 0x01, 0xC4]
    codes[1, 32:34] = [0x38, 0xC4]
    sb = np.array([[127, 127], [0, 130]], np.uint8)
    v = mx.dequant_mxfp8(codes, sb)
    assert v[0, :4].tolist() == [1.0, 448.0, 2.0 ** -9, -3.0] and np.all(v[0, 4:] == 0)
    assert v[1, 32:34].tolist() == [8.0, -24.0] and np.all(v[1, :32] == 0)
    # and the quantiser's values are the dequantisation of some codes: every
    # quantised block divided by its scale is an E4M3 value
    rng = np.random.default_rng(12)
    x = rng.standard_normal((5, 96)) * 3
    q = mx.quantize_mxfp8(x)
    t = q / np.repeat(np.ldexp(1.0, mx.block_exponents(x)), 32, axis=-1)
    assert set(np.unique(np.abs(t))) <= set(_e4m3_table())


def test_expert_h_mx_matches_the_layer():
    """expert_h_mx's h is the one expert_ffn_mx quantises (y = W_d Q(h))."""
    x, wg, wu, wd = _bound_case(256, 128, 3)
    h, dh = mx.expert_h_mx(x, wg, wu)
    assert np.array_equal(wd @ mx.quantize_mxfp8(h), mx.expert_ffn_mx(x, wg, wu, wd))
    assert np.all(dh > 0)
