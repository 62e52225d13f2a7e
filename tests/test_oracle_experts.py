"""Pins for the oracle's expert FFN and combine (no GPU)."""
import numpy as np
import pytest
from scipy.special import expit

from oracle import experts, mxfp4, router
from workload import gen


def _dense_masked_reference(x, gate_matrix, mats, shared=None):
    """Every expert on every token as whole-batch matrix products (fp64),
    weighted by a dense [T][E] gate matrix that is zero off the selection."""
    X = x.astype(np.float64)
    Y = np.zeros((X.shape[0], mats[0][2].shape[0]))
    for e, (wg, wu, wd) in enumerate(mats):
        A = X @ wg.astype(np.float64).T
        B = X @ wu.astype(np.float64).T
        Hh = A * expit(A) * B
        Y += gate_matrix[:, e:e + 1] * (Hh @ wd.astype(np.float64).T)
    if shared is not None:
        wg, wu, wd = shared
        A = X @ wg.astype(np.float64).T
        B = X @ wu.astype(np.float64).T
        Y += (A * expit(A) * B) @ wd.astype(np.float64).T
    return Y


@pytest.mark.parametrize("seed,shared,I", [(0, False, 512), (1, False, 512), (2, True, 512),
                                           (3, True, 512), (4, True, 256)])
def test_tiny_layer_equals_dense_masked_reference(seed, shared, I):
    """I = H = 256 is the square case, where a transposed operand would not
    change the shapes."""
    shape = gen.Shape(H=256, I=I, E=8, k=2, shared=shared)
    x = gen.bf16_bits_to_f32(gen.tokens(shape, 0, 0, 4, seed))
    wr = gen.router_weights(shape, 0, seed)
    _, ids, g = router.route(x, wr, shape.k)
    mats = [experts.dequant_expert(gen.expert_weights(shape, 0, e, seed)) for e in range(shape.E)]
    sh = experts.dequant_expert(gen.expert_weights(shape, 0, -1, seed)) if shared else None
    y = experts.moe_layer(x, ids, g, lambda e: mats[e], shared=sh)
    dense = np.zeros((4, shape.E))
    for t in range(4):
        dense[t, ids[t]] = g[t]
    ref = _dense_masked_reference(x, dense, mats, sh)
    assert np.max(np.abs(y - ref)) <= 1e-10 * np.sqrt(np.mean(ref ** 2))
    # the gates in the combine matter: zeroing one selection changes y
    assert np.max(np.abs(y)) > 0


def test_zero_gate_weights_leave_only_shared():
    shape = gen.Shape(H=64, I=64, E=4, k=2, shared=True)
    x = gen.bf16_bits_to_f32(gen.tokens(shape, 0, 0, 3, 5))
    zero = np.zeros((64, 64), np.float32)
    mats = [(zero, experts.dequant_expert(gen.expert_weights(shape, 0, e, 5))[1],
             experts.dequant_expert(gen.expert_weights(shape, 0, e, 5))[2]) for e in range(4)]
    sh = experts.dequant_expert(gen.expert_weights(shape, 0, -1, 5))
    ids = np.array([[0, 1], [2, 3], [1, 2]], np.int32)
    g = np.full((3, 2), 0.5, np.float32)
    y = experts.moe_layer(x, ids, g, lambda e: mats[e], shared=sh)
    y_sh = np.stack([experts.expert_ffn(x[t], *sh) for t in range(3)])
    assert np.array_equal(y, y_sh)
    y0 = experts.moe_layer(x, ids, g, lambda e: mats[e], shared=None)
    assert np.all(y0 == 0)


def test_identity_down_projection_returns_swiglu():
    H = I = 64
    rng = np.random.default_rng(4)
    # identity W_d from code 2 (1.0) on the diagonal, code 0 elsewhere, s = 127
    codes = np.zeros((H, I), np.uint8)
    codes[np.arange(H), np.arange(I)] = 2
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    wd = mxfp4.dequant(packed, np.full((H, I // 32), 127, np.uint8))
    assert np.array_equal(wd, np.eye(H, dtype=np.float32))
    wg = (rng.standard_normal((I, H)) * 0.1).astype(np.float32)
    wu = (rng.standard_normal((I, H)) * 0.1).astype(np.float32)
    x = rng.standard_normal(H).astype(np.float32)
    a, b = wg.astype(np.float64) @ x, wu.astype(np.float64) @ x
    want = a * expit(a) * b
    got = experts.expert_ffn(x, wg, wu, wd)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15)


def test_all_ones_closed_form():
    # W_g = W_u = W_d = all ones, x = c: a = b = H c, h_i = silu(Hc) Hc, o = I h
    H = I = 32
    ones = np.ones((I, H), np.float32)
    c = 0.125
    o = experts.expert_ffn(np.full(H, c, np.float32), ones, ones, ones)
    a = H * c
    assert np.allclose(o, I * (a / (1 + np.exp(-a))) * a, rtol=1e-14)
