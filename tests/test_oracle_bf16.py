"""Pins for the oracle's bf16 experts (no GPU): the bit-pattern decoding, and
agreement with the MXFP4 path on an expert whose values both formats hold
exactly (E2M1 times a power of two has at most two significant bits)."""
import numpy as np

from oracle import experts as oexp
from workload import gen


def test_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC020, 0x0001, 0x7F7F, 0x8000, 0x0000, 0x4049], dtype=np.uint16)
    v = oexp.bf16_values(bits)
    assert v[0] == 1.0 and v[1] == -2.5
    assert v[2] == np.float32(2.0 ** -133)                    # smallest subnormal bf16
    assert v[3] == np.float32((2 - 2.0 ** -7) * 2.0 ** 127)   # largest finite bf16
    assert v[4] == 0.0 and np.signbit(v[4]) and v[5] == 0.0 and not np.signbit(v[5])
    assert v[6] == np.float32(3.140625)


def _as_bf16_expert(mats):
    out = []
    for m in mats:
        u = np.ascontiguousarray(m, dtype=np.float32).view(np.uint32)
        assert np.all(u & 0xFFFF == 0)  # exact in bf16
        out.append((u >> 16).astype(np.uint16))
    return gen.ExpertWeightsBF16(*out)


def test_bf16_path_matches_mxfp4_on_shared_values():
    sh = gen.Shape(H=256, I=128, E=4, k=2)
    rng = np.random.default_rng(3)
    x = gen.bf16_bits_to_f32(gen.tokens(sh, 0, 0, 5))
    for e in range(3):
        w4 = gen.expert_weights(sh, 0, e)
        m4 = oexp.dequant_expert(w4)
        m16 = oexp.dequant_expert(_as_bf16_expert(m4))
        for a, b in zip(m4, m16):
            assert np.array_equal(a, b)
        ids = rng.integers(0, 3, size=(5, 2))
        ids[:, 1] = (ids[:, 0] + 1) % 3
        g = rng.random((5, 2))
        mats4 = {i: oexp.dequant_expert(gen.expert_weights(sh, 0, i)) for i in range(3)}
        mats16 = {i: oexp.dequant_expert(_as_bf16_expert(mats4[i])) for i in range(3)}
        y4 = oexp.moe_layer(x, ids, g, lambda i: mats4[i])
        y16 = oexp.moe_layer(x, ids, g, lambda i: mats16[i])
        assert np.array_equal(y4, y16)


def test_bf16_generator():
    sh = gen.Shape(H=512, I=256, E=4, k=2, weights="bf16")
    w = gen.expert_weights_bf16(sh, 1, 2)
    assert w.wg.shape == (256, 512) and w.wd.shape == (512, 256) and w.wg.dtype == np.uint16
    assert np.array_equal(w.wu, gen.expert_weights_bf16(sh, 1, 2).wu)        # seeded
    assert not np.array_equal(w.wg, gen.expert_weights_bf16(sh, 1, 3).wg)
    sd = float(np.std(oexp.bf16_values(w.wg)))
    assert abs(sd - 2.0 ** -5) < 0.05 * 2.0 ** -5
    assert sh.expert_bytes() == 3 * 512 * 256 * 2
    assert isinstance(gen.expert_weights_of(sh, 0, 0), gen.ExpertWeightsBF16)
