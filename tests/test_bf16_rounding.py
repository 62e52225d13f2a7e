"""Pins for the fp32 -> bf16 rounding used to store synthetic activations and
to check the library's bf16 outputs (workload.gen.f32_to_bf16_bits), against
torch's own float32 -> bfloat16 conversion, which rounds to nearest with
ties to even (no GPU)."""
import numpy as np
import torch

from workload import gen


def _torch_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def test_ties_go_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: 1 + 2^-6 wins
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), -(1 + 3 * 2.0 ** -8)],
                 dtype=np.float32)
    want = np.array([0x3F80, 0x3F82, 0xBF80, 0xBF82], dtype=np.uint16)
    assert np.array_equal(gen.f32_to_bf16_bits(x), want)
    assert np.array_equal(_torch_bits(x), want)
    # just above / below the halfway point round away from / towards it
    above = _f32([0x3F808001, 0x3F817FFF])
    assert np.array_equal(gen.f32_to_bf16_bits(above), np.array([0x3F81, 0x3F81], np.uint16))


def test_special_values_match_torch():
    x = np.concatenate([
        _f32([0x00000000, 0x80000000,            # +-0
              0x00000001, 0x807FFFFF,            # fp32 subnormals
              0x00008000, 0x00018000,            # subnormal halfway cases
              0x00800000, 0x00807FFF, 0x00808000,  # smallest normal and neighbours
              0x7F7FFFFF, 0xFF7FFFFF,            # +-max finite (round to +-inf)
              0x7F7F7FFF, 0x7F7F8000,            # largest finite bf16 / halfway above it
              0x7F800000, 0xFF800000]),          # +-inf
        np.array([3.140625, -2.5, 65504.0, 1e-30, -1e30], np.float32)])
    assert np.array_equal(gen.f32_to_bf16_bits(x), _torch_bits(x))


def test_random_values_match_torch():
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(gen.f32_to_bf16_bits(x), _torch_bits(x))
    # normal activations, as the generator draws them, and every tie pattern
    y = rng.standard_normal(100_000).astype(np.float32)
    assert np.array_equal(gen.f32_to_bf16_bits(y), _torch_bits(y))
    ties = (rng.integers(0, 2 ** 16, size=50_000).astype(np.uint32) << 16) | 0x8000
    t = ties.view(np.float32)
    t = t[np.isfinite(t)]
    assert np.array_equal(gen.f32_to_bf16_bits(t), _torch_bits(t))


def test_widening_matches_torch():
    bits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = gen.bf16_bits_to_f32(bits)
    finite = np.isfinite(want)
    assert np.array_equal(got.view(np.uint32)[finite], want.view(np.uint32)[finite])
    assert np.array_equal(np.isnan(got), np.isnan(want))
