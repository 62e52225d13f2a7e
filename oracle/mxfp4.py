"""MXFP4 weights: E2M1 elements with one E8M0 power-of-two scale per 32.

Test infrastructure (see the package docstring).

The pages name the format only ("MXFP4" for DeepSeek-V4-Flash, jansverre.net
FreeToken article, section "Hvor raskt kjører modellene?"; "FP4" in the
aiforradalom.hu article, section "A Mixture-of-Experts (MoE) kihívásai és a
FreeToken megoldásai").  The element and scale encodings are those of the OCP
Microscaling Formats (MX) v1.0 specification:

* E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit; codes 0..7 are
  0, 0.5, 1, 1.5, 2, 3, 4, 6 and codes 8..15 their negatives (8 is -0).
* E8M0: an unsigned biased exponent, value 2^(s - 127); 255 is NaN.
* A block is 32 consecutive elements along the reduction axis of a row.

Packing reading (the pages are silent): element 2i sits in the low nibble of
byte i, element 2i+1 in the high nibble.
"""
import numpy as np

#: value of each 4-bit E2M1 code, from the sign/exponent/mantissa fields
E2M1_VALUES = np.array(
    [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float32)


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """Map 4-bit codes (0..15) to their fp32 values."""
    return E2M1_VALUES[np.asarray(codes, dtype=np.uint8)]


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[rows][K/2] bytes -> [rows][K] codes, low nibble first."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[r, c] = E2M1(q[r, c]) * 2^(s[r, c // 32] - 127), exact in fp32.

    packed: [rows][K/2] uint8; scales: [rows][K/32] uint8 (E8M0, never 255).
    """
    s = np.asarray(scales, dtype=np.uint8)
    assert not np.any(s == 255), "E8M0 code 255 is NaN"
    vals = decode_e2m1(unpack_nibbles(packed))                 # [rows][K]
    rows, K = vals.shape
    assert s.shape == (rows, K // 32)
    exp = s.astype(np.int32) - 127                              # [rows][K/32]
    mult = np.ldexp(np.float32(1.0), np.repeat(exp, 32, axis=1)).astype(np.float32)
    return (vals * mult).astype(np.float32)
