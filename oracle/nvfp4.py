"""NVFP4 weights: E2M1 elements, one E4M3 scale per 16 consecutive elements
along K, and one fp32 scale per matrix.

Test infrastructure (see the package docstring).

The pages run the 35B-A3B model in NVFP4 on a laptop GPU (jansverre.net
FreeToken article, section "Hvor raskt kjører modellene?") without spelling
the format out.  This is NVIDIA's published NVFP4 definition:

* elements are E2M1 codes, packed as in MXFP4 (oracle.mxfp4: element 2i in
  the low nibble of byte i);
* each block of 16 consecutive elements of a row has a scale stored as an
  8-bit E4M3 value (sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
  subnormals m/8 * 2^-6, 0x7F and 0xFF NaN); block scales are non-negative;
* each matrix has one fp32 scale;
* an element's value is e2m1(code) * e4m3(block scale) * matrix scale.

Every value is exact in fp64 (2 + 4 + 24 significant bits).
"""
import numpy as np

from .mxfp4 import decode_e2m1, unpack_nibbles

BLOCK = 16


def e4m3_values(codes: np.ndarray) -> np.ndarray:
    """fp64 value of each E4M3 code, from its sign, exponent and mantissa
    fields; NaN for 0x7F and 0xFF."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    v = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def dequant(packed: np.ndarray, scales: np.ndarray, matrix_scale) -> np.ndarray:
    """[rows][K/2] codes, [rows][K/16] E4M3 scale bytes and the matrix's
    fp32 scale -> [rows][K] fp64 values."""
    vals = decode_e2m1(unpack_nibbles(packed)).astype(np.float64)
    s = np.repeat(e4m3_values(scales), BLOCK, axis=-1)
    return vals * s * float(np.float32(matrix_scale))
