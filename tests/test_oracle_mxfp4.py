"""Pins for the oracle's MXFP4 dequantisation (no GPU)."""
import math
import os

import numpy as np

from oracle import mxfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_ocp_mx_v1.txt")


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, sign, exp, man, val = line.split()
            rows.append((int(code, 16), int(sign), int(exp, 2), int(man), float(val)))
    return rows


def test_e2m1_table_matches_spec_fixture():
    rows = _golden_rows()
    assert len(rows) == 16
    for code, sign, exp, man, val in rows:
        got = float(mxfp4.decode_e2m1(np.array([code]))[0])
        assert got == val and math.copysign(1.0, got) == math.copysign(1.0, val), code
        # the code's own bit fields agree with the fixture's columns
        assert sign == code >> 3 and exp == (code >> 1) & 3 and man == code & 1


def test_e2m1_table_matches_bitfield_closed_form():
    # value = (-1)^s * 2^(e-1) * (1 + m/2) for e > 0, (-1)^s * m/2 for e = 0
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = (m * 0.5) if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
        want = -mag if s else mag
        got = float(mxfp4.decode_e2m1(np.array([code]))[0])
        assert got == want


def test_nibble_order_low_first():
    codes = np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8)
    packed = np.array([[1 | (2 << 4), 3 | (4 << 4), 15 | (0 << 4)]], dtype=np.uint8)
    assert np.array_equal(mxfp4.unpack_nibbles(packed), codes)


def test_dequant_all_codes_all_scales():
    # every code at every C1 scale exponent, against ldexp in Python floats
    for s in (119, 120, 121, 122, 123, 1, 127, 200):
        codes = np.arange(32, dtype=np.uint8) % 16
        packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
        w = mxfp4.dequant(packed, np.array([[s]], dtype=np.uint8))
        for c in range(32):
            code = int(codes[c])
            sgn = -1.0 if code & 8 else 1.0
            e, m = (code >> 1) & 3, code & 1
            mag = (m * 0.5) if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
            assert float(w[0, c]) == math.ldexp(sgn * mag, s - 127)


def test_dequant_constant_block():
    packed = np.full((1, 16), 0x22, dtype=np.uint8)     # code 2 (=1.0) everywhere
    w = mxfp4.dequant(packed, np.array([[123]], dtype=np.uint8))
    assert np.all(w == np.float32(2.0 ** -4))


def test_dequant_block_boundary_and_rows():
    # 2 rows x 64 elements: each (row, block) gets its own scale; element 31
    # and 32 of a row must use different blocks, rows must not mix.
    packed = np.full((2, 32), 0x22, dtype=np.uint8)
    scales = np.array([[120, 124], [110, 130]], dtype=np.uint8)
    w = mxfp4.dequant(packed, scales)
    assert w[0, 31] == 2.0 ** (120 - 127) and w[0, 32] == 2.0 ** (124 - 127)
    assert w[1, 0] == 2.0 ** (110 - 127) and w[1, 63] == 2.0 ** (130 - 127)
