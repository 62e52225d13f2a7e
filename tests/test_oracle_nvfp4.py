"""Pins for the oracle's NVFP4 weights (no GPU)."""
import numpy as np
import pytest

from oracle import experts, mxfp4, nvfp4
from workload import gen


def test_e4m3_decoding_matches_torch_float8():
    """Every E4M3 code against torch's float8_e4m3fn conversion (a library
    decoding of the same encoding), NaN codes included."""
    import torch
    c = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = nvfp4.e4m3_values(c)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])


def test_block_of_16_and_matrix_scale():
    """Codes all 1.0 (code 2): each row reads back its block scales, each
    repeated over exactly 16 elements, times the matrix scale."""
    rng = np.random.default_rng(1)
    rows, K = 3, 64
    packed = np.full((rows, K // 2), 0x22, dtype=np.uint8)
    sc = rng.choice(gen.NV_SCALE_CODES, size=(rows, K // 16))
    t = np.float32(0.3125)
    w = nvfp4.dequant(packed, sc, t)
    s_vals = nvfp4.e4m3_values(sc)
    for r in range(rows):
        for k in range(K):
            assert w[r, k] == s_vals[r, k // 16] * 0.3125
    # the matrix scale enters as its fp32 value
    w2 = nvfp4.dequant(packed, sc, 0.1)
    assert np.array_equal(w2, nvfp4.e4m3_values(sc).repeat(16, axis=1) * float(np.float32(0.1)))


def test_power_of_two_scales_reduce_to_mxfp4():
    """Block scales that are powers of two, equal over each pair of blocks,
    with matrix scale 1, give exactly the MXFP4 matrix with E8M0 scales of
    the same exponents (the E2M1 decoding and nibble order are MXFP4's)."""
    rng = np.random.default_rng(2)
    rows, K = 5, 128
    packed = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    exps = rng.integers(-6, 2, size=(rows, K // 32))            # 2^-6 .. 2^1
    e8m0 = (exps + 127).astype(np.uint8)
    e4m3 = ((exps + 7) << 3).astype(np.uint8)                    # mantissa 0
    nv_scales = np.repeat(e4m3, 2, axis=1)
    assert np.array_equal(nvfp4.dequant(packed, nv_scales, 1.0),
                          mxfp4.dequant(packed, e8m0).astype(np.float64))


def test_mantissa_scales_are_exact_products():
    """Scales with mantissa bits: each element is the exact product of its
    E2M1 value, the block's E4M3 value and the matrix scale (brute force
    over every code pair on a small matrix)."""
    codes = np.arange(16, dtype=np.uint8)
    rows = []
    for sc in (0x01, 0x07, 0x0F, 0x1D, 0x33, 0x3F, 0x45, 0x7E):
        row = np.repeat(codes, 2)[::2]                            # 16 codes
        packed = (row[0::2] | (row[1::2] << 4)).astype(np.uint8)  # [8]
        rows.append((packed, sc))
    t = np.float32(0.7)
    for packed, sc in rows:
        w = nvfp4.dequant(packed[None, :], np.array([[sc]], np.uint8), t)[0]
        for i in range(16):
            want = float(mxfp4.E2M1_VALUES[i]) * nvfp4.e4m3_values(np.array([sc]))[0] * float(t)
            assert w[i] == want


def test_expert_dequant_uses_each_matrix_scale():
    sh = gen.Shape(H=256, I=128, E=2, k=1, weights="nvfp4")
    w = gen.expert_weights_nvfp4(sh, 0, 1, 3)
    wg, wu, wd = experts.dequant_expert(w)
    assert wg.shape == (128, 256) and wd.shape == (256, 128)
    assert np.array_equal(wg, nvfp4.dequant(w.qg, w.sg, w.tg))
    assert np.array_equal(wu, nvfp4.dequant(w.qu, w.su, w.tu))
    assert np.array_equal(wd, nvfp4.dequant(w.qd, w.sd, w.td))
    assert w.tg != w.tu or w.tu != w.td
