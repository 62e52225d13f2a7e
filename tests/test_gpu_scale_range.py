"""Parity over the whole E8M0 scale range (GPU).

The other tests draw scale bytes from 119..123.  Here they span 0..250, so
the FP4 -> bf16 convert produces weights from bf16's subnormal range
(0.5 * 2^-127) up to 6 * 2^123, and the scaled fp6 x fp4 MFMA of the prefill
down GEMM sees the same scale bytes.  Inputs are laid out so that every
block's contribution is visible in the checked outputs:

- gate/up: the scale of K block b is centred on e_b (0..250 across the
  blocks), and the activations of that block carry 2^(125 - e_b), so every
  block contributes O(1) to each dot product (activations run from bf16's
  subnormal range up to ~2^126);
- down: the scale of output row r is centred on e_r, and each output column
  is checked against its own RMS.  fp32 cannot hold both ends of 0..250 in
  one product with a fixed h, so the range is split: rows over 0..125 with
  activations scaled to make h ~ 2^50, rows over 125..250 with h ~ 2^-18.

The router matrix is zero and a bias with distinct values on a drawn set
forces the routing (logits equal the bias exactly).
"""
import numpy as np
import pytest

from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu

SHAPE = gen.Shape(H=2048, I=512, E=8, k=2, shared=True)


class ScaledModel(H.Model):
    def __init__(self, shape, seed, gu=None, dn=None):
        super().__init__(shape, seed, cache_entries=shape.E + 1)
        self.routers = [np.zeros((shape.H, shape.E), np.float32) for _ in range(shape.layers)]
        self.gu, self.dn = gu, dn

    def expert(self, layer, e):
        return gen.expert_weights_scaled(self.shape, layer, e, self.seed, self.gu, self.dn)


def _bias(E, k, T, seed):
    rng = np.random.default_rng(seed)
    b = np.zeros((T, E), np.float32)
    for t in range(T):
        sel = rng.choice(E, k, replace=False)
        b[t, sel] = 32.0 + rng.uniform(-1.0, 1.0, k).astype(np.float32)
    return b


def _cases():
    nb, Hh = SHAPE.H // 32, SHAPE.H
    gu = np.rint(np.arange(nb) * 250 / (nb - 1)).astype(np.int64)
    lo = np.rint(np.arange(Hh) * 125 / (Hh - 1)).astype(np.int64)
    hi = 125 + np.rint(np.arange(Hh) * 125 / (Hh - 1)).astype(np.int64)
    return {
        # name: (gate/up block centres, down row centres, activation block shifts)
        "gateup_0_250": (gu, None, 125 - gu),
        "down_0_125": (None, lo, np.full(nb, 24)),
        "down_125_250": (None, hi, np.full(nb, -10)),
    }


def _check_columns(y, y_ref, rtol, what):
    """Each output column against its own RMS over the tokens."""
    y_ref = y_ref.astype(np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2, axis=0))
    assert np.all(np.isfinite(y)) and np.all(rms > 0), what
    err = np.max(np.abs(y.astype(np.float64) - y_ref), axis=0) / rms
    worst = int(np.argmax(err))
    assert err[worst] <= rtol, f"{what}: column {worst} err {err[worst]:.3g} x its rms"
    return float(err.max())


@pytest.mark.parametrize("case", list(_cases()))
def test_decode_scale_range(case):
    import torch
    gu, dn, shift = _cases()[case]
    T = 16
    print(f"case: decode scale range {case} T={T}", flush=True)
    m = ScaledModel(SHAPE, seed=31, gu=gu, dn=dn)
    wl = gen.Workload("scales", SHAPE, Ts=(T,), steps=2, cache_slots=SHAPE.E,
                      staging_slots=SHAPE.E, preload_all=True)
    eng = H.make_engine(SHAPE, T, wl.cache_slots, wl.staging_slots)
    m.load(eng)
    eng.cache_fill(0, list(range(SHAPE.E)))
    dev = torch.device("cuda")
    ids = torch.empty((T, SHAPE.k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, SHAPE.k), dtype=torch.float32, device=dev)
    y32 = torch.empty((T, SHAPE.H), dtype=torch.float32, device=dev)
    for step in range(2):
        xb = gen.tokens_block_scaled(SHAPE, 0, step, T, shift, m.seed)
        bias = _bias(SHAPE.E, SHAPE.k, T, 100 + step)
        y = eng.forward(0, H.bf16_dev(xb), bias=torch.from_numpy(bias).to(dev), ids=ids,
                        gates=gates, y32=y32)
        xf = gen.bf16_bits_to_f32(xb)
        _, ids_ref, g_ref = m.route(0, xf, bias)
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        assert np.max(np.abs(gates.cpu().numpy() - g_ref)) <= H.ATOL_G
        H.check_rounding(y, y32, f"{case} step {step}")
        y_ref = m.layer_out(0, xf, ids_ref, g_ref)
        got = y32.cpu().numpy()
        if dn is None:
            err = H.check_y(got, y_ref, what=f"{case} step {step}", rtol=H.RTOL_Y_DECODE)
        else:
            err = _check_columns(got, y_ref, H.RTOL_Y_DECODE, f"{case} step {step}")
        print(f"  step {step}: max err/rms {err:.3e}", flush=True)
    eng.close()


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8"])
@pytest.mark.parametrize("case", list(_cases()))
def test_prefill_scale_range(case, fmt):
    """Both prefill modes; the MXFP8 mode is compared with its own oracle
    (activations quantised by the stated rule) element by element within that
    oracle's allowance, so that every weight scale byte is still checked."""
    import oracle.mx
    gu, dn, shift = _cases()[case]
    T = 96
    print(f"case: prefill scale range {case} T={T} {fmt}", flush=True)
    m = ScaledModel(SHAPE, seed=32, gu=gu, dn=dn)
    bias = _bias(SHAPE.E, SHAPE.k, T, 200)
    run = H.PrefillRun(SHAPE, T, seed=32, model=m, bias_sets=[bias], prefill_format=fmt)
    run.xb = [gen.tokens_block_scaled(SHAPE, 0, 0, T, shift, m.seed)]
    run.xs = [H.bf16_dev(run.xb[0])]
    run.run()
    xf, ids_ref, g_ref = run.check_routing(0)
    H.check_rounding(run.ys[0], run.y32[0], f"prefill {case}")
    got = run.y32[0].cpu().numpy()
    if fmt == "mxfp8":
        ref = H.oracle_rows(m, 0, xf, ids_ref, g_ref, list(range(T)),
                            layer_fn=oracle.mx.moe_layer_mx_bound)
        err, _, _ = H.check_y_mx(got, ref, what=f"prefill {case} {fmt}")
        share, _ = H.check_mx_decisions(run, what=f"prefill {case} {fmt}")
        print(f"  h codes off the oracle's choice: {share:.3%}", flush=True)
    else:
        y_ref = H.oracle_rows(m, 0, xf, ids_ref, g_ref, list(range(T)))
        if dn is None:
            err = H.check_y(got, y_ref, what=f"prefill {case} {fmt}", rtol=H.RTOL_Y_PREFILL)
        else:
            err = _check_columns(got, y_ref, H.RTOL_Y_PREFILL, f"prefill {case} {fmt}")
    print(f"  max err/rms {err:.3e}", flush=True)
    run.close()
