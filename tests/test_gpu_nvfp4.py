"""NVFP4 experts on the decode path (GPU): bit-identical to MXFP4 where the
two formats hold the same values, a decode trace against the oracle, every
E4M3 block-scale code with varied matrix scales, and the host checks of the
scale arrays."""
from dataclasses import replace

import numpy as np
import pytest

from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu


def _as_nvfp4(w: gen.ExpertWeights) -> gen.ExpertWeightsNV:
    """The same values as an MXFP4 expert: each E8M0 scale 2^x becomes two
    E4M3 block scales of 2^x (x = -8, -7 as subnormals 0x02, 0x04), matrix
    scales 1."""
    def conv(s):
        x = s.astype(np.int64) - 127
        assert x.min() >= -8 and x.max() <= 8
        code = np.where(x == -8, 0x02, np.where(x == -7, 0x04, (x + 7) << 3)).astype(np.uint8)
        return np.repeat(code, 2, axis=-1)
    one = np.float32(1.0)
    return gen.ExpertWeightsNV(qg=w.qg, qu=w.qu, qd=w.qd, sg=conv(w.sg), su=conv(w.su),
                               sd=conv(w.sd), tg=one, tu=one, td=one)


class _Model(H.Model):
    def __init__(self, shape, seed, fn):
        super().__init__(shape, seed)
        self.fn = fn

    def expert(self, layer, e):
        return self.fn(self.shape, layer, e, self.seed)


@pytest.mark.parametrize("T", [1, 16])
def test_nvfp4_equal_values_are_bit_identical_to_mxfp4(T):
    import torch
    sh_mx = H.small_shape(H=512, I=256, E=32, k=4, shared=True, layers=2)
    sh_nv = replace(sh_mx, weights="nvfp4")
    wl = gen.Workload("nv_eq", sh_mx, Ts=(T,), steps=6, cache_slots=10,
                      staging_slots=min(T * sh_mx.k, sh_mx.E), zipf_s=1.1, overlap=0.5)
    print(f"case: nvfp4 == mxfp4 on equal values, T={T}", flush=True)
    m_mx = H.Model(sh_mx, seed=9)
    m_nv = _Model(sh_nv, 9, lambda sh, l, e, s: _as_nvfp4(
        gen.expert_weights(replace(sh, weights="mxfp4"), l, e, s)))
    a = H.DecodeRun(wl, m_mx, T=T)
    b = H.DecodeRun(replace(wl, shape=sh_nv), m_nv, T=T)
    for s in range(wl.steps):
        for l in range(sh_mx.layers):
            ya, _ = a.step(l, s, check_out=(s == 0))
            yb, _ = b.step(l, s, check_out=(s == 0))
            torch.cuda.synchronize()
            assert torch.equal(ya, yb) and torch.equal(a.y32, b.y32), f"step {s} layer {l}"
    a.close()
    b.close()


@pytest.mark.parametrize("T", [1, 4, 16])
def test_nvfp4_decode_trace_against_oracle(T):
    """A 35B-A3B-like small trace (cold cache, fills and evictions) with
    NVFP4 experts: state bit-exact, outputs against the oracle."""
    sh = H.small_shape(H=1024, I=256, E=64, k=8, shared=True, layers=2)
    sh = replace(sh, weights="nvfp4")
    wl = gen.Workload("nv_trace", sh, Ts=(T,), steps=12, cache_slots=24,
                      staging_slots=min(T * sh.k, sh.E), zipf_s=1.1, overlap=0.6)
    print(f"case: nvfp4 decode trace T={T}", flush=True)
    m = H.Model(sh, seed=3)
    run = H.DecodeRun(wl, m, T=T)
    errs = []
    for s in range(wl.steps):
        for l in range(sh.layers):
            _, err = run.step(l, s, check_out=(s % 3 == 0))
            if err is not None:
                errs.append(err)
    print(f"  max err/rms {max(errs):.2e}", flush=True)
    run.close()


def test_nvfp4_every_scale_code():
    """Block scales drawn over every non-negative, non-NaN E4M3 code (zero,
    the subnormals, up to 448) and matrix scales from 2^-6 to 2^7: outputs
    against the oracle."""
    sh = replace(H.small_shape(H=512, I=256, E=8, k=2, shared=True), weights="nvfp4")
    codes = np.arange(0, 0x7F, dtype=np.uint8)

    def draw(shape, layer, e, seed):
        w = gen.expert_weights_nvfp4(shape, layer, e, seed, scale_codes=codes)
        g = np.random.default_rng(1000 + e + 17 * layer)
        t = np.exp2(g.integers(-6, 7, 3)).astype(np.float32) * np.float32(1.0 + g.random())
        return replace(w, tg=t[0], tu=t[1], td=t[2])
    T = 16
    wl = gen.Workload("nv_codes", sh, Ts=(T,), steps=4, cache_slots=sh.E,
                      staging_slots=sh.E, preload_all=True)
    print("case: nvfp4 every block-scale code", flush=True)
    m = _Model(sh, 5, draw)
    run = H.DecodeRun(wl, m, T=T)
    for s in range(wl.steps):
        run.step(0, s, check_out=True)
    run.close()


def test_nvfp4_scale_checks():
    """Negative and NaN block scales and a non-finite matrix scale are
    rejected before anything is written."""
    from expert_offload_serving_amd import MoEError
    sh = replace(H.small_shape(H=256, I=128, E=4, k=2), weights="nvfp4")
    eng = H.make_engine(sh, 4, 4, 8)
    w = gen.expert_weights_nvfp4(sh, 0, 0, 1)
    eng.set_expert(0, 0, w)
    for bad in ({"sg": np.where(np.arange(w.sg.size).reshape(w.sg.shape) == 3, 0x7F, w.sg).astype(np.uint8)},
                {"su": np.where(np.arange(w.su.size).reshape(w.su.shape) == 5, 0x90, w.su).astype(np.uint8)},
                {"td": np.float32(np.inf)}):
        with pytest.raises(MoEError) as e:
            eng.set_expert(0, 1, replace(w, **bad))
        assert e.value.name == "INVALID_ARG"
    eng.close()
