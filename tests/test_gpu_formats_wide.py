"""bf16 and NVFP4 experts beyond 16 tokens per decode call (the kernels for
more than 16 rows per item) and in prefill (grouped GEMMs with h as two
bf16 planes), against the oracle; NVFP4 bit-identical to MXFP4 on equal
values on the decode kernels."""
from dataclasses import replace

import numpy as np
import pytest

from workload import gen
from tests import harness as H
from tests.test_gpu_nvfp4 import _Model, _as_nvfp4

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,T,kw", [
    ("bf16", 33, {}), ("bf16", 64, {}), ("nvfp4", 33, {}), ("nvfp4", 64, {}),
    ("bf16", 17, dict(H=4096, I=256, E=16, k=2)),      # the largest K a bf16 wave split takes
    ("nvfp4", 64, dict(H=6144, I=256, E=16, k=4)),
])
def test_decode_beyond_16_tokens(fmt, T, kw):
    base = dict(H=1024, I=512, E=64, k=6, shared=True, layers=2)
    base.update(kw)
    sh = replace(H.small_shape(**base), weights=fmt)
    wl = gen.Workload("wide", sh, Ts=(T,), steps=6, cache_slots=min(40, sh.E * sh.layers),
                      staging_slots=min(T * sh.k, sh.E), zipf_s=1.1, overlap=0.5)
    print(f"case: {fmt} decode T={T} {kw}", flush=True)
    m = H.Model(sh, seed=11)
    run = H.DecodeRun(wl, m, T=T, max_tokens=64)
    for s in range(wl.steps):
        for l in range(sh.layers):
            run.step(l, s, check_out=(s % 2 == 0), out_tokens=[0, 7, T - 1])
    run.close()


def test_nvfp4_beyond_16_tokens_equals_mxfp4():
    import torch
    sh_mx = H.small_shape(H=512, I=256, E=32, k=4, shared=True, layers=2)
    sh_nv = replace(sh_mx, weights="nvfp4")
    T = 40
    wl = gen.Workload("nv_wide", sh_mx, Ts=(T,), steps=4, cache_slots=12,
                      staging_slots=min(T * sh_mx.k, sh_mx.E), zipf_s=1.1, overlap=0.5)
    print("case: nvfp4 == mxfp4 at T=40", flush=True)
    m_mx = H.Model(sh_mx, seed=12)
    m_nv = _Model(sh_nv, 12, lambda sh, l, e, s: _as_nvfp4(
        gen.expert_weights(replace(sh, weights="mxfp4"), l, e, s)))
    a = H.DecodeRun(wl, m_mx, T=T, max_tokens=64)
    b = H.DecodeRun(replace(wl, shape=sh_nv), m_nv, T=T, max_tokens=64)
    for s in range(wl.steps):
        for l in range(sh_mx.layers):
            ya, _ = a.step(l, s)
            yb, _ = b.step(l, s)
            torch.cuda.synchronize()
            assert torch.equal(ya, yb) and torch.equal(a.y32, b.y32), f"step {s} layer {l}"
    a.close()
    b.close()


@pytest.mark.parametrize("fmt,T,kw", [
    ("bf16", 300, dict(H=512, I=256, E=32, k=4, shared=True, layers=2)),
    ("nvfp4", 300, dict(H=512, I=256, E=32, k=4, shared=True, layers=2)),
    ("bf16", 129, dict(H=384, I=256, E=16, k=2)),
    ("nvfp4", 700, dict(H=256, I=256, E=1024, k=16, shared=True)),
    ("bf16", 1, dict(H=256, I=128, E=8, k=2, shared=True)),
    ("nvfp4", 17, dict(H=256, I=128, E=8, k=2, shared=True)),
    ("bf16", 40, dict(H=4096, I=128, E=4, k=2)),
    ("bf16", 70, dict(H=6144, I=256, E=4, k=2, shared=True)),   # the largest H
    ("nvfp4", 70, dict(H=6144, I=384, E=4, k=2, shared=True)),
])
def test_prefill_other_formats(fmt, T, kw):
    """Every token of every layer: routing and permutation bit-exact,
    outputs against the oracle at the decode bar (h carried as two bf16
    planes)."""
    sh = replace(H.small_shape(**kw), weights=fmt)
    print(f"case: {fmt} prefill T={T} {kw}", flush=True)
    run = H.PrefillRun(sh, T, seed=13)
    run.run()
    for l in range(sh.layers):
        xf, ids_ref, g_ref = run.check_routing(l)
        H.check_rounding(run.ys[l], run.y32[l], f"{fmt} prefill layer {l}")
        y_ref = H.oracle_rows(run.model, l, xf, ids_ref, g_ref, list(range(T)))
        err = H.check_y(run.y32[l].cpu().numpy(), y_ref, what=f"{fmt} prefill layer {l}",
                        rtol=H.RTOL_Y_DECODE)
        print(f"  layer {l}: max err/rms {err:.2e}", flush=True)
    run.close()


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4"])
def test_prefill_a3b_shape(fmt):
    """A 35B-A3B-shaped layer pair (H=2048, I=512, E=256, top-8) at T=1024,
    sampled tokens against the oracle."""
    sh = replace(gen.WORKLOADS["a3b_decode"].shape, layers=2, weights=fmt)
    T = 1024
    print(f"case: {fmt} prefill 35B-A3B shape T={T}", flush=True)
    run = H.PrefillRun(sh, T, seed=14, model=H.Model(sh, seed=14, cache_entries=64))
    run.run()
    rng = np.random.default_rng(7)
    for l in range(sh.layers):
        xf, ids_ref, g_ref = run.check_routing(l)
        toks = sorted({0, T - 1} | set(rng.choice(T, 62, replace=False).tolist()))
        y_ref = H.oracle_rows(run.model, l, xf, ids_ref, g_ref, toks)
        err = H.check_y(run.y32[l].cpu().numpy()[toks], y_ref, what=f"{fmt} a3b prefill layer {l}",
                        rtol=H.RTOL_Y_DECODE)
        print(f"  layer {l}: max err/rms {err:.2e}", flush=True)
    run.close()
