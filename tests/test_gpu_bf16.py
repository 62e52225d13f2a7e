"""bf16 experts on the decode path (GPU): against the oracle, and bit for bit
against MXFP4 contexts whose experts hold the same values."""
from dataclasses import replace

import numpy as np
import pytest

from oracle import experts as oexp
from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu


def _bf16_of(w4):
    """The MXFP4 expert's values as a bf16 expert (exact: E2M1 times a power
    of two has at most two significant bits)."""
    mats = []
    for m in oexp.dequant_expert(w4):
        u = np.ascontiguousarray(m, dtype=np.float32).view(np.uint32)
        assert np.all(u & 0xFFFF == 0)
        mats.append((u >> 16).astype(np.uint16))
    return gen.ExpertWeightsBF16(*mats)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_bf16_equals_mxfp4_on_the_same_values(T):
    import torch
    sh4 = H.small_shape(H=512, I=384, E=16, k=4, layers=2, shared=True)
    sh16 = replace(sh4, weights="bf16")
    print(f"case: bf16 vs mxfp4 T={T}", flush=True)
    engs = {}
    for name, sh in (("mxfp4", sh4), ("bf16", sh16)):
        eng = H.make_engine(sh, T, cache_slots=12, staging_slots=min(T * sh.k, sh.E))
        for l in range(sh.layers):
            eng.set_router(l, gen.router_weights(sh, l, 3))
            for e in list(range(sh.E)) + [-1]:
                w4 = gen.expert_weights(sh4, l, e, 3)
                eng.set_expert(l, e, w4 if name == "mxfp4" else _bf16_of(w4))
        engs[name] = eng
    y32 = {n: torch.empty((T, sh4.H), dtype=torch.float32, device="cuda") for n in engs}
    for s in range(6):
        for l in range(sh4.layers):
            x = H.bf16_dev(gen.tokens(sh4, l, s, T, 3))
            ys = {n: engs[n].forward(l, x, y32=y32[n]) for n in engs}
            torch.cuda.synchronize()
            assert torch.equal(y32["mxfp4"], y32["bf16"]), f"step {s} layer {l}"
            assert torch.equal(ys["mxfp4"], ys["bf16"])
    for eng in engs.values():
        eng.close()


@pytest.mark.parametrize("T", [1, 16])
def test_bf16_a3b_trace(T):
    """35B-A3B-shaped layer with bf16 experts (the pages' format for that
    model), 64-slot LRU from cold, Zipf trace: routing, permutation, slots and
    cache state every step; outputs against the oracle every 16th step."""
    base = gen.WORKLOADS["a3b_decode"]
    wl = replace(base, shape=replace(base.shape, weights="bf16"), steps=48)
    print(f"case: bf16 a3b T={T}", flush=True)
    m = H.Model(wl.shape, cache_entries=64)
    run = H.DecodeRun(wl, m, T=T)
    errs = []
    for s in range(wl.steps):
        _, err = run.step(0, s, check_out=(s % 16 == 0))
        if err is not None:
            errs.append(err)
    st = run.eng.stats()
    assert st["hits"] == run.cache.hits and st["fills"] == run.cache.fills
    assert st["bytes_h2d"] == (st["fills"] + st["bypasses"]) * wl.shape.expert_bytes()
    print(f"bf16 a3b T={T}: hit rate {st['hits'] / st['lookups']:.3f}, max err/rms {max(errs):.2e}",
          flush=True)
    run.close()


@pytest.mark.parametrize("kw", [dict(H=256, I=3072, E=4, k=2), dict(H=4608, I=128, E=4, k=2),
                                dict(H=1152, I=640, E=8, k=2, shared=True)])
def test_bf16_shape_variants(kw):
    """K of 2 to 36 chunks in either kernel (one to eight waves, one to
    eight chunks per wave)."""
    sh = H.small_shape(weights="bf16", **kw)
    wl = replace(gen.WORKLOADS["tiny"], shape=sh, cache_slots=sh.E, staging_slots=8,
                 preload_all=True)
    print(f"case: bf16 shape {kw}", flush=True)
    m = H.Model(sh, seed=5)
    run = H.DecodeRun(wl, m, T=4)
    run.step(0, 0, check_out=True)
    run.close()


def test_bf16_limits():
    from expert_offload_serving_amd import binding
    sh = H.small_shape(weights="bf16")
    big = H.small_shape(H=6144, I=256, weights="bf16")
    # above 16 tokens per decode call, bf16 experts need H, I <= 4096
    with pytest.raises(binding.MoEError) as ei:
        H.make_engine(big, 17, 8, 8)
    assert ei.value.status == -6  # UNSUPPORTED
    H.make_engine(sh, 17, 8, 64).close()
    H.make_engine(big, 4, 8, 8, max_prefill_tokens=64).close()   # prefill: any size
    eng = H.make_engine(sh, 4, 8, 8)
    w4 = gen.expert_weights(H.small_shape(), 0, 0)
    w = gen.expert_weights_bf16(sh, 0, 0)
    with pytest.raises(binding.MoEError) as ei:  # scale arrays with bf16 weights
        binding.moe_set_expert(eng.ctx, 0, 0, w.wg, w.wu, w.wd, w4.sg, w4.su, w4.sd)
    assert ei.value.status == -1
    eng.close()
