"""Cache placement policies (global LRU, per-layer shares, static set) on the
GPU against the oracle's cache model: slots and the whole cache state after
every call, counters, and outputs that do not depend on the placement."""
from dataclasses import replace

import numpy as np
import pytest

from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu

POLICIES = ("global", "per_layer", "static")


def _workload(T, C):
    # 3 layers of 64 experts, top-4, Zipf(1.1) traces with 50% step overlap;
    # staging covers every miss of a call (the static policy bypasses them all)
    base = gen.WORKLOADS["dsv4_decode"]
    sh = H.small_shape(H=256, I=256, E=64, k=4, layers=3, shared=True)
    return replace(base, name="policy", shape=sh, Ts=(T,), steps=40, cache_slots=C,
                   staging_slots=min(T * sh.k, sh.E))


def _preload_popular(run, per_layer):
    """The static set: each layer's per_layer most popular experts, placed by
    fills of at most T*k experts (the most one call may name)."""
    sh = run.wl.shape
    step = run.T * sh.k
    for l in range(sh.layers):
        top = sorted(gen.popularity_order(sh, l, run.model.seed)[:per_layer].tolist())
        for i in range(0, len(top), step):
            run.preload(l, top[i:i + step])


@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("T,C", [(1, 24), (8, 24), (8, 7)])
def test_policy_trace(policy, T, C):
    wl = _workload(T, C)
    sh = wl.shape
    print(f"case: policy {policy} T={T} C={C}", flush=True)
    m = H.Model(sh, seed=11)
    run = H.DecodeRun(wl, m, T=T, cache_policy=policy)
    if policy == "static":
        _preload_popular(run, C // sh.layers)
    for s in range(wl.steps):
        for l in range(sh.layers):
            run.step(l, s, check_out=(s % 13 == 0 and l == 1))
    st = run.eng.stats()
    c = run.cache
    assert (st["hits"], st["fills"], st["bypasses"], st["evictions"]) == \
        (c.hits, c.fills, c.bypasses, c.evictions)
    if policy == "static":
        assert st["fills"] == C // sh.layers * sh.layers  # the preload only
    print(f"policy {policy} T={T} C={C}: hit rate {st['hits'] / st['lookups']:.3f}", flush=True)
    run.close()


def test_outputs_do_not_depend_on_the_policy():
    import torch
    wl = _workload(8, 24)
    m = H.Model(wl.shape, seed=12)
    outs = {}
    for policy in POLICIES:
        print(f"case: outputs under {policy}", flush=True)
        run = H.DecodeRun(wl, m, T=8, cache_policy=policy)
        if policy == "static":
            _preload_popular(run, 8)
        ys = []
        for s in range(12):
            for l in range(wl.shape.layers):
                y, _ = run.step(l, s, check_state=False)
                ys.append(y.clone())
        torch.cuda.synchronize()
        outs[policy] = torch.stack(ys).cpu().numpy()
        run.close()
    for policy in POLICIES[1:]:
        assert np.array_equal(outs[policy], outs["global"]), f"{policy} changed the outputs"


def test_resize_is_global_only():
    from expert_offload_serving_amd import binding
    wl = _workload(1, 24)
    for policy in ("per_layer", "static"):
        eng = H.make_engine(wl.shape, 1, 24, 4, cache_policy=policy)
        with pytest.raises(binding.MoEError) as ei:
            eng.cache_resize(12)
        assert ei.value.status == -6  # UNSUPPORTED
        eng.close()
