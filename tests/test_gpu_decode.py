"""Decode-path parity: the HIP library against the CPU oracle (GPU)."""
import numpy as np
import pytest

from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def test_tiny_layer_full_parity():
    wl = gen.WORKLOADS["tiny"]
    _flush("case: tiny T=4 seed 0")
    m = H.Model(wl.shape)
    run = H.DecodeRun(wl, m, T=4)
    run.step(0, 0, check_out=True)
    # resident slot of expert e is e after the preload
    key, stamp, clock = run.eng.cache_snapshot()
    assert sorted(key.tolist()) == list(range(8))
    run.close()


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5, 6, 7, 8, 9])
def test_tiny_layer_seeds(seed):
    wl = gen.WORKLOADS["tiny"]
    _flush(f"case: tiny T=4 seed {seed}")
    m = H.Model(wl.shape, seed=seed)
    run = H.DecodeRun(wl, m, T=4)
    run.step(0, 0, check_out=True)
    run.close()


@pytest.mark.parametrize("T", [1, 4, 16])
def test_a3b_decode_trace(T):
    """35B-A3B-shaped layer, 64-slot LRU from cold, Zipf(1.1) trace with 60%
    overlap, 512 steps: ids, gates, permutation, slots and cache state every
    step; outputs every 32nd step (all tokens)."""
    wl = gen.WORKLOADS["a3b_decode"]
    _flush(f"case: a3b_decode T={T}")
    m = H.Model(wl.shape)
    run = H.DecodeRun(wl, m, T=T)
    errs = []
    for s in range(wl.steps):
        _, err = run.step(0, s, check_out=(s % 32 == 0 or s == wl.steps - 1))
        if err is not None:
            errs.append(err)
    st = run.eng.stats()
    assert st["hits"] + st["fills"] + st["bypasses"] == st["lookups"]
    assert st["hits"] == run.cache.hits and st["fills"] == run.cache.fills
    assert st["bypasses"] == run.cache.bypasses and st["evictions"] == run.cache.evictions
    _flush(f"a3b T={T}: hit rate {st['hits'] / st['lookups']:.3f}, max err/rms {max(errs):.2e}")
    run.close()


def test_outputs_independent_of_cache_capacity():
    """Offloading is exact: the same inputs give bit-identical outputs with
    a large cache, a small cache and no cache at all (all misses bypass)."""
    import torch
    wl = gen.WORKLOADS["a3b_decode"]
    m = H.Model(wl.shape)
    T = 16
    outs = {}
    for C, S in ((256, 0), (64, 128), (1, 128), (0, 128)):
        _flush(f"case: capacity {C}")
        run = H.DecodeRun(wl, m, T=T, cache_slots=C, staging_slots=S, steps=24)
        ys = []
        for s in range(24):
            y, _ = run.step(0, s, check_out=False, check_state=(s % 6 == 0))
            ys.append(y.clone())
        torch.cuda.synchronize()
        outs[C] = torch.stack(ys).cpu().numpy()
        run.close()
    for C in (64, 1, 0):
        assert np.array_equal(outs[C], outs[256]), f"capacity {C} changed the outputs"


@pytest.mark.parametrize("T", [0, 1, 7, 13, 64])
def test_ragged_token_counts(T):
    import torch
    sh = H.small_shape(E=32, k=4)
    wl = gen.Workload("small", sh, Ts=(T,), steps=3, cache_slots=12, staging_slots=64)
    _flush(f"case: ragged T={T}")
    m = H.Model(sh, seed=11)
    run = H.DecodeRun(wl, m, T=max(T, 1), max_tokens=64)
    if T == 0:
        x = torch.empty((0, sh.H), dtype=torch.int16, device="cuda")
        run.eng.forward(0, x)
        key, stamp, clock = run.eng.cache_snapshot()
        assert clock == 0 and (key == -1).all()
    else:
        for s in range(3):
            run.step(0, s, check_out=True)
    run.close()


@pytest.mark.parametrize("kw", [dict(k=1), dict(E=64, k=16), dict(E=200, k=6), dict(renormalize=False),
                                dict(shared=True), dict(H=384, I=128), dict(H=128, I=128, E=4, k=2),
                                dict(layers=3, E=16, k=3),
                                # split of K in the expert kernels: down with 4 chunks per
                                # wave (K = 24 chunks), gate/up with 16 chunks per wave and
                                # a last wave past K (36 chunks), odd chunk counts (9 and 5)
                                dict(H=256, I=3072, E=4, k=2), dict(H=4608, I=128, E=4, k=2),
                                dict(H=1152, I=640, E=8, k=2)])
def test_shape_variants(kw):
    sh = H.small_shape(**kw)
    T = 9
    wl = gen.Workload("variant", sh, Ts=(T,), steps=2, cache_slots=min(5, sh.layers * sh.E),
                      staging_slots=T * sh.k)
    _flush(f"case: variant {kw}")
    m = H.Model(sh, seed=3)
    run = H.DecodeRun(wl, m, T=T)
    for s in range(2):
        for l in range(sh.layers):
            run.step(l, s, check_out=True)
    run.close()


def test_all_bypass_and_capacity_error():
    sh = H.small_shape(E=16, k=4)
    wl = gen.Workload("bypass", sh, Ts=(8,), steps=2, cache_slots=0, staging_slots=16)
    m = H.Model(sh, seed=5)
    run = H.DecodeRun(wl, m, T=8)
    for s in range(2):
        run.step(0, s, check_out=True)
    st = run.eng.stats()
    assert st["hits"] == 0 and st["fills"] == 0 and st["bypasses"] == st["lookups"] > 0
    run.close()
    from expert_offload_serving_amd import MoEError
    import torch
    eng = H.make_engine(sh, max_tokens=8, cache_slots=2, staging_slots=3)
    m.load(eng)
    x = H.bf16_dev(gen.tokens(sh, 0, 0, 8))
    with pytest.raises(MoEError) as ei:
        eng.forward(0, x)
    assert ei.value.name == "CAPACITY"
    with pytest.raises(MoEError) as ei:
        eng.forward(1, x)
    assert ei.value.name == "INVALID_ARG"
    y = eng.forward(0, x[:1])          # T=1 fits: worst case bypass 2
    torch.cuda.synchronize()
    eng.close()


def test_cache_lookup_and_fill_api():
    import torch
    sh = H.small_shape(E=16, k=4, layers=2)
    m = H.Model(sh, seed=2)
    eng = H.make_engine(sh, max_tokens=4, cache_slots=6, staging_slots=16)
    m.load(eng)
    import oracle
    ref = oracle.SlotCache(6, sh.E)
    rng = np.random.default_rng(0)
    for it in range(40):
        layer = int(rng.integers(0, 2))
        n = int(rng.integers(0, 12))
        U = sorted(rng.choice(sh.E, n, replace=False).tolist())
        if it % 2:
            eng.cache_fill(layer, U)
            ref.fill(layer, U)
        else:
            d_ids = torch.tensor(U + [0], dtype=torch.int32, device="cuda")
            d_n = torch.tensor([n], dtype=torch.int32, device="cuda")
            d_slot = torch.full((max(n, 1),), 12345, dtype=torch.int32, device="cuda")
            eng.cache_lookup(layer, d_ids, d_n, d_slot)
            slots, _, _ = ref.lookup(layer, U)
            assert d_slot[:n].cpu().tolist() == slots
        key, stamp, clock = eng.cache_snapshot()
        k_ref, s_ref, c_ref = ref.snapshot()
        assert key.tolist() == k_ref and stamp.tolist() == s_ref and clock == c_ref
    from expert_offload_serving_amd import MoEError
    for bad in ([3, 2], [1, 1], [16], [-1]):
        with pytest.raises(MoEError):
            eng.cache_fill(0, bad)
    # a device-side list that breaks the order: the ascending prefix is
    # looked up, every entry from the first break on is rejected (INT_MIN)
    # and changes nothing
    int_min = -2 ** 31
    for U in ([4, 4, 9], [7, 2, 11], [1, 5, 5, 6], [3, 16, 2], [0, 17, 18]):
        d_ids = torch.tensor(U, dtype=torch.int32, device="cuda")
        d_n = torch.tensor([len(U)], dtype=torch.int32, device="cuda")
        d_slot = torch.full((len(U),), 12345, dtype=torch.int32, device="cuda")
        eng.cache_lookup(1, d_ids, d_n, d_slot)
        first_bad = next((u for u in range(1, len(U)) if U[u] <= U[u - 1]), len(U))
        ok = [u for u in range(first_bad) if 0 <= U[u] < sh.E]
        slots, _, _ = ref.lookup(1, [U[u] for u in ok])
        want = [int_min] * len(U)
        for u, sl in zip(ok, slots):
            want[u] = sl
        assert d_slot.cpu().tolist() == want, (U, d_slot.cpu().tolist(), want)
        key, stamp, clock = eng.cache_snapshot()
        k_ref, s_ref, c_ref = ref.snapshot()
        assert key.tolist() == k_ref and stamp.tolist() == s_ref and clock == c_ref, U
    eng.close()
