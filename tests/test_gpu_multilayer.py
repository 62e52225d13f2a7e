"""Multi-layer decode with a global LRU, the shared expert and elastic
resize: the HIP library against the CPU oracle (GPU)."""
import numpy as np
import pytest

from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("T", [1, 32])
def test_dsv4_decode_trace(T):
    """DeepSeek-V4-Flash-shaped decode: 4 layers, top-6 + shared expert, one
    global LRU of 256 slots over all layers, 512 steps.  Routing, permutation,
    slot codes and cache state are compared on every layer of every step;
    outputs on sampled steps and tokens."""
    wl = gen.WORKLOADS["dsv4_decode"]
    _flush(f"case: dsv4_decode T={T}")
    m = H.Model(wl.shape, cache_entries=8)
    run = H.DecodeRun(wl, m, T=T)
    out_steps = {0, 255, wl.steps - 1} if T == 1 else {0, wl.steps - 1}
    toks = None if T == 1 else [0, 13, T - 1]
    errs = []
    for s in range(wl.steps):
        for l in range(wl.shape.layers):
            check = s in out_steps and (T == 1 or l in (0, 3))
            _, err = run.step(l, s, check_out=check, out_tokens=toks)
            if err is not None:
                errs.append(err)
    st = run.eng.stats()
    _flush(f"dsv4 T={T}: hit rate {st['hits'] / st['lookups']:.3f}, max err/rms {max(errs):.2e}")
    run.close()


def test_glm_decode_with_resize():
    """GLM-5.2-shaped decode: 8 layers, top-8 + shared, T=1, 1024 steps over a
    41 GB host pool; the cache is resized from 1228 to 614 slots without a
    restart before step 512.  State is compared every call and right after
    the resize; outputs on sampled steps."""
    wl = gen.WORKLOADS["glm_decode"]
    _flush("case: glm_decode (loading the 41 GB expert pool)")
    m = H.Model(wl.shape, cache_entries=10)
    run = H.DecodeRun(wl, m, T=1)
    resize = dict(wl.resize)
    errs = []
    for s in range(wl.steps):
        if s in resize:
            run.eng.cache_resize(resize[s])
            moves, evicted = run.cache.resize(resize[s])
            key, stamp, clock = run.eng.cache_snapshot()
            k_ref, s_ref, c_ref = run.cache.snapshot()
            assert key.tolist() == k_ref and stamp.tolist() == s_ref and clock == c_ref
            # at most C' records move, and only those are copied
            assert len(moves) <= resize[s]
            assert run.eng.stats()["bytes_d2d"] == len(moves) * wl.shape.expert_bytes()
            _flush(f"resized to {resize[s]} slots at step {s}: {len(evicted)} evicted, "
                   f"{len(moves)} moved")
        for l in range(wl.shape.layers):
            check = s in (0, 511, 512, wl.steps - 1) and l in (0, 7)
            _, err = run.step(l, s, check_out=check)
            if err is not None:
                errs.append(err)
    st = run.eng.stats()
    assert st["resizes"] == 1
    _flush(f"glm: hit rate {st['hits'] / st['lookups']:.3f}, max err/rms {max(errs):.2e}, "
           f"d2d bytes {st['bytes_d2d']}")
    run.close()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_resize_sequences_against_oracle(seed):
    """Random forwards interleaved with resizes to random sizes (including 0
    and growth), on a 3-layer shape: cache state matches the oracle after
    every operation and outputs stay identical to an uncached reference."""
    import torch
    sh = H.small_shape(E=16, k=3, layers=3, shared=True)
    T = 6
    rng = np.random.default_rng(seed)
    m = H.Model(sh, seed=seed)
    wl = gen.Workload("resize", sh, Ts=(T,), steps=40, cache_slots=10, staging_slots=T * sh.k,
                      zipf_s=1.1, overlap=0.5)
    run = H.DecodeRun(wl, m, T=T)
    ref = H.DecodeRun(wl, m, T=T, cache_slots=0)
    moved = 0
    for s in range(wl.steps):
        if rng.random() < 0.3:
            C2 = int(rng.choice([0, 1, 2, 5, 10, 17, 30, 48]))
            run.eng.cache_resize(C2)
            moves, _ = run.cache.resize(C2)
            moved += len(moves)
            key, stamp, clock = run.eng.cache_snapshot()
            k_ref, s_ref, c_ref = run.cache.snapshot()
            assert key.tolist() == k_ref and stamp.tolist() == s_ref and clock == c_ref
            # only the records that change slots are copied
            assert run.eng.stats()["bytes_d2d"] == moved * sh.expert_bytes()
        l = int(rng.integers(0, sh.layers))
        y, _ = run.step(l, s, check_out=(s % 10 == 0))
        y0, _ = ref.step(l, s, check_state=False)
        torch.cuda.synchronize()
        assert torch.equal(y, y0), f"resize history changed the output at step {s}"
    run.close()
    ref.close()
