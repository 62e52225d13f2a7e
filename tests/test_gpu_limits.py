"""Parity at the edges of the supported configuration space (GPU)."""
import pytest

from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def test_largest_experts():
    """H = I = 6144 (the largest supported): 60 MB experts, 2 cache slots for
    4 experts, so most calls fill and bypass; outputs every step."""
    sh = H.small_shape(H=6144, I=6144, E=4, k=2)
    T = 3
    wl = gen.Workload("largest", sh, Ts=(T,), steps=3, cache_slots=2, staging_slots=4)
    _flush("case: H=I=6144, E=4, k=2, T=3")
    m = H.Model(sh, seed=21, cache_entries=4)
    run = H.DecodeRun(wl, m, T=T)
    for s in range(3):
        run.step(0, s, check_out=True)
    st = run.eng.stats()
    assert st["fills"] + st["bypasses"] > 0
    run.close()


@pytest.mark.parametrize("k", [16])
def test_most_experts_top16(k):
    """E = 1024 (the most supported) with top-16 and Zipf routing through a
    200-slot cache: routing, permutation, slots and state every step, outputs
    on every step."""
    sh = H.small_shape(H=128, I=128, E=1024, k=k)
    T = 8
    wl = gen.Workload("manyexperts", sh, Ts=(T,), steps=6, cache_slots=200, staging_slots=T * k,
                      zipf_s=1.1, overlap=0.5)
    _flush(f"case: E=1024 k={k} T={T}")
    m = H.Model(sh, seed=22, cache_entries=256)
    run = H.DecodeRun(wl, m, T=T)
    for s in range(wl.steps):
        run.step(0, s, check_out=True)
    run.close()


def test_top_k_equals_experts():
    """k = E: every token uses every expert (gates are the full softmax)."""
    sh = H.small_shape(E=16, k=16, shared=True)
    T = 5
    wl = gen.Workload("allexperts", sh, Ts=(T,), steps=2, cache_slots=6, staging_slots=16)
    _flush("case: E=k=16 with shared expert")
    m = H.Model(sh, seed=23)
    run = H.DecodeRun(wl, m, T=T)
    for s in range(2):
        run.step(0, s, check_out=True)
    run.close()


def test_prefill_most_experts_top16():
    """Prefill with E = 1024 and top-16: many small groups (about 11 rows per
    expert), ragged tiles everywhere; every token of both layers."""
    from tests import test_gpu_prefill as TP
    sh = H.small_shape(H=256, I=256, E=1024, k=16, layers=2, shared=True)
    T = 700
    _flush(f"case: prefill E=1024 k=16 T={T}")
    run = H.PrefillRun(sh, T, seed=24)
    run.run()
    for l in range(sh.layers):
        TP._check_layer(run, l, list(range(T)))
    run.close()
