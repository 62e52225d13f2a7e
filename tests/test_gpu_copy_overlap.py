"""Decode with the copies of missed experts running beside the resident
experts' kernels (GPU).  Execution order must change nothing: two engines
fed the same trace, one with the overlap forced on and one with it off, give
bit-identical outputs, routing and cache state after every call, and the
overlapped engine matches the oracle.  Also the overlapped calls' kernel
timing and the forward under stream capture, which stays on one stream."""
import numpy as np
import pytest

from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,kw,C", [
    (1, dict(E=32, k=4, shared=True, layers=3), 10),
    (7, dict(E=32, k=4, layers=2), 12),
    (16, dict(E=64, k=8, shared=True), 20),
    (33, dict(E=64, k=6, shared=True, layers=2), 24),   # the T > 16 kernels
    (64, dict(E=200, k=16), 40),
    (16, dict(E=64, k=8, shared=True), 0),              # every expert bypasses
])
def test_overlap_on_and_off_are_identical(T, kw, C):
    import torch
    sh = H.small_shape(**kw)
    wl = gen.Workload("overlap", sh, Ts=(T,), steps=10, cache_slots=C,
                      staging_slots=min(T * sh.k, sh.E), zipf_s=1.1, overlap=0.5)
    print(f"case: copy overlap on/off T={T} {kw} C={C}", flush=True)
    m = H.Model(sh, seed=40 + T)
    on = H.DecodeRun(wl, m, T=T)
    off = H.DecodeRun(wl, m, T=T)
    on.eng.set_copy_overlap(1)
    off.eng.set_copy_overlap(0)
    for s in range(wl.steps):
        for l in range(sh.layers):
            y1, _ = on.step(l, s, check_out=(s % 3 == 0))
            y0, _ = off.step(l, s, check_state=(s % 3 == 1))
            torch.cuda.synchronize()
            assert torch.equal(y1, y0), f"outputs differ at step {s} layer {l}"
            assert torch.equal(on.y32, off.y32), f"fp32 outputs differ at step {s} layer {l}"
            assert torch.equal(on.ids, off.ids) and torch.equal(on.gates, off.gates)
            k1, s1, c1 = on.eng.cache_snapshot()
            k0, s0, c0 = off.eng.cache_snapshot()
            assert np.array_equal(k1, k0) and np.array_equal(s1, s0) and c1 == c0
    st1, st0 = on.eng.stats(), off.eng.stats()
    for k in ("lookups", "hits", "fills", "bypasses", "evictions", "bytes_h2d"):
        assert st1[k] == st0[k], k
    on.close()
    off.close()


def test_overlapped_calls_are_timed():
    """Timing mode on overlapped calls: every call is counted as split, the
    two launches of gate/up and down are summed into theirs, and the
    outputs equal those of untimed calls."""
    import torch
    sh = H.small_shape(E=32, k=4, shared=True, layers=2)
    T = 4
    wl = gen.Workload("overlap_t", sh, Ts=(T,), steps=6, cache_slots=8,
                      staging_slots=T * sh.k, zipf_s=1.1, overlap=0.5)
    print("case: timing of overlapped calls", flush=True)
    m = H.Model(sh, seed=3)
    a, b = H.DecodeRun(wl, m, T=T), H.DecodeRun(wl, m, T=T)
    a.eng.set_copy_overlap(1)
    b.eng.set_copy_overlap(1)
    a.eng.set_timing(True)
    calls = 0
    for s in range(wl.steps):
        for l in range(sh.layers):
            ya, _ = a.step(l, s)
            yb, _ = b.step(l, s, check_state=False)
            torch.cuda.synchronize()
            assert torch.equal(ya, yb)
            calls += 1
    tm = a.eng.get_timing()
    assert tm["n_decode"] == calls and tm["n_decode_split"] == calls
    ms = tm["decode_ms"]
    assert all(np.isfinite(v) and v >= 0 for v in ms.values())
    assert ms["gateup"] > 0 and ms["down"] > 0 and ms["router"] > 0
    a.close()
    b.close()


def test_capture_keeps_one_stream():
    """With the overlap forced on, a forward captured into a HIP graph runs
    on the capturing stream alone and replays as the eager overlapped
    call."""
    import torch
    sh = H.small_shape(E=32, k=4, shared=True, layers=2)
    T, steps, seed = 4, 4, 8
    print("case: capture with the copy overlap on", flush=True)
    m = H.Model(sh, seed=seed)
    engs = []
    for _ in range(2):
        eng = H.make_engine(sh, T, cache_slots=10, staging_slots=T * sh.k)
        m.load(eng)
        eng.set_copy_overlap(1)
        engs.append(eng)
    sets = [gen.zipf_sets(sh, l, T, steps, 1.1, 0.5, seed) for l in range(sh.layers)]
    xs = [[H.bf16_dev(gen.tokens(sh, l, s, T, seed)) for s in range(steps)] for l in range(sh.layers)]
    bs = [[torch.from_numpy(gen.bias_from_sets(sets[l][s], sh.E)).cuda() for s in range(steps)]
          for l in range(sh.layers)]
    ys = [torch.empty((T, sh.H), dtype=torch.int16, device="cuda") for _ in range(sh.layers)]

    def step(eng, s):
        for l in range(sh.layers):
            eng.forward(l, xs[l][s], bias=bs[l][s], y=ys[l])

    ref = []
    for s in range(steps):
        step(engs[0], s)
        torch.cuda.synchronize()
        ref.append([y.clone() for y in ys])
    graphs = []
    for s in range(steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(engs[1], s)
        graphs.append(g)
    torch.cuda.synchronize()
    for s in range(steps):
        for y in ys:
            y.fill_(0x7FFF)
        graphs[s].replay()
        torch.cuda.synchronize()
        for l in range(sh.layers):
            assert torch.equal(ys[l], ref[s][l]), f"replay of step {s} layer {l}"
    k0, s0, c0 = engs[0].cache_snapshot()
    k1, s1, c1 = engs[1].cache_snapshot()
    assert np.array_equal(k0, k1) and np.array_equal(s0, s1) and c0 == c1
    for eng in engs:
        eng.close()
