"""Decode calls captured into HIP graphs (GPU).  moe_layer_forward enqueues
kernels only (no memset, copy or host synchronisation), so a captured step
must replay exactly as the eager call: every replay is checked against an
eager engine fed the same sequence, with the program's own eager work and
synchronisations between replays, and each step's graph is replayed twice
(the second replay sees the cache state the first one left)."""
import numpy as np
import pytest

from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    import torch
    sh = H.small_shape(H=512, I=256, E=32, k=4, layers=2, shared=True)
    T, steps, seed = 4, 6, 21
    print("case: graph replay vs eager, T=4, 2 layers, 12-slot cache", flush=True)
    m = H.Model(sh, seed=seed)
    engs = []
    for _ in range(2):
        eng = H.make_engine(sh, T, cache_slots=12, staging_slots=T * sh.k)
        m.load(eng)
        engs.append(eng)
    sets = [gen.zipf_sets(sh, l, T, steps, 1.1, 0.5, seed) for l in range(sh.layers)]
    xs = [[H.bf16_dev(gen.tokens(sh, l, s, T, seed)) for s in range(steps)] for l in range(sh.layers)]
    bs = [[torch.from_numpy(gen.bias_from_sets(sets[l][s], sh.E)).cuda() for s in range(steps)]
          for l in range(sh.layers)]
    ys = [torch.empty((T, sh.H), dtype=torch.int16, device="cuda") for _ in range(sh.layers)]
    y32s = [torch.empty((T, sh.H), dtype=torch.float32, device="cuda") for _ in range(sh.layers)]

    def step(eng, s):
        for l in range(sh.layers):
            eng.forward(l, xs[l][s], bias=bs[l][s], y=ys[l], y32=y32s[l])

    ref = []
    for s in range(steps):
        for _ in range(2):
            step(engs[0], s)
            torch.cuda.synchronize()
            ref.append([(ys[l].clone(), y32s[l].clone()) for l in range(sh.layers)])
    graphs = []
    for s in range(steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(engs[1], s)
        graphs.append(g)
    torch.cuda.synchronize()
    i = 0
    for s in range(steps):
        for _ in range(2):
            for l in range(sh.layers):  # stale values must be overwritten by the replay
                ys[l].fill_(0x7FFF)
                y32s[l].fill_(float("nan"))
            graphs[s].replay()
            torch.cuda.synchronize()
            (torch.ones(4096, device="cuda") * 3.0).sum().item()  # eager work between replays
            for l in range(sh.layers):
                assert torch.equal(ys[l], ref[i][l][0]), f"step {s} replay {i % 2} layer {l}"
                assert torch.equal(y32s[l], ref[i][l][1]), f"step {s} replay {i % 2} layer {l}"
            i += 1
    snaps = [e.cache_snapshot() for e in engs]
    for a, b in zip(snaps[0], snaps[1]):
        assert np.array_equal(np.asarray(a), np.asarray(b))
    s0, s1 = engs[0].stats(), engs[1].stats()
    for k in ("lookups", "hits", "fills", "bypasses", "evictions", "bytes_h2d"):
        assert s0[k] == s1[k], k
    assert s0["hits"] > 0 and s0["fills"] > 0  # the trace exercised both paths
    for eng in engs:
        eng.close()
