"""Top-k with exact logit ties, decode and prefill (GPU).

With x = 0 the router logits are exactly the bias (fp64 sums of zero
products plus the bias, rounded once to fp32), so a bias that takes a few
values makes many experts tie.  The order must be (logit descending, expert
ascending), the reading the oracle's top-k follows, whether the tied experts
sit in different lanes of the selecting wave or in the same lane (experts e
and e + 64 share a lane).
"""
import numpy as np
import pytest

from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu


def _tie_bias(E: int, T: int) -> np.ndarray:
    e = np.arange(E)
    rows = [np.zeros(E),                                   # every expert ties
            (e % 5 == 0).astype(np.float64),               # ties across lanes
            (e // 64).astype(np.float64),                  # the top block of 64 ties
            (e % 64 == 7) * 2.0 + (e % 3 == 1),            # one lane's experts tie on top
            -(e % 2).astype(np.float64),                   # half the experts tie on top
            (e % 64 == 63) * 1.0 + (e >= E - 2) * 1.0]     # a two-level tie in the last lane
    b = np.stack([rows[t % len(rows)] for t in range(T)])
    return b.astype(np.float32)


def _zeros_bf16(T, H_):
    return np.zeros((T, H_), dtype=np.uint16)


@pytest.mark.parametrize("E,k", [(256, 8), (200, 6), (64, 16)])
def test_decode_topk_ties(E, k):
    import torch
    sh = H.small_shape(H=128, I=128, E=E, k=k)
    T = 6
    print(f"case: decode top-k ties E={E} k={k}", flush=True)
    m = H.Model(sh, seed=41)
    eng = H.make_engine(sh, T, cache_slots=E, staging_slots=T * k)
    m.load(eng)
    bias = _tie_bias(E, T)
    x = H.bf16_dev(_zeros_bf16(T, sh.H))
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    eng.forward(0, x, bias=torch.from_numpy(bias).cuda(), ids=ids, gates=gates)
    torch.cuda.synchronize()
    _, ids_ref, g_ref = m.route(0, np.zeros((T, sh.H), np.float32), bias)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.max(np.abs(gates.cpu().numpy() - g_ref)) <= H.ATOL_G
    assert ids_ref[0].tolist() == list(range(k))  # all equal: the lowest experts
    eng.close()


def test_prefill_topk_ties():
    import torch
    sh = H.small_shape(H=128, I=128, E=256, k=8)
    T = 70
    print("case: prefill top-k ties E=256 k=8", flush=True)
    bias = _tie_bias(sh.E, T)
    run = H.PrefillRun(sh, T, seed=42, bias_sets=[bias])
    run.xb = [_zeros_bf16(T, sh.H)]
    run.xs = [H.bf16_dev(run.xb[0])]
    run.run()
    run.check_routing(0)
    torch.cuda.synchronize()
    run.close()
