"""Pins for the oracle's router: logits, top-k and gates (no GPU)."""
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import router


def _nearest_f32(q: Fraction) -> np.float32:
    """Correctly rounded (ties to even) fp32 of an exact rational."""
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.array(c).view(np.uint32)) & 1))
    return best


def test_logits_are_exact_sum_rounded_once():
    rng = np.random.default_rng(3)
    T, H, E = 3, 64, 5
    x = rng.standard_normal((T, H)).astype(np.float32)
    x = x.astype(np.float32)  # values are bf16-like floats; any float works
    w = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
    b = rng.standard_normal((T, E)).astype(np.float32)
    lg = router.logits(x, w, b)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(x[t, h])) * Fraction(float(w[h, e])) for h in range(H))
            exact += Fraction(float(b[t, e]))
            assert lg[t, e] == _nearest_f32(exact)


def test_uniform_logits_pick_lowest_ids_equal_gates():
    T, H, E, k = 4, 32, 16, 6
    lg, ids, g = router.route(np.ones((T, H), np.float32), np.zeros((H, E), np.float32), k)
    assert np.all(lg == 0)
    assert np.array_equal(ids, np.tile(np.arange(k), (T, 1)))
    assert np.allclose(g, 1.0 / k, atol=0, rtol=1e-7)


def test_duplicated_columns_tie_to_lower_id():
    rng = np.random.default_rng(0)
    H, E = 32, 8
    w = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
    w[:, 5] = w[:, 2]
    x = rng.standard_normal((1, H)).astype(np.float32)
    lg = router.logits(x, w)
    assert lg[0, 5] == lg[0, 2]
    ids = router.topk(lg, E)[0].tolist()
    assert ids.index(2) < ids.index(5)
    assert ids.index(5) == ids.index(2) + 1 or lg[0, ids[ids.index(2) + 1]] == lg[0, 2]


def test_topk_against_python_sort():
    rng = np.random.default_rng(7)
    for _ in range(50):
        E = int(rng.integers(2, 40))
        k = int(rng.integers(1, E + 1))
        # coarse values so ties happen often
        lg = rng.integers(-3, 4, size=(3, E)).astype(np.float32)
        ids = router.topk(lg, k)
        for t in range(3):
            want = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
            assert ids[t].tolist() == want


def test_forced_bias_selects_the_set():
    rng = np.random.default_rng(1)
    H, E, k = 256, 64, 8
    x = rng.standard_normal((2, H)).astype(np.float32)
    w = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
    bias = np.zeros((2, E), np.float32)
    S = [sorted(rng.choice(E, k, replace=False).tolist()) for _ in range(2)]
    for t in range(2):
        bias[t, S[t]] = 32.0
    _, ids, g = router.route(x, w, k, bias)
    for t in range(2):
        assert sorted(ids[t].tolist()) == S[t]
    # the bias is common to the chosen set, so it cancels in the gates
    lg0 = router.logits(x, w)
    g0 = router.gates(lg0, ids)
    assert np.allclose(g, g0, rtol=1e-5, atol=1e-7)


def test_two_expert_gate_closed_form():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((20, 9)).astype(np.float32)
    ids = router.topk(lg, 2)
    g = router.gates(lg, ids)
    for t in range(20):
        l0, l1 = float(lg[t, ids[t, 0]]), float(lg[t, ids[t, 1]])
        assert abs(g[t, 0] - expit(l0 - l1)) < 1e-7
        assert abs(g[t, 1] - expit(l1 - l0)) < 1e-7


@pytest.mark.parametrize("k", [1, 3, 8])
def test_gates_sum_to_one_and_match_softmax(k):
    rng = np.random.default_rng(k)
    lg = (rng.standard_normal((10, 32)) * 3).astype(np.float32)
    ids = router.topk(lg, k)
    g = router.gates(lg, ids, renormalize=True)
    assert np.all(np.abs(g.astype(np.float64).sum(1) - 1.0) <= 1e-6)
    p = softmax(lg.astype(np.float64), axis=1)
    for t in range(10):
        sel = p[t, ids[t]]
        assert np.allclose(g[t], sel / sel.sum(), rtol=2e-7, atol=1e-9)
    g_full = router.gates(lg, ids, renormalize=False)
    for t in range(10):
        assert np.allclose(g_full[t], p[t, ids[t]], rtol=2e-7, atol=1e-9)
    # gates follow the order of the ids: non-increasing
    assert np.all(np.diff(g, axis=1) <= 0)
