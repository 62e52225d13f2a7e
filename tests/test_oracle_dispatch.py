"""Pins for the oracle's dispatch permutation (no GPU)."""
import numpy as np
import pytest

from oracle import dispatch


@pytest.mark.parametrize("T,k,E", [(1, 1, 4), (4, 2, 8), (16, 8, 256), (37, 6, 256), (300, 8, 64)])
def test_permutation_matches_numpy(T, k, E):
    rng = np.random.default_rng(T * 131 + k)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    p = dispatch.permutation(ids, E)
    flat = ids.reshape(-1)
    assert np.array_equal(p["sorted"], np.argsort(flat, kind="stable"))
    assert np.array_equal(p["counts"], np.bincount(flat, minlength=E))
    assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(p["inv"][p["sorted"]], np.arange(T * k))
    assert np.array_equal(p["unique"], np.unique(flat))


def test_permutation_empty():
    p = dispatch.permutation(np.zeros((0, 4), np.int32), 8)
    assert p["sorted"].size == 0 and p["unique"].size == 0
    assert np.all(p["offsets"] == 0)
