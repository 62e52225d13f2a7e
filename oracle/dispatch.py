"""Token-to-expert dispatch: counts, offsets and a stable permutation.

Test infrastructure (see the package docstring).

Each (token, choice) pair is sent to its expert and the partial results are
summed at the end (jansverre.net FreeToken article, section "Hva er
FreeToken?").  Reading: pair f = t*k + j; the permutation lists pairs grouped
by ascending expert, and within an expert by ascending f.
"""
import numpy as np


def permutation(ids: np.ndarray, E: int):
    """Returns dict(counts[E], offsets[E+1], sorted[T*k], inv[T*k], unique).

    sorted[p] is the pair f placed at position p; inv[f] is the position of
    pair f; unique lists the experts with at least one pair, ascending.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    n = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    sorted_ = np.empty(n, dtype=np.int64)
    inv = np.empty(n, dtype=np.int64)
    for f in range(n):                    # ascending f keeps ties stable
        e = flat[f]
        p = cursor[e]
        cursor[e] += 1
        sorted_[p] = f
        inv[f] = p
    unique = np.array([e for e in range(E) if counts[e] > 0], dtype=np.int64)
    return dict(counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
                sorted=sorted_.astype(np.int32), inv=inv.astype(np.int32),
                unique=unique.astype(np.int32))
