"""The library's host-side resize planner (csrc/resize_plan.h), built on its
own with g++ under the address and undefined-behaviour sanitizers, against
the oracle's SlotCache.resize on random slot tables (no GPU): the new table,
the moves, the evicted keys, and the recency order the device lookup
continues from."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.cache import SlotCache

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHIFT = 12


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("plan") / "resize_plan_check")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-o", exe,
                    os.path.join(ROOT, "tests", "resize_plan_check.cpp")], check=True)
    return exe


def _random_table(rng, C, E):
    """A table the lookup rule can produce: distinct keys, distinct positive
    stamps on the occupied slots, 0 on the empty ones."""
    occ = rng.random(C) < rng.uniform(0.2, 1.0)
    keys = rng.choice(E, size=C, replace=False) if C <= E else rng.permutation(C)
    stamps = rng.permutation(np.arange(1, C + 1)) * int(rng.integers(1, 4))
    key = [int(k) if o else -1 for k, o in zip(keys, occ)]
    stamp = [int(s) if o else 0 for s, o in zip(stamps, occ)]
    return key, stamp


def _run(exe, cases):
    text = "".join(f"{C} {C2}\n" + "".join(f"{k} {s}\n" for k, s in zip(key, stamp))
                   for key, stamp, C, C2 in cases)
    r = subprocess.run([exe], input=text, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-2000:]
    lines = r.stdout.splitlines()
    out, i = [], 0
    for key, stamp, C, C2 in cases:
        assert lines[i] == "plan"
        rows = [tuple(int(v) for v in l.split()) for l in lines[i + 1:i + 1 + C2]]
        i += 1 + C2
        n = int(lines[i].split()[1])
        moves = [tuple(int(v) for v in l.split()) for l in lines[i + 1:i + 1 + n]]
        i += 1 + n
        m = int(lines[i].split()[1])
        ev = [int(v) for v in lines[i + 1].split()] if m else []
        i += 2
        out.append((rows, moves, ev))
    return out


def test_planner_matches_oracle(planner):
    rng = np.random.default_rng(9)
    cases = []
    for _ in range(400):
        C = int(rng.integers(0, 40))
        key, stamp = _random_table(rng, C, 200)
        C2 = int(rng.integers(0, 50))
        cases.append((key, stamp, C, C2))
    for (key, stamp, C, C2), (rows, moves, ev) in zip(cases, _run(planner, cases)):
        ref = SlotCache(C, 200)
        ref.key, ref.stamp = list(key), list(stamp)
        ref_moves, ref_ev = ref.resize(C2)
        assert [r[0] for r in rows] == ref.key and [r[1] for r in rows] == ref.stamp
        assert moves == ref_moves and ev == ref_ev
        # recency order: empty slots by index, then occupied by ascending stamp
        want = sorted(range(C2), key=lambda s: (ref.key[s] >= 0, ref.stamp[s], s))
        assert [r[2] for r in rows] == [s | ((ref.key[s] + 1) << SHIFT) for s in want]
        # only survivors past the new capacity move, each into a slot below it
        assert all(s >= C2 > d for s, d in moves) and len(moves) <= C2


def test_planner_edge_cases(planner):
    full = (list(range(10)), list(range(1, 11)))
    cases = [([], [], 0, 0), ([], [], 0, 7), (*full, 10, 0), (*full, 10, 10), (*full, 10, 3),
             ([-1] * 6, [0] * 6, 6, 2), ([5, -1, 7], [3, 0, 1], 3, 1)]
    out = _run(planner, cases)
    assert [r[0] for r in out[2][0]] == [] and out[2][2] == list(range(10))
    assert [r[0] for r in out[4][0]] == [7, 8, 9] and len(out[4][1]) == 3
    assert [r[0] for r in out[6][0]] == [5] and out[6][2] == [7]
