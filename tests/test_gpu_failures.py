"""Failure handling, forced from the host (GPU; no kernel faults or hangs):
the per-stage synchronising debug mode, an injected copy failure and the
cache reset that recovers from it, and the first request of a cold process
completing in bounded time."""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("overlap", [0, 1])
def test_debug_sync_is_bit_identical(overlap):
    """MOE_DEBUG_SYNC waits and checks after every stage; results and cache
    state equal those of the unsynchronised run, with and without the
    copies beside the resident experts."""
    import torch
    sh = H.small_shape(E=32, k=4, shared=True, layers=2)
    T = 8
    wl = gen.Workload("dbg", sh, Ts=(T,), steps=6, cache_slots=10,
                      staging_slots=min(T * sh.k, sh.E), zipf_s=1.1, overlap=0.5)
    print(f"case: debug sync, overlap {overlap}", flush=True)
    m = H.Model(sh, seed=17)
    a, b = H.DecodeRun(wl, m, T=T), H.DecodeRun(wl, m, T=T)
    for r in (a, b):
        r.eng.set_copy_overlap(overlap)
    a.eng.set_debug(sync=True)
    for s in range(wl.steps):
        for l in range(sh.layers):
            ya, _ = a.step(l, s, check_out=(s == 2))
            yb, _ = b.step(l, s, check_state=False)
            torch.cuda.synchronize()
            assert torch.equal(ya, yb) and torch.equal(a.y32, b.y32)
    ka, sa, ca = a.eng.cache_snapshot()
    kb, sb, cb = b.eng.cache_snapshot()
    assert np.array_equal(ka, kb) and np.array_equal(sa, sb) and ca == cb
    a.close()
    b.close()


@pytest.mark.parametrize("overlap", [0, 1])
def test_injected_fill_failure_and_reset(overlap):
    """The next copy step fails as a failed copy would: the call returns a
    HIP error, every later forward and cache call returns STATE (the state
    may name experts whose bytes did not land), the state can still be read,
    and expert_cache_reset empties the cache.  The engine then continues in
    step with the oracle's cache reset at the same point, outputs checked."""
    import torch
    from expert_offload_serving_amd import MoEError
    sh = H.small_shape(E=32, k=4, shared=True, layers=2)
    T = 4
    wl = gen.Workload("fail", sh, Ts=(T,), steps=8, cache_slots=12,
                      staging_slots=min(T * sh.k, sh.E), zipf_s=1.1, overlap=0.5)
    print(f"case: injected fill failure, overlap {overlap}", flush=True)
    m = H.Model(sh, seed=23)
    run = H.DecodeRun(wl, m, T=T)
    run.eng.set_copy_overlap(overlap)
    for s in range(3):
        for l in range(sh.layers):
            run.step(l, s)
    run.eng.set_debug(fail_next_fill=True)
    xb, bias = run.inputs(0, 3)
    x = H.bf16_dev(xb)
    bdev = torch.from_numpy(bias).cuda()
    with pytest.raises(MoEError) as e:
        run.eng.forward(0, x, bias=bdev)
    assert e.value.name == "HIP" and "injected" in str(e.value)
    torch.cuda.synchronize()
    for call in (lambda: run.eng.forward(0, x, bias=bdev),
                 lambda: run.eng.cache_fill(0, [1, 2]),
                 lambda: run.eng.cache_resize(8)):
        with pytest.raises(MoEError) as e:
            call()
        assert e.value.name == "STATE"
    key, stamp, clock = run.eng.cache_snapshot()   # still readable
    assert len(key) == 12
    # what the device did: the failed call's lookup (hits stamped, misses
    # inserted, the clock advanced), then the reset
    import oracle
    xf = gen.bf16_bits_to_f32(xb)
    _, ids_ref, _ = run.model.route(0, xf, bias)
    run.cache.lookup(0, oracle.permutation(ids_ref, sh.E)["unique"])
    assert key.tolist() == run.cache.snapshot()[0] and clock == run.cache.snapshot()[2]
    run.eng.cache_reset()
    assert run.cache.reset() > 0
    key, stamp, clock = run.eng.cache_snapshot()
    assert (key == -1).all() and (stamp == 0).all()
    assert (key.tolist(), stamp.tolist(), clock) == run.cache.snapshot()
    for s in range(3, wl.steps):
        for l in range(sh.layers):
            run.step(l, s, check_out=(s in (3, wl.steps - 1)))
    st = run.eng.stats()
    assert st["fills"] > 0
    run.close()


def test_first_request_of_a_cold_process_completes():
    """A fresh process creates an engine and sends a 180-token prefill and
    then a decode call as its first requests (the pages' cold-server report
    was a prompt of about 180 tokens that hung in prefill); both must finish
    and be checked within the time limit."""
    script = textwrap.dedent(f"""
        import sys, time
        sys.path.insert(0, {ROOT!r})
        t0 = time.time()
        import numpy as np, torch
        from workload import gen
        from tests import harness as H
        sh = H.small_shape(E=32, k=4, shared=True, layers=2)
        run = H.PrefillRun(sh, 180, seed=1)
        run.run()
        xf, ids_ref, g_ref = run.check_routing(1)
        y_ref = H.oracle_rows(run.model, 1, xf, ids_ref, g_ref, list(range(0, 180, 7)))
        H.check_y(run.y32[1].cpu().numpy()[list(range(0, 180, 7))], y_ref,
                  rtol=H.RTOL_Y_PREFILL)
        x = torch.zeros((1, sh.H), dtype=torch.int16, device="cuda")
        run.eng.forward(0, x)
        torch.cuda.synchronize()
        print("first requests done in %.1f s" % (time.time() - t0), flush=True)
        run.close()
    """)
    print("case: cold process, first prefill and decode", flush=True)
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True,
                       timeout=240, cwd=ROOT)
    print(r.stdout[-500:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "first requests done" in r.stdout


def test_prefill_debug_sync_is_bit_identical():
    """MOE_DEBUG_SYNC on prefill (a synchronisation after every layer): the
    outputs of a 3-layer call equal those of the unsynchronised call."""
    import torch
    sh = H.small_shape(E=32, k=4, shared=True, layers=3)
    print("case: prefill debug sync", flush=True)
    run = H.PrefillRun(sh, 300, seed=4)
    run.run()
    ref = [y.clone() for y in run.y32]
    run.eng.set_debug(sync=True)
    run.run()
    assert all(torch.equal(a, b) for a, b in zip(ref, run.y32))
    run.close()
