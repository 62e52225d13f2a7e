"""Prefill-path parity: the HIP library against the CPU oracle (GPU)."""
import numpy as np
import pytest

from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu


def _check_layer(run, layer, tokens):
    """Routing and dispatch of the layer bit for bit (every token), then the
    fp32 outputs of the listed tokens against oracle.moe_layer."""
    xf, ids_ref, g_ref = run.check_routing(layer)
    H.check_rounding(run.ys[layer], run.y32[layer], f"prefill layer {layer}")
    y_ref = H.oracle_rows(run.model, layer, xf, ids_ref, g_ref, tokens)
    y32 = run.y32[layer].cpu().numpy()[tokens]
    err = H.check_y(y32, y_ref, what=f"prefill layer {layer}", rtol=H.RTOL_Y_PREFILL)
    print(f"  prefill layer {layer}: {len(tokens)} tokens, max err/rms {err:.3e}", flush=True)
    return err


@pytest.mark.parametrize("T,kw", [(300, dict(E=32, k=4, shared=True, layers=3)),
                                  (129, dict(E=16, k=2, layers=2)),
                                  (64, dict(E=64, k=8, shared=True, renormalize=False)),
                                  (1000, dict(H=384, I=256, E=40, k=6, layers=2)),
                                  # I = 3 chunks of 128 (h's last remainder records come from
                                  # a half-filled gate/up column block), H = 640 (the last down
                                  # column block is partial)
                                  (200, dict(H=640, I=384, E=12, k=3, shared=True))])
def test_prefill_small_all_tokens(T, kw):
    """Ragged token counts (not multiples of the 64/128-row tiles), every
    layer, every token."""
    sh = H.small_shape(**kw)
    print(f"case: prefill T={T} {kw}", flush=True)
    run = H.PrefillRun(sh, T, seed=4)
    run.run()
    for l in range(sh.layers):
        _check_layer(run, l, list(range(T)))
    run.close()


def test_prefill_single_token_and_bias():
    sh = H.small_shape(E=16, k=4, shared=True, layers=2)
    T = 1
    sets = [gen.zipf_sets(sh, l, T, 1, 1.1, 0.5, 0)[0] for l in range(2)]
    bias = [gen.bias_from_sets(s, sh.E) for s in sets]
    run = H.PrefillRun(sh, T, seed=7, bias_sets=bias)
    run.run()
    for l in range(2):
        _check_layer(run, l, [0])
        ids = run.eng.inspect_prefill(l)["ids"]
        assert sorted(ids[0].tolist()) == sorted(sets[l][0].tolist())
    run.close()


@pytest.mark.timeout(1200)
def test_prefill_dsv4_full_size():
    """DeepSeek-V4-Flash-shaped prefill, T=4096, 4 layers, double-buffered
    uploads: on every layer the routing and dispatch of all 4096 tokens bit
    for bit, and the outputs of 512 seeded tokens (always including the first
    and the last) against oracle.moe_layer."""
    wl = gen.WORKLOADS["dsv4_prefill"]
    sh = wl.shape
    T = wl.Ts[0]
    print("case: dsv4_prefill T=4096 (loading 13.7 GB expert pool)", flush=True)
    run = H.PrefillRun(sh, T, seed=0, model=H.Model(sh, cache_entries=4))
    run.run()
    errs = []
    for l in range(sh.layers):
        rng = np.random.default_rng(1000 + l)
        toks = sorted({0, T - 1} | set(rng.choice(T, 510, replace=False).tolist()))
        errs.append(_check_layer(run, l, toks))
    print(f"dsv4 prefill max err/rms {max(errs):.3e}", flush=True)
    # a second call reuses the layer buffers: same outputs bit for bit
    import torch
    first = [y.clone() for y in run.ys]
    run.run()
    assert all(torch.equal(a, b) for a, b in zip(first, run.ys))
    run.close()


def test_prefill_outputs_ignore_earlier_calls():
    """Row loads past a tile's valid rows are not issued, so those LDS rows
    hold whatever an earlier workgroup left there.  Valid outputs must not
    depend on it: after a call whose activations are scaled by 2^124 (gate/up
    overflows, h becomes inf/NaN in the epilogue's LDS), the original call
    gives the same bits as before.  Both calls use ragged tiles (T=300,
    32 experts, top-4)."""
    import torch
    sh = H.small_shape(E=32, k=4, shared=True, layers=1)
    T = 300
    print("case: prefill after an overflowing call", flush=True)
    run = H.PrefillRun(sh, T, seed=4)
    run.run()
    ref32, refb = run.y32[0].clone(), run.ys[0].clone()
    big = gen.f32_to_bf16_bits(gen.bf16_bits_to_f32(run.xb[0]) * np.float32(2.0 ** 124))
    assert np.all(np.isfinite(gen.bf16_bits_to_f32(big)))
    good = run.xs[0]
    run.xs = [H.bf16_dev(big)]
    run.run()
    assert not torch.isfinite(run.y32[0]).all()  # the poisoning call did overflow
    run.xs = [good]
    run.run()
    assert torch.equal(run.y32[0], ref32) and torch.equal(run.ys[0], refb)
    run.close()
