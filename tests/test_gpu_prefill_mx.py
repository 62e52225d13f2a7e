"""The opt-in MXFP8 prefill mode (native-MX: MXFP8 activations x MXFP4
weights on the scaled matrix instructions) against the oracle of that mode,
element by element within oracle.mx.moe_layer_mx_bound's allowance for h's
rounding decisions and the fp32 arithmetic; on the last layer of a call the
decisions themselves are read back and checked (harness.check_mx_decisions);
and against the plain layer at the mode's stated accuracy (GPU)."""
import numpy as np
import pytest

from oracle import mx as omx
from workload import gen
from tests import harness as H

pytestmark = pytest.mark.gpu


def _check_layer_mx(run, layer, tokens, plain=True):
    xf, ids_ref, g_ref = run.check_routing(layer)
    H.check_rounding(run.ys[layer], run.y32[layer], f"mx prefill layer {layer}")
    y32 = run.y32[layer].cpu().numpy()[tokens]
    ref = H.oracle_rows(run.model, layer, xf, ids_ref, g_ref, tokens,
                        layer_fn=omx.moe_layer_mx_bound)
    err, allow, flipped = H.check_y_mx(y32, ref, what=f"mx prefill layer {layer} vs the MX oracle")
    msg = (f"  mx prefill layer {layer}: {len(tokens)} tokens, max err/rms {err:.3e} "
           f"(MX oracle; allowance up to {allow:.2e} x rms, {flipped:.2%} of elements past the "
           f"arithmetic allowance)")
    if layer == run.shape.layers - 1:
        share, werr = H.check_mx_decisions(run, tokens, what=f"mx prefill layer {layer}")
        msg += f"; decisions: {share:.3%} of h codes off the oracle's, y vs own h {werr:.2e} x rms"
    if plain:
        y_pl = H.oracle_rows(run.model, layer, xf, ids_ref, g_ref, tokens)
        e2 = H.check_y(y32, y_pl, what=f"mx prefill layer {layer} vs the plain layer",
                       rtol=H.RTOL_Y_MX_PLAIN)
        rr = float(np.sqrt(np.mean((y32 - y_pl) ** 2) / np.mean(y_pl ** 2)))
        assert rr <= H.RRMS_MX_PLAIN, f"relative rms {rr:.3g} from the plain layer"
        msg += f", {e2:.3e} / rel rms {rr:.3e} (plain)"
    print(msg, flush=True)
    return err


@pytest.mark.parametrize("T,kw", [(300, dict(E=32, k=4, shared=True, layers=2)),
                                  (129, dict(E=16, k=2)),
                                  (64, dict(E=64, k=8, shared=True, renormalize=False)),
                                  (1000, dict(H=384, I=256, E=40, k=6)),
                                  (200, dict(H=640, I=384, E=12, k=3, shared=True)),
                                  (700, dict(H=256, I=256, E=1024, k=16, shared=True)),
                                  # one K chunk (I = 128) and more work items than
                                  # workgroups: items run in turn without chaining
                                  (600, dict(H=256, I=128, E=512, k=8))])
def test_mx_prefill_small_all_tokens(T, kw):
    sh = H.small_shape(**kw)
    print(f"case: mx prefill T={T} {kw}", flush=True)
    run = H.PrefillRun(sh, T, seed=5, prefill_format="mxfp8")
    run.run()
    for l in range(sh.layers):
        _check_layer_mx(run, l, list(range(T)))
    run.close()


def test_mx_and_bf16_modes_on_one_engine():
    """Switching the mode between calls: the bf16 outputs come back bit for
    bit after an MXFP8 call, and a repeated MXFP8 call is bit-identical."""
    import torch
    sh = H.small_shape(E=32, k=4, shared=True, layers=2)
    T = 257
    print("case: mode switch bf16 -> mxfp8 -> bf16", flush=True)
    run = H.PrefillRun(sh, T, seed=6)
    run.run()
    ref = [y.clone() for y in run.y32]
    run.eng.set_prefill_format("mxfp8")
    run.run()
    mx1 = [y.clone() for y in run.y32]
    assert not all(torch.equal(a, b) for a, b in zip(ref, mx1))
    run.run()
    assert all(torch.equal(a, b) for a, b in zip(mx1, run.y32))
    _check_layer_mx(run, 1, list(range(0, T, 3)))
    run.eng.set_prefill_format("bf16")
    run.run()
    assert all(torch.equal(a, b) for a, b in zip(ref, run.y32))
    run.close()


@pytest.mark.timeout(1200)
def test_mx_prefill_dsv4_full_size():
    """DeepSeek-V4-Flash-shaped prefill, T=4096, 4 layers, MXFP8 mode: every
    layer's routing and dispatch bit for bit, 128 seeded tokens per layer
    against the MX oracle (64 of them also against the plain layer)."""
    wl = gen.WORKLOADS["dsv4_prefill"]
    sh = wl.shape
    T = wl.Ts[0]
    print("case: mx dsv4_prefill T=4096 (loading 13.7 GB expert pool)", flush=True)
    run = H.PrefillRun(sh, T, seed=0, model=H.Model(sh, cache_entries=4), prefill_format="mxfp8")
    run.run()
    for l in range(sh.layers):
        rng = np.random.default_rng(2000 + l)
        toks = sorted({0, T - 1} | set(rng.choice(T, 126, replace=False).tolist()))
        _check_layer_mx(run, l, toks, plain=(l == 0))
    run.close()
