"""Benchmark of the routed MoE expert-layer forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--T T]
                [--prefill-steps P] [--dsv4-decode-steps D] [--no-context] ...

A step is one decode call per MoE layer of the workload (router, top-k,
dispatch, cache lookup, miss copies, expert FFN, combine) for a batch of T
tokens, with every step's activations and router bias already resident in
HBM.  The headline workload is the GLM-5.2-shaped decode: 8 MoE layers,
H=6144, E=256 routed experts top-8 plus one shared expert, I=2048, MXFP4
experts (a 41 GB pool in pinned host memory), T=1, Zipf(1.2) routing with
55% step-to-step overlap, through one global HBM expert cache of 1228
slots (60% of the experts) from a cold start; the cache is resized to 614
slots (30%) without a restart before the middle timed step.  W untimed
steps run first, then K timed ones.

`value` is tokens/s of whole forwards, miss copies over PCIe included (the
expert pool lives in host memory by design).  The roofline object is the
gate/up expert kernel's, the dominant HBM-bound kernel of a layer (the miss
copies are bound by PCIe and reported as pcie_h2d_gbs), with the down kernel
and the layer as a whole (router, finalize, gate/up, down, combine) beside
it; kernel durations come from a second pass over the timed steps in which
every kernel carries HIP start and stop events recorded by its own dispatch.
A check pass then runs sampled (step, layer) pairs again with their routing
and fp32 outputs read back, and the CPU oracle evaluates the same pairs:
that comparison is `parity`, and its timing `cpu_baseline`.

Context legs (skipped with --no-context): the 35B-A3B-shaped layer at T=16
(its 107 MB cache stays in the 256 MB Infinity Cache, so its kernel rates
are MALL rates), and the DeepSeek-V4-Flash-shaped stack: prefill of T=4096
(grouped MFMA GEMMs, layer uploads double-buffered) and T=1 decode.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense fp8 (an fp8 A operand sets the scaled instruction's rate)

# decode steps of the kernel-timing pass
TIMING_STEPS = 128
# (warmup, timed steps) when --warmup / --steps are not given
DEFAULT_STEPS = {"glm_decode": (0, 1024), "a3b_decode": (32, 512), "dsv4_decode": (16, 256)}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="glm_decode")
    ap.add_argument("--T", type=int, default=None, help="tokens per step (default: largest of the workload)")
    ap.add_argument("--distinct", type=int, default=8,
                    help="generated expert records per layer of the headline workload (expert e "
                         "holds record e mod N; the same bytes move, set-up is faster; 0: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--check-pairs", type=int, default=4,
                    help="(step, layer) pairs read back and compared with the oracle")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the 35B-A3B and DeepSeek-V4-Flash context legs")
    ap.add_argument("--extra-T", default="1,4", help="35B-A3B context leg: also time these T")
    ap.add_argument("--graph-T", default="",
                    help="35B-A3B context leg: also time these T with every step replayed from a "
                         "HIP graph (e.g. 1,4,16; default: none)")
    ap.add_argument("--prefill-steps", type=int, default=3,
                    help="prefill passes of the DeepSeek-V4-Flash-shaped stack (0: skip)")
    ap.add_argument("--legs", default="headline,a3b,dsv4,formats",
                    help="workloads to run: the headline decode line and the context legs "
                         "(35B-A3B decode, DeepSeek-V4-Flash prefill and decode, prefill with "
                         "bf16 and NVFP4 experts; each runs whole; without the headline only "
                         "the context is printed)")
    ap.add_argument("--prefill-formats", default="bf16,mxfp8",
                    help="prefill modes timed on the DeepSeek-V4-Flash-shaped stack")
    ap.add_argument("--dsv4-decode-steps", type=int, default=256,
                    help="T=1 decode steps of the DeepSeek-V4-Flash-shaped stack (0: skip)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="also run one plain copy of this many MiB (counter calibration)")
    ap.add_argument("--weights", choices=("mxfp4", "bf16", "nvfp4"), default="mxfp4",
                    help="expert format of the headline workload (no context legs)")
    ap.add_argument("--copy-overlap", type=int, choices=(-1, 0, 1), default=-1,
                    help="headline decode: copies beside the resident experts' kernels "
                         "(-1: the library's choice by record size, 0: never, 1: always)")
    ap.add_argument("--prefetch-study", type=int, default=0, metavar="STEPS",
                    help="instead of the benchmark line: GLM-5.2-shaped decode with each "
                         "cross-layer prefetch predictor (STEPS timed steps per run)")
    ap.add_argument("--prefetch-kinds", default="none,exact,half,popular,random",
                    help="predictors the prefetch study runs")
    ap.add_argument("--prefetch-slots", default="",
                    help="cache capacities the prefetch study runs (default: 1228,614)")
    ap.add_argument("--policy-study", type=int, default=0, metavar="STEPS",
                    help="instead of the benchmark line: DeepSeek-V4-Flash-shaped decode under "
                         "each cache placement policy (STEPS timed steps per run)")
    return ap.parse_args(argv)


# ------------------------------------------------------------ byte accounting
def kernel_bytes(sh, lookups, calls, pairs, T_total):
    """Algorithmic HBM bytes of the two decode expert kernels over `calls`
    calls, as (gate/up, down).  Weights: every looked-up expert once, plus
    the shared expert once per call; gate/up is 2/3 of an MXFP4 expert, down
    1/3.  Activations: gate/up reads each token row once and writes h as two
    bf16 planes; down reads those planes and writes fp32 expert outputs."""
    b_e = sh.expert_bytes()
    experts = lookups + (calls if sh.shared else 0)
    rows = pairs + (T_total if sh.shared else 0)
    gateup = experts * (2 * b_e // 3) + T_total * sh.H * 2 + rows * sh.I * 2 * 2
    down = experts * (b_e // 3) + rows * sh.I * 2 * 2 + rows * sh.H * 4
    return gateup, down


def layer_bytes(sh, lookups, calls, pairs, T_total, bias=True):
    """Algorithmic HBM bytes of a layer's compute kernels over `calls` calls
    (the miss copies move host-pool bytes over PCIe and are counted apart):
    the router reads W_r (fp32 H x E) once per call, the token rows and the
    bias, and writes the logits; the expert kernels as in kernel_bytes; the
    combine reads every fp32 expert output row once and writes y in bf16."""
    gu, dn = kernel_bytes(sh, lookups, calls, pairs, T_total)
    rows = pairs + (T_total if sh.shared else 0)
    router = calls * sh.H * sh.E * 4 + T_total * (sh.H * 2 + sh.E * 4 * (2 if bias else 1))
    combine = rows * sh.H * 4 + T_total * sh.H * 2
    return router + gu + dn + combine


# --------------------------------------------------------------- set-up
def make_engine(sh, T, cache_slots, staging_slots, prefill_tokens=0, cache_policy="global"):
    from expert_offload_serving_amd import MoEEngine
    return MoEEngine(sh.H, sh.I, sh.E, sh.k, n_layers=sh.layers, has_shared=sh.shared,
                     renormalize=sh.renormalize, max_tokens=T, cache_slots=cache_slots,
                     staging_slots=staging_slots, max_prefill_tokens=prefill_tokens,
                     cache_policy=cache_policy, weight_format=sh.weights)


def record_of(e, distinct):
    """The generated record expert e holds (all distinct when distinct is 0)."""
    return e if not distinct or e < 0 else e % distinct


def load_weights(eng, sh, seed=0, distinct=None):
    """Router and expert weights of every layer.  distinct = n reuses n
    generated expert records per layer (same sizes and bytes moved, less
    set-up time) where the expert values do not matter."""
    from workload import gen
    for l in range(sh.layers):
        eng.set_router(l, gen.router_weights(sh, l, seed))
        recs = {}
        for e in range(sh.E):
            src = record_of(e, distinct)
            if src not in recs:
                recs[src] = gen.expert_weights_of(sh, l, src, seed)
            eng.set_expert(l, e, recs[src])
            if not distinct:
                recs.clear()
        if sh.shared:
            eng.set_expert(l, -1, gen.expert_weights_of(sh, l, -1, seed))


def bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def decode_inputs(wl, T, n, seed=0):
    """Per layer: activations [n][T][H] (bf16 bits) and router bias [n][T][E]
    on the device, and the same on the host."""
    import torch
    from workload import gen
    sh = wl.shape
    dev = torch.device("cuda")
    xs, bs, hx, hb = [], [], [], []
    for l in range(sh.layers):
        sets = gen.zipf_sets(sh, l, T, n, wl.zipf_s, wl.overlap, seed) if wl.zipf_s else None
        x = np.stack([gen.tokens(sh, l, s, T, seed) for s in range(n)])
        b = np.stack([gen.bias_from_sets(sets[s], sh.E) for s in range(n)]) if sets is not None else None
        hx.append(x)
        hb.append(b)
        xs.append(torch.from_numpy(x.view(np.int16)).to(dev))
        bs.append(torch.from_numpy(b).to(dev) if b is not None else None)
    return xs, bs, hx, hb


# ------------------------------------------------------------ decode runs
def run_decode(wl, T, steps, warmup, seed=0, eng=None, distinct=None, resize_at=None,
               check_pairs=(), prefetch_plan=None, copy_overlap=-1):
    """Decode throughput: W untimed steps, then K timed steps by wall clock
    (host submission included; a cache resize placed at step `resize_at` is
    inside the timed region).  Then a kernel-timing pass over the same K
    steps, queued behind a spin kernel so that the kernels run back to back
    as in the timed pass, in which every kernel carries start and stop
    events recorded by its own dispatch.  Then a check pass: the listed
    (step, layer) pairs again with routing and fp32 outputs read back (the
    outputs do not depend on the cache state).  prefetch_plan: {(step,
    layer): (layer', device int32 experts)} armed before that call."""
    import torch

    sh = wl.shape
    own = eng is None
    if own:
        eng = make_engine(sh, T, wl.cache_slots, wl.staging_slots)
        load_weights(eng, sh, seed, distinct)
    eng.set_copy_overlap(copy_overlap)
    n = warmup + steps
    xs, bs, hx, hb = decode_inputs(wl, T, n, seed)
    y = torch.empty((T, sh.H), dtype=torch.int16, device="cuda")
    resize_to = wl.resize[0][1] if wl.resize else None
    resize_info = {}

    # the first step from the cold cache, by events recorded on the stream
    # (no synchronisation inside a timed region): its first call (every
    # expert a miss, first launches included) and the whole step
    cold_ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if own else None

    def do_step(s, allow_resize=True, mark=False):
        if allow_resize and resize_to is not None and s == resize_at:
            # the resize waits for the queued steps; time only its own work
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            before = eng.stats()
            eng.cache_resize(resize_to)
            after = eng.stats()
            resize_info.update(before_step=s, slots=[wl.cache_slots, resize_to],
                               wall_ms=round(1e3 * (time.perf_counter() - t0), 3),
                               evicted=after["evictions"] - before["evictions"],
                               bytes_d2d=after["bytes_d2d"] - before["bytes_d2d"])
        mark = mark and cold_ev is not None
        for l in range(sh.layers):
            if prefetch_plan is not None and (s, l) in prefetch_plan:
                eng.set_prefetch(*prefetch_plan[(s, l)])
            if mark and l == 0:
                cold_ev[0].record()
            eng.forward(l, xs[l][s], bias=None if bs[l] is None else bs[l][s], y=y)
            if mark and l == 0:
                cold_ev[1].record()
        if mark:
            cold_ev[2].record()

    for s in range(warmup):
        do_step(s, mark=s == 0)
    torch.cuda.synchronize()
    eng.reset_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(warmup, warmup + steps):
        do_step(s, mark=s == 0)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    cold = {}
    if cold_ev is not None and warmup + steps > 0:
        cold = {"first_call_ms": round(cold_ev[0].elapsed_time(cold_ev[1]), 3),
                "first_step_ms": round(cold_ev[0].elapsed_time(cold_ev[2]), 3)}
    st = eng.stats()
    elapsed = t1 - t0
    # kernel-timing pass over the first timed steps, at most TIMING_STEPS of
    # them (every call records 16 events); the cache state continues from
    # the first pass, so the byte counts come from this pass's stats
    n_t = min(steps, TIMING_STEPS)
    eng.reset_stats()
    eng.set_timing(True)
    torch.cuda._sleep(int(2e8))  # ~0.1 s spin: the host queues the steps meanwhile
    for s in range(warmup, warmup + n_t):
        do_step(s, allow_resize=False)
    torch.cuda.synchronize()
    tm = eng.get_timing()
    eng.set_timing(False)
    st2 = eng.stats()
    calls_t = n_t * sh.layers
    pairs_t = calls_t * T * sh.k
    gb, db = kernel_bytes(sh, st2["lookups"], calls_t, pairs_t, calls_t * T)
    lb = layer_bytes(sh, st2["lookups"], calls_t, pairs_t, calls_t * T, bias=wl.zipf_s is not None)
    checked = []
    if check_pairs:
        ids = torch.empty((T, sh.k), dtype=torch.int32, device="cuda")
        gates = torch.empty((T, sh.k), dtype=torch.float32, device="cuda")
        y32 = torch.empty((T, sh.H), dtype=torch.float32, device="cuda")
        for (s, l) in check_pairs:
            eng.forward(l, xs[l][s], bias=None if bs[l] is None else bs[l][s], y=y, ids=ids,
                        gates=gates, y32=y32)
            torch.cuda.synchronize()
            checked.append(dict(step=s, layer=l, x=hx[l][s], bias=None if hb[l] is None else hb[l][s],
                                ids=ids.cpu().numpy(), gates=gates.cpu().numpy(),
                                y32=y32.cpu().numpy(), y=y.cpu().numpy().view(np.uint16)))
    if own:
        eng.close()
    nl = max(tm["n_decode"], 1)
    ms = tm["decode_ms"]
    layer_ms = ms["router"] + ms["finalize"] + ms["gateup"] + ms["down"] + ms["combine"]

    def gbs(nbytes, t_ms):
        return nbytes / (t_ms * 1e6) if t_ms > 0 else None
    # a call whose copies ran beside the resident experts' kernels launched
    # gate/up and down twice: per-launch figures count both launches (as
    # rocprof's per-dispatch averages do); bytes over time is unchanged
    nlaunch = max(tm["n_decode"] + tm.get("n_decode_split", 0), 1)
    return dict(T=T, steps=steps, elapsed_s=elapsed, tokens_per_s=T * steps / elapsed,
                ms_per_step=1e3 * elapsed / steps, stats=st,
                hit_rate=st["hits"] / max(st["lookups"], 1),
                launches=nlaunch, split_calls=tm.get("n_decode_split", 0), calls=tm["n_decode"],
                kernel_us={k: round(1e3 * v / nl, 3) for k, v in ms.items()},
                gateup_us=1e3 * ms["gateup"] / nlaunch, down_us=1e3 * ms["down"] / nlaunch,
                gateup_bytes=gb / nlaunch, down_bytes=db / nlaunch, layer_bytes=lb / nl,
                layer_us=1e3 * layer_ms / nl,
                gateup_gbs=gbs(gb, ms["gateup"]), down_gbs=gbs(db, ms["down"]),
                layer_gbs=gbs(lb, layer_ms),
                h2d_gbs=st["bytes_h2d"] / (elapsed * 1e9),
                fill_gbs=gbs(st2["bytes_h2d"], ms["fill"]),
                resize=resize_info, checked=checked, cold=cold)


def run_decode_graph(wl, T, steps, warmup, seed=0):
    """Decode throughput with every timed step replayed from its own HIP
    graph (captured after the eager warm-up; capture runs nothing), so the
    host's launch work is out of the timed region.  Same inputs, cache and
    kernels as run_decode; the steps run in the same order."""
    import torch

    sh = wl.shape
    assert not wl.resize, "a cache resize cannot be captured"
    eng = make_engine(sh, T, wl.cache_slots, wl.staging_slots)
    load_weights(eng, sh, seed)
    n = warmup + steps
    xs, bs, _, _ = decode_inputs(wl, T, n, seed)
    y = torch.empty((T, sh.H), dtype=torch.int16, device="cuda")

    def do_step(s):
        for l in range(sh.layers):
            if prefetch_plan is not None and (s, l) in prefetch_plan:
                eng.set_prefetch(*prefetch_plan[(s, l)])
            eng.forward(l, xs[l][s], bias=None if bs[l] is None else bs[l][s], y=y)

    for s in range(warmup):
        do_step(s)
    torch.cuda.synchronize()
    graphs = []
    for s in range(warmup, warmup + steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            do_step(s)
        graphs.append(g)
    torch.cuda.synchronize()
    eng.reset_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st = eng.stats()
    eng.close()
    return dict(T=T, steps=steps, tokens_per_s=T * steps / elapsed, ms_per_step=1e3 * elapsed / steps,
                hit_rate=st["hits"] / max(st["lookups"], 1))


def decode_kernels(T):
    """Names of the decode expert kernels the library launches for T tokens:
    the streaming variants up to 16 tokens per call, else the others."""
    if T <= 16:
        return "gateup_stream_kernel", "down_stream_kernel"
    return "gateup_decode_kernel", "down_decode_kernel"


def roofline_entry(name, gbs, us, nbytes, launches, bound="hbm"):
    return {"kernel": name, "bound": bound,
            "achieved": None if gbs is None else round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": None if gbs is None else round(gbs / HBM_PEAK_GBS, 4),
            "launches": launches, "avg_launch_us": round(us, 3), "bytes_per_launch": round(nbytes)}


def layer_entry(r, bound="hbm"):
    """The layer as a whole: algorithmic bytes of its compute kernels over
    the sum of their durations (router, finalize, gate/up, down, combine)."""
    gbs = r["layer_gbs"]
    return {"bound": bound, "achieved": None if gbs is None else round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": None if gbs is None else round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_layer": round(r["layer_bytes"]), "us_per_layer": round(r["layer_us"], 3)}


def decode_summary(r, bound="hbm"):
    kgu, kdn = decode_kernels(r["T"])
    return {"tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 4),
            "hit_rate": round(r["hit_rate"], 4), "h2d_gbs": round(r["h2d_gbs"], 2),
            "fill_kernel_gbs": None if r["fill_gbs"] is None else round(r["fill_gbs"], 2),
            "kernel_us": r["kernel_us"],
            "roofline": [roofline_entry(kgu, r["gateup_gbs"], r["gateup_us"], r["gateup_bytes"],
                                        r["launches"], bound),
                         roofline_entry(kdn, r["down_gbs"], r["down_us"], r["down_bytes"],
                                        r["launches"], bound)],
            "layer": layer_entry(r, bound)}


# ------------------------------------------------------------ context legs
def time_prefill(eng, sh, T, xs, ys, steps, fmt, name, kernels=None):
    """steps timed prefill passes of the whole stack in one mode (after one
    untimed pass): end-to-end rate and the per-stage kernel times.
    kernels: names of the gate/up and down kernels (default: those of the
    mode's grouped GEMMs for MXFP4 experts)."""
    import torch
    eng.set_prefill_format(fmt)
    eng.prefill(xs, ys)
    torch.cuda.synchronize()
    eng.reset_stats()
    eng.set_timing(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        eng.prefill(xs, ys)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tm = eng.get_timing()
    eng.set_timing(False)
    el = t1 - t0
    layers = steps * sh.layers
    # algorithmic flops per layer: 3 matrices of H x I per (token, expert),
    # k routed experts plus the shared one, 2 flops per multiply-add
    flops_layer = 2 * 3 * sh.H * sh.I * T * (sh.k + (1 if sh.shared else 0))
    nl = max(tm["n_prefill"], 1)
    pm = tm["prefill_ms"]
    gu_ms, dn_ms = pm["gateup"] / nl, pm["down"] / nl
    gemm_ms = gu_ms + dn_ms
    tflops = flops_layer / (gemm_ms * 1e9)
    peak = MFMA_FP8_PEAK_TFLOPS if fmt == "mxfp8" else MFMA_BF16_PEAK_TFLOPS
    upload = sh.E * sh.expert_bytes() * layers
    kn = kernels or {"bf16": ("gateup_prefill_kernel", "down_prefill_kernel"),
                     "mxfp8": ("gateup_mx_kernel", "down_mx_kernel")}[fmt]
    return {
        "workload": name, "format": fmt, "T": T, "layers": sh.layers, "steps": steps,
        "tokens_per_s_end_to_end": round(T * steps / el, 1),
        "ms_per_step": round(1e3 * el / steps, 2),
        "gemm_ms_per_layer": round(gemm_ms, 4),
        "stage_us_per_layer": {k: round(1e3 * v / nl, 1) for k, v in pm.items()},
        "gemm_launches": 2 * tm["n_prefill"],
        "tokens_per_s_gemm_only": round(T / (gemm_ms * 1e-3) / sh.layers, 1),
        "flops_per_layer": flops_layer,
        "mfma_tflops": round(tflops, 1),
        "mfma_peak_tflops": peak,
        "mfma_frac": round(tflops / peak, 4),
        kn[0]: {"avg_us": round(1e3 * gu_ms, 1),
                "tflops": round(2 * flops_layer / 3 / (gu_ms * 1e9), 1)},
        kn[1]: {"avg_us": round(1e3 * dn_ms, 1),
                "tflops": round(flops_layer / 3 / (dn_ms * 1e9), 1)},
        "pcie_h2d_gbs": round(upload / (el * 1e9), 2)}


def run_dsv4(prefill_steps, decode_steps, decode_warmup, seed=0, formats=("bf16", "mxfp8")):
    """The DeepSeek-V4-Flash-shaped stack on one engine: prefill of all
    layers per step (layer uploads included) in each prefill mode, then T=1
    and T=32 decode through the global LRU (13.4 MB experts: HBM-bound, not
    cache-resident)."""
    import torch
    from workload import gen
    wp, wd = gen.WORKLOADS["dsv4_prefill"], gen.WORKLOADS["dsv4_decode"]
    sh = wp.shape
    T = wp.Ts[0]
    eng = make_engine(sh, max(wd.Ts), wd.cache_slots, wd.staging_slots, prefill_tokens=T)
    load_weights(eng, sh, seed)
    out = {}
    if prefill_steps > 0:
        xs = [bf16_dev(gen.tokens(sh, l, 0, T, seed)) for l in range(sh.layers)]
        ys = [torch.empty((T, sh.H), dtype=torch.int16, device="cuda") for _ in range(sh.layers)]
        for fmt in formats:
            key = "prefill" if fmt == "bf16" else f"prefill_{fmt}"
            out[key] = time_prefill(eng, sh, T, xs, ys, prefill_steps, fmt, wp.name)
            kn = {"bf16": ("gateup_prefill_kernel", "down_prefill_kernel"),
                  "mxfp8": ("gateup_mx_kernel", "down_mx_kernel")}[fmt]
            xb, hb = (2.0, 2.0 + 13 / 16) if fmt == "bf16" else (1 + 1 / 32, 1 + 1 / 32)
            out[key]["hbm"] = prefill_streamed_hbm(sh, T, out[key], kn, xb, hb)
            log(f"prefill {fmt}: {out[key]['mfma_tflops']} TFLOP/s "
                f"({out[key]['mfma_frac']:.3f} of {out[key]['mfma_peak_tflops']})")
        # matrix-core busy share by counters (profiles/mfma_busy_*.md)
        if "prefill" in out:
            out["prefill"]["mfma_busy_counters"] = mfma_busy_from_profile()
        if "prefill_mxfp8" in out:
            out["prefill_mxfp8"]["mfma_busy_counters"] = mfma_busy_from_profile(
                ("gateup_mx_kernel", "down_mx_kernel"))
        eng.set_prefill_format("bf16")
    if decode_steps > 0:
        r = run_decode(wd, 1, decode_steps, decode_warmup, seed, eng=eng)
        out["dsv4_decode_T1"] = decode_summary(r)
        # T = 32 from an emptied cache: about 87 unique experts per layer
        # against 256 slots over 4 layers, so most lookups miss (PCIe-bound);
        # the kernels for more than 16 tokens per call
        eng.cache_reset()
        n32 = max(decode_steps // 8, 16)
        r = run_decode(wd, 32, n32, max(n32 // 4, 4), seed, eng=eng)
        out["dsv4_decode_T32"] = decode_summary(r)
    eng.close()
    return out


def prefill_streamed_hbm(sh, T, r, kernels, x_bytes=2.0, h_bytes=4.0):
    """HBM roofline of a pair of prefill GEMMs: algorithmic bytes per layer
    over each kernel's time.  The bytes: every expert's weights once (at
    T*k/E rows per expert all are routed; the shared expert's weights, which
    each of its T/128 tiles reads, count once), the token rows once, h written
    by gate/up and read by down, the fp32 expert outputs.  x_bytes and h_bytes
    are the bytes per element of x and h as the GEMMs move them: bf16 x with
    h as two bf16 planes (bf16 and NVFP4 experts: 2, 4), bf16 x with h as a
    bf16 plane plus its fp6 remainder records (2, 2 + 13/16), MXFP8 x and h
    (1 + 1/32 each).  flops_per_weight_byte against the matrix cores' ridge
    (peak flops over 8 TB/s: 312 for bf16, 625 for fp8) says which bound
    applies: below it the GEMMs are bounded by HBM."""
    rows = T * sh.k + (T if sh.shared else 0)
    n_exp = sh.E + (1 if sh.shared else 0)
    wbytes = sh.expert_bytes() * n_exp
    gu_w, dn_w = wbytes * 2 / 3, wbytes / 3
    gu = gu_w + T * sh.H * x_bytes + rows * sh.I * h_bytes
    dn = dn_w + rows * sh.I * h_bytes + rows * sh.H * 4
    gu_us = r[kernels[0]]["avg_us"]
    dn_us = r[kernels[1]]["avg_us"]
    f = lambda b, us: round(b / (us * 1e3) / HBM_PEAK_GBS, 4)
    return {"bytes_gateup": round(gu), "bytes_down": round(dn), "peak_gbs": HBM_PEAK_GBS,
            "gateup_frac": f(gu, gu_us), "down_frac": f(dn, dn_us),
            "layer_frac": f(gu + dn, gu_us + dn_us),
            "flops_per_weight_byte": round(r["flops_per_layer"] / wbytes, 1),
            "ridge_flops_per_byte": round(r["mfma_peak_tflops"] * 1e12 / (HBM_PEAK_GBS * 1e9), 1)}


def run_prefill_formats(steps, T=4096, layers=2, seed=0, formats=("bf16", "nvfp4")):
    """Prefill with bf16 and NVFP4 experts on a 35B-A3B-shaped stack (H=2048,
    I=512, E=256, top-8): the grouped bf16 GEMMs of each format (NVFP4 is
    dequantised to bf16 on its way from LDS to the matrix cores).  Eight
    generated records per layer are reused for all 256 experts; the routing
    is the layer's own, so every expert is uploaded and run."""
    import torch
    from dataclasses import replace
    from workload import gen
    out = {}
    for w in formats:
        sh = replace(gen.WORKLOADS["a3b_decode"].shape, layers=layers, weights=w)
        eng = make_engine(sh, 1, 0, sh.k, prefill_tokens=T)
        load_weights(eng, sh, seed, distinct=8)
        xs = [bf16_dev(gen.tokens(sh, l, 0, T, seed)) for l in range(sh.layers)]
        ys = [torch.empty((T, sh.H), dtype=torch.int16, device="cuda") for _ in range(sh.layers)]
        kn = {"bf16": ("gateup_prefill_bw_kernel", "down_prefill_bw_kernel"),
              "nvfp4": ("gateup_prefill_nv_kernel", "down_prefill_nv_kernel")}[w]
        r = time_prefill(eng, sh, T, xs, ys, steps, "bf16", f"a3b_prefill_{w}", kernels=kn)
        r["weights"] = w
        r["hbm"] = prefill_streamed_hbm(sh, T, r, kn)
        out[f"prefill_{w}_experts"] = r
        log(f"prefill with {w} experts: {r['mfma_tflops']} TFLOP/s ({r['mfma_frac']:.3f} of "
            f"{r['mfma_peak_tflops']})")
        eng.close()
    return out


def run_a3b(steps, warmup, extra_T, graph_T, seed=0):
    """The 35B-A3B-shaped layer from a cold 64-slot cache: T=16 and the
    extra T.  Its 107 MB cache fits the 256 MB Infinity Cache, so the kernel
    rates are labelled as MALL rates."""
    from workload import gen
    wl = gen.WORKLOADS["a3b_decode"]
    out = {}
    for T in [16] + [t for t in extra_T if t != 16 and t in wl.Ts]:
        r = run_decode(wl, T, steps, warmup, seed)
        out[f"T={T}"] = decode_summary(r, bound="mall")
    for T in graph_T:
        if T in wl.Ts:
            r = run_decode_graph(wl, T, steps, warmup, seed)
            out[f"graph_T={T}"] = {"tokens_per_s": round(r["tokens_per_s"], 1),
                                   "ms_per_step": round(r["ms_per_step"], 4),
                                   "hit_rate": round(r["hit_rate"], 4)}
    return out


def policy_study(steps, warmup, seed=0):
    """Decode of the DeepSeek-V4-Flash-shaped stack (4 layers, 256 experts of
    13.4 MB, 256 slots = a quarter of each layer's experts) under each cache
    placement policy at equal capacity, T = 1 and 32, each run from a fresh
    engine: the global LRU, per-layer shares of 64 slots, and a static set
    (each layer's 64 most popular experts under the trace's ranking, placed
    before the run; every other expert bypasses through staging)."""
    from workload import gen
    wl = gen.WORKLOADS["dsv4_decode"]
    sh = wl.shape
    rows = []
    for policy in ("global", "per_layer", "static"):
        for T in wl.Ts:
            eng = make_engine(sh, T, wl.cache_slots, wl.staging_slots, cache_policy=policy)
            load_weights(eng, sh, seed, distinct=8)
            if policy == "static":
                per = wl.cache_slots // sh.layers
                for l in range(sh.layers):
                    top = sorted(gen.popularity_order(sh, l, seed)[:per].tolist())
                    for i in range(0, per, T * sh.k):
                        eng.cache_fill(l, top[i:i + T * sh.k])
            eng.reset_stats()
            r = run_decode(wl, T, steps, warmup, seed, eng=eng)
            st = r["stats"]
            n = max(st["lookups"], 1)
            rows.append({"policy": policy, "T": T, "hit_rate": round(st["hits"] / n, 4),
                         "fill_rate": round(st["fills"] / n, 4),
                         "bypass_rate": round(st["bypasses"] / n, 4),
                         "tokens_per_s": round(r["tokens_per_s"], 1),
                         "ms_per_step": round(r["ms_per_step"], 3),
                         "h2d_gbs": round(r["h2d_gbs"], 2)})
            print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
            eng.close()
    return {"policy_study": rows, "config": {"workload": wl.name, "layers": sh.layers, "E": sh.E,
            "k": sh.k, "cache_slots": wl.cache_slots, "staging_slots": wl.staging_slots,
            "steps": steps, "warmup": warmup, "zipf_s": wl.zipf_s, "overlap": wl.overlap}}


def prefetch_plans(wl, T, n, seed=0):
    """Predicted expert sets of the call after each (step, layer) of a decode
    trace, as device lists, for the prefetch study.  Computed from the
    workload generator before any timing:
      exact   - the next call's drawn sets (its routing under the trace's
                bias): a perfect predictor, the most a prefetch can give;
      half    - each of those experts kept with probability 1/2, else
                replaced by a uniformly drawn other expert;
      popular - the next layer's most popular experts under the trace's
                ranking, as many as T * k (activation statistics);
      random  - as many uniformly drawn experts as the exact set has."""
    import torch
    from workload import gen
    sh = wl.shape
    sets = [gen.zipf_sets(sh, l, T, n, wl.zipf_s, wl.overlap, seed) for l in range(sh.layers)]
    rng = np.random.default_rng(seed + 99)
    m = min(T * sh.k, sh.E)
    popular = [torch.tensor(sorted(gen.popularity_order(sh, l, seed)[:m].tolist()),
                            dtype=torch.int32, device="cuda") for l in range(sh.layers)]
    plans = {k: {} for k in ("exact", "half", "popular", "random")}
    for st in range(n):
        for l in range(sh.layers):
            nl, ns = (l + 1) % sh.layers, st + (1 if l + 1 == sh.layers else 0)
            if ns >= n:
                continue
            true = sorted(set(sets[nl][ns].ravel().tolist()))
            others = np.setdiff1d(np.arange(sh.E), true)
            half = [e if rng.random() < 0.5 else int(rng.choice(others)) for e in true]
            rnd = rng.choice(sh.E, len(true), replace=False).tolist()
            for k, lst in (("exact", true), ("half", sorted(set(half))), ("random", sorted(rnd))):
                plans[k][(st, l)] = (nl, torch.tensor(lst, dtype=torch.int32, device="cuda"))
            plans["popular"][(st, l)] = (nl, popular[nl])
    return plans


def prefetch_study(steps, warmup, seed=0, kinds=("none", "exact", "half", "popular", "random"),
                   caps=None):
    """The GLM-5.2-shaped decode (T = 1, 8 layers, 20 MB experts) at two
    cache capacities (60% and 30% of the experts, no resize inside a run),
    each run from an empty cache: without prefetch, and with each layer's
    call prefetching the next call's experts as predicted by prefetch_plans."""
    from dataclasses import replace
    from workload import gen
    wl = replace(gen.WORKLOADS["glm_decode"], resize=())
    sh = wl.shape
    T = 1
    eng = make_engine(sh, T, wl.cache_slots, wl.staging_slots)
    load_weights(eng, sh, seed, distinct=8)
    plans = prefetch_plans(wl, T, warmup + steps, seed)
    rows = []
    for cap in caps or (wl.cache_slots, wl.cache_slots // 2):
        for kind in kinds:
            eng.cache_resize(cap)
            eng.cache_reset()
            r = run_decode(replace(wl, cache_slots=cap), T, steps, warmup, seed, eng=eng,
                           prefetch_plan=None if kind == "none" else plans[kind])
            st = r["stats"]
            n = max(st["lookups"], 1)
            rows.append({"cache_slots": cap, "predictor": kind,
                         "tokens_per_s": round(r["tokens_per_s"], 1),
                         "ms_per_step": round(r["ms_per_step"], 3),
                         "hit_rate": round(st["hits"] / n, 4),
                         "prefetch_fills_per_call": round(st["prefetch_fills"] /
                                                          (steps * sh.layers), 3),
                         "prefetch_hit_rate": round(st["prefetch_hits"] /
                                                    max(st["prefetch_lookups"], 1), 4),
                         "h2d_gbs": round(r["h2d_gbs"], 2)})
            print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    eng.close()
    return {"prefetch_study": rows, "config": {"workload": wl.name, "T": T, "layers": sh.layers,
            "E": sh.E, "k": sh.k, "shared_expert": sh.shared, "steps": steps, "warmup": warmup,
            "zipf_s": wl.zipf_s, "overlap": wl.overlap, "expert_records_per_layer": 8}}


# ------------------------------------------------------ oracle on the sample
def check_pairs_of(wl, warmup, steps, n_pairs):
    """(step, layer) pairs spread over the timed steps and the layers (the
    last timed step is always one of them)."""
    L = wl.shape.layers
    if n_pairs <= 0 or steps <= 0:
        return []
    out = []
    for i in range(n_pairs):
        s = warmup + steps - 1 - (i * steps) // n_pairs
        out.append((s, (L - 1 - (i * max(L - 1, 1)) // max(n_pairs - 1, 1)) % L))
    return sorted(set(out))


def oracle_pair(sh, pair, routers, records, shared_recs):
    """The CPU oracle on one (step, layer) pair: routing, dispatch and the
    per-token expert loops, each expert dequantised where it is used."""
    import oracle
    from oracle import experts as oexp
    from workload import gen
    l = pair["layer"]
    x = gen.bf16_bits_to_f32(pair["x"])
    lg, ids, g = oracle.route(x, routers[l], sh.k, pair["bias"], sh.renormalize)
    oracle.permutation(ids, sh.E)
    shared = oexp.dequant_expert(shared_recs[l]) if sh.shared else None
    y = oracle.moe_layer(x, ids, g, lambda e: oexp.dequant_expert(records[l][e]), shared=shared)
    return ids, g, y


def cpu_baseline(wl, checked, seconds, distinct, seed=0):
    """The oracle as it stands on the check pass's sample: timed on all the
    threads numpy may use, plus one pair on one thread; and compared with the
    GPU's results for the same pairs (routing bit for bit, gates, fp32
    outputs against 2e-2 x rms)."""
    from workload import gen
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = len(os.sched_getaffinity(0))
    sh = wl.shape
    routers = {p["layer"]: gen.router_weights(sh, p["layer"], seed) for p in checked}
    records = {}
    for p in checked:
        l = p["layer"]
        recs = records.setdefault(l, {})
        for e in range(sh.E):
            if record_of(e, distinct) not in recs:
                recs[record_of(e, distinct)] = gen.expert_weights_of(sh, l, record_of(e, distinct), seed)
    by_expert = {l: {e: records[l][record_of(e, distinct)] for e in range(sh.E)} for l in records}
    shared = {l: gen.expert_weights_of(sh, l, -1, seed) for l in records} if sh.shared else {}
    done, worst, ids_ok, gates_ok = 0, 0.0, True, True
    t0 = time.perf_counter()
    for p in checked:
        if done and time.perf_counter() - t0 > seconds:
            break
        ids, g, y = oracle_pair(sh, p, routers, by_expert, shared)
        ids_ok &= bool(np.array_equal(ids, p["ids"]))
        gates_ok &= bool(np.max(np.abs(g - p["gates"])) <= 1e-6)
        rms = float(np.sqrt(np.mean(y ** 2)))
        worst = max(worst, float(np.max(np.abs(p["y32"].astype(np.float64) - y))) / rms)
        done += 1
    el = time.perf_counter() - t0
    T = p["x"].shape[0]
    one = None
    if threadpool_limits is not None and checked:
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            oracle_pair(sh, checked[0], routers, by_expert, shared)
            one = time.perf_counter() - t1
    L = sh.layers
    base = {"value": round(T * done / L / el, 4), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} (step, layer) pairs of {wl.name} at T={T} (routing, dispatch, "
                      f"per-token fp64 expert loops with each expert dequantised where used) in "
                      f"{el:.1f}s; a token is {L} layer-steps",
            "one_thread": None if one is None else {"value": round(T / L / one, 4),
                                                    "unit": "tokens/s", "cores": 1,
                                                    "sample": "the first pair on one thread"}}
    parity = {"pairs": [(p["step"], p["layer"]) for p in checked[:done]], "ids_exact": ids_ok,
              "gates_within_1e-6": gates_ok, "max_err_over_rms": round(worst, 8),
              "tolerance": 2e-2, "ok": bool(ids_ok and gates_ok and worst <= 2e-2)}
    return base, parity


# ---------------------------------------------------------------- profiles
def profile_fields(name):
    """The `- key: value` fields of a committed counter summary in profiles/,
    or None when the file is missing or was taken on another version of the
    source file it names (its source_sha256)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].strip().split(": ", 1)
            fields[k.strip("`")] = v.strip().strip("`")
    src = os.path.join(ROOT, fields.get("source", ""))
    if not os.path.isfile(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != fields.get("source_sha256"):
        return None
    return fields


def mfma_busy_from_profile(kernels=("gateup_prefill_kernel", "down_prefill_kernel")):
    """Matrix-core busy share (SQ_VALU_MFMA_BUSY_CYCLES per SIMD over
    GRBM_GUI_ACTIVE per XCD) of prefill GEMMs from the committed counter
    summary, or None."""
    f = profile_fields("mfma_busy_prefill_dsv4_T4096.md")
    if f is None:
        return None
    try:
        return {k: float(f["busy_" + k]) for k in kernels}
    except (KeyError, ValueError):
        return None


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/traffic_<kernel>_<workload>.md), if it was taken on the current
    source of the kernel's file; else None."""
    f = profile_fields(f"traffic_{kernel}_{workload}.md")
    try:
        return int(f["hbm_bytes_per_launch"]) if f else None
    except (KeyError, ValueError):
        return None


def probe_bandwidth(mb=1024, reps=3):
    """Reference rates for the two links the path moves bytes over: a pinned
    host buffer copied to the device by the DMA engines (hipMemcpyAsync via
    torch; the fill kernel's PCIe rate is set against it), and the library's
    device-to-device copy kernel (bytes read plus bytes written per second).
    Best of `reps` copies of `mb` MiB each, timed with HIP events."""
    import torch
    from expert_offload_serving_amd import binding
    n = mb << 20
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    dev = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(dev)

    def best(fn):
        t = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            t.append(e0.elapsed_time(e1))
        return min(t)
    h2d_ms = best(lambda: dev.copy_(host, non_blocking=True))
    d2d_ms = best(lambda: binding.moe_probe_copy(dev.data_ptr(), dst.data_ptr(), n))
    del host, dev, dst
    return {"pcie_h2d_peak_gbs": round(n / (h2d_ms * 1e6), 2),
            "copy_kernel_gbs": round(2 * n / (d2d_ms * 1e6), 1), "mib": mb,
            "how": "best of 3: pinned host -> device DMA copy; library copy kernel "
                   "device -> device, read + write bytes"}


def calibrate_copy(mb):
    """One plain device-to-device copy of `mb` MiB through the library's copy
    kernel, for scaling traffic counters to bytes."""
    import torch
    from expert_offload_serving_amd import binding
    n = mb << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    binding.moe_probe_copy(src.data_ptr(), dst.data_ptr(), n)
    torch.cuda.synchronize()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    from dataclasses import replace
    from workload import gen
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.prefetch_study > 0:
        print(json.dumps(prefetch_study(
            a.prefetch_study, min(a.warmup or 16, a.prefetch_study),
            kinds=tuple(k for k in a.prefetch_kinds.split(",") if k),
            caps=tuple(int(v) for v in a.prefetch_slots.split(",") if v) or None)), flush=True)
        return
    if a.policy_study > 0:
        print(json.dumps(policy_study(a.policy_study, min(a.warmup or 16, a.policy_study))),
              flush=True)
        return
    legs = {v.strip() for v in a.legs.split(",") if v.strip()}
    line = {}
    wl = gen.WORKLOADS[a.workload]
    if a.weights != "mxfp4":
        wl = replace(wl, name=f"{wl.name}_{a.weights}", shape=replace(wl.shape, weights=a.weights))
    W0, K0 = DEFAULT_STEPS.get(a.workload, (32, 512))
    W = W0 if a.warmup is None else a.warmup
    K = K0 if a.steps is None else a.steps
    if "headline" in legs:
        T = a.T or max(wl.Ts)
        sh = wl.shape
        resize_at = W + K // 2 if wl.resize else None
        pairs = check_pairs_of(wl, W, K, 0 if a.no_cpu_baseline else a.check_pairs)
        log(f"headline {wl.name} T={T}: {W} warm-up + {K} timed steps (loading the expert pool)")
        res = run_decode(wl, T, K, W, distinct=a.distinct, resize_at=resize_at, check_pairs=pairs,
                         copy_overlap=a.copy_overlap)
        log(f"headline done: {res['tokens_per_s']:.1f} tokens/s")
        kgu, kdn = decode_kernels(T)
        roof = roofline_entry(kgu, res["gateup_gbs"], res["gateup_us"], res["gateup_bytes"],
                              res["launches"])
        roof["traffic"] = traffic_from_profile(kgu, f"{wl.name}_T{T}")
        roof["other_kernels"] = [roofline_entry(kdn, res["down_gbs"], res["down_us"],
                                                res["down_bytes"], res["launches"])]
        roof["layer"] = layer_entry(res)
        cfg = {"workload": wl.name, "T": T, "H": sh.H, "I": sh.I, "E": sh.E, "k": sh.k,
               "layers": sh.layers, "shared_expert": sh.shared, "cache_slots": wl.cache_slots,
               "staging_slots": wl.staging_slots,
               "weights": ("MXFP4 (E2M1 + E8M0/32)" if sh.weights == "mxfp4" else sh.weights),
               "zipf_s": wl.zipf_s, "overlap": wl.overlap, "cold_start": True,
               "expert_records_per_layer": a.distinct or sh.E}
        if wl.resize:
            cfg["resize"] = {"to_slots": wl.resize[0][1], "before_step": resize_at}
        line.update({
            "metric": "MoE-layer decode tokens/s",
            "value": round(res["tokens_per_s"], 2),
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": K,
            "warmup": W,
            "ms_per_step": round(res["ms_per_step"], 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": cfg,
            "roofline": roof,
            "kernel_us_per_layer": res["kernel_us"],
            "cache": {"hit_rate": round(res["hit_rate"], 4), **{k: res["stats"][k] for k in
                      ("lookups", "hits", "fills", "bypasses", "evictions", "bytes_d2d")}},
            "resize": res["resize"] or None,
            "pcie_h2d_gbs": round(res["h2d_gbs"], 2),
            "cold_start": res["cold"] or None,
            "copy_overlap": {"split_calls": res["split_calls"], "timed_calls": res["calls"]},
            "fill_kernel_gbs": None if res["fill_gbs"] is None else round(res["fill_gbs"], 2),
        })
        if not a.no_cpu_baseline and res["checked"]:
            log("oracle on the check pairs")
            base, parity = cpu_baseline(wl, res["checked"], a.cpu_seconds, a.distinct)
            line["cpu_baseline"] = base
            line["parity"] = parity
        line["probes"] = probe_bandwidth()
    if not a.no_context and a.weights == "mxfp4":
        ctx = line.setdefault("context", {})
        if "a3b" in legs:
            log("context: 35B-A3B-shaped layer")
            ctx["a3b_decode"] = run_a3b(
                K if a.steps is not None else DEFAULT_STEPS["a3b_decode"][1],
                W if a.warmup is not None else DEFAULT_STEPS["a3b_decode"][0],
                [int(v) for v in a.extra_T.split(",") if v.strip()],
                [int(v) for v in a.graph_T.split(",") if v.strip()])
        if "dsv4" in legs and (a.prefill_steps > 0 or a.dsv4_decode_steps > 0):
            log("context: DeepSeek-V4-Flash-shaped stack")
            ctx.update(run_dsv4(a.prefill_steps, a.dsv4_decode_steps,
                                max(a.dsv4_decode_steps // 4, 1),
                                formats=tuple(f for f in a.prefill_formats.split(",") if f)))
        if "formats" in legs and a.prefill_steps > 0:
            log("context: prefill with bf16 and NVFP4 experts")
            ctx.update(run_prefill_formats(a.prefill_steps))
    if a.calibrate_copy_mb > 0:
        calibrate_copy(a.calibrate_copy_mb)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
