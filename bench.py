"""Benchmark of the routed MoE expert-layer forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--T T]
                [--prefill-steps P] [--dsv4-decode-steps D] [--calibrate-copy-mb M]

A step is one decode call per layer of the workload (router, top-k, dispatch,
cache lookup, miss fills, expert FFN, combine) for a batch of T tokens, with
all inputs already resident in HBM.  Default workload: the 35B-A3B-shaped
decode layer (H=2048, E=256, top-8, I=512, MXFP4 experts, bf16 activations,
64-slot LRU from a cold start, Zipf(1.1) routing with 60% step overlap), T=16.
The roofline object is the gate/up expert kernel's (the dominant HBM-bound
kernel; the miss-fill kernel is bound by PCIe and reported as pcie_h2d_gbs),
from per-kernel HIP events taken in a second pass: the library launches
each expert kernel with start and stop events recorded by the dispatch
itself, so an interval is the kernel's own duration.  The line also carries the DeepSeek-V4-Flash-shaped stack (4 layers,
H=4096, I=2048, E=256, top-6 + shared): prefill of T=4096 with whole-layer
uploads from the pinned pool (grouped-GEMM time and MFMA utilisation), and
T=1 decode through its global LRU.
With --graph-T, `graph_replay` repeats the decode workload at those T with
each timed step replayed from its own HIP graph; `value` is always the
eager, host-submitted rate.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="a3b_decode")
    ap.add_argument("--T", type=int, default=None, help="tokens per step (default: largest of the workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--extra-T", default="1,4", help="also time these T (decode)")
    ap.add_argument("--graph-T", default="",
                    help="also time these T with every step replayed from a HIP graph "
                         "(e.g. 1,4,16; default: none)")
    ap.add_argument("--prefill-steps", type=int, default=3,
                    help="prefill passes of the DeepSeek-V4-Flash-shaped stack (0: skip)")
    ap.add_argument("--dsv4-decode-steps", type=int, default=256,
                    help="T=1 decode steps of the DeepSeek-V4-Flash-shaped stack (0: skip)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="also run one plain copy of this many MiB (counter calibration)")
    ap.add_argument("--weights", choices=("mxfp4", "bf16"), default="mxfp4",
                    help="expert format of the decode workload (bf16: decode only, no "
                         "DeepSeek-V4-Flash legs)")
    ap.add_argument("--policy-study", type=int, default=0, metavar="STEPS",
                    help="instead of the benchmark line: DeepSeek-V4-Flash-shaped decode under "
                         "each cache placement policy (STEPS timed steps per run)")
    return ap.parse_args()


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


def make_engine(sh, T, cache_slots, staging_slots, prefill_tokens=0, cache_policy="global"):
    from expert_offload_serving_amd import MoEEngine
    return MoEEngine(sh.H, sh.I, sh.E, sh.k, n_layers=sh.layers, has_shared=sh.shared,
                     renormalize=sh.renormalize, max_tokens=T, cache_slots=cache_slots,
                     staging_slots=staging_slots, max_prefill_tokens=prefill_tokens,
                     cache_policy=cache_policy, weight_format=sh.weights)


def load_weights(eng, sh, seed=0, distinct=None):
    """Router and expert weights of every layer.  distinct = n reuses n
    generated expert records per layer (same sizes and bytes moved, less
    set-up time) where the expert values do not matter."""
    from workload import gen
    for l in range(sh.layers):
        eng.set_router(l, gen.router_weights(sh, l, seed))
        recs = {}
        for e in range(sh.E):
            src = e if distinct is None else e % distinct
            if src not in recs:
                recs[src] = gen.expert_weights_of(sh, l, src, seed)
            eng.set_expert(l, e, recs[src])
            if distinct is None:
                recs.clear()
        if sh.shared:
            eng.set_expert(l, -1, gen.expert_weights_of(sh, l, -1, seed))


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


def bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def decode_inputs(wl, T, n, seed=0):
    import torch
    from workload import gen
    sh = wl.shape
    dev = torch.device("cuda")
    xs, bs = [], []
    for l in range(sh.layers):
        sets = gen.zipf_sets(sh, l, T, n, wl.zipf_s, wl.overlap, seed) if wl.zipf_s else None
        xs.append(torch.stack([bf16_dev(gen.tokens(sh, l, s, T, seed)) for s in range(n)]))
        bs.append(torch.from_numpy(np.stack([gen.bias_from_sets(sets[s], sh.E) for s in range(n)])).to(dev)
                  if sets is not None else None)
    return xs, bs


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
    n = min(wl.steps, steps + warmup)
    xs, bs = decode_inputs(wl, T, n, seed)
    y = torch.empty((T, sh.H), dtype=torch.int16, device="cuda")

    def do_step(s):
        for l in range(sh.layers):
            eng.forward(l, xs[l][s % n], bias=None if bs[l] is None else bs[l][s % n], y=y)

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


def run_decode(wl, T, steps, warmup, seed=0, eng=None):
    """Decode throughput (wall clock over `steps` steps, host submission
    included), then a kernel-timing pass over the same number of steps, in
    which each expert kernel carries HIP start and stop events recorded by
    its dispatch (queued behind a spin kernel, so that the kernels also run
    back to back as in the timed pass and not at the host's pace)."""
    import torch

    sh = wl.shape
    own = eng is None
    if own:
        eng = make_engine(sh, T, wl.cache_slots, wl.staging_slots)
        load_weights(eng, sh, seed)
    n = min(wl.steps, steps + warmup)
    xs, bs = decode_inputs(wl, T, n, seed)
    y = torch.empty((T, sh.H), dtype=torch.int16, device="cuda")
    resize = dict(wl.resize)

    def do_step(s):
        if s in resize:
            eng.cache_resize(resize[s])
        for l in range(sh.layers):
            eng.forward(l, xs[l][s % n], bias=None if bs[l] is None else bs[l][s % n], y=y)

    for s in range(warmup):
        do_step(s)
    torch.cuda.synchronize()
    eng.reset_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(warmup, warmup + steps):
        do_step(s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    st = eng.stats()
    elapsed = t1 - t0
    calls = steps * sh.layers
    pairs = calls * T * sh.k
    gb, db = kernel_bytes(sh, st["lookups"], calls, pairs, calls * T)
    # kernel-timing pass over the same step range (the cache state differs:
    # it continues from the first pass, so the byte count is recomputed)
    eng.reset_stats()
    eng.set_timing(True)
    torch.cuda._sleep(int(2e8))  # ~0.1 s spin: the host queues the steps meanwhile
    for s in range(warmup, warmup + steps):
        do_step(s)
    torch.cuda.synchronize()
    tm = eng.get_timing()
    eng.set_timing(False)
    st2 = eng.stats()
    gb2, db2 = kernel_bytes(sh, st2["lookups"], calls, pairs, calls * T)
    if own:
        eng.close()
    nl = max(tm["n_decode"], 1)
    return dict(T=T, steps=steps, elapsed_s=elapsed, tokens_per_s=T * steps / elapsed,
                ms_per_step=1e3 * elapsed / steps, stats=st,
                hit_rate=st["hits"] / max(st["lookups"], 1),
                launches=tm["n_decode"],
                gateup_us=1e3 * tm["ms_decode_gateup"] / nl, down_us=1e3 * tm["ms_decode_down"] / nl,
                gateup_bytes=gb2 / nl, down_bytes=db2 / nl,
                gateup_gbs=gb2 / (tm["ms_decode_gateup"] * 1e6) if tm["ms_decode_gateup"] > 0 else None,
                down_gbs=db2 / (tm["ms_decode_down"] * 1e6) if tm["ms_decode_down"] > 0 else None,
                ffn_gbs=(gb2 + db2) / (tm["ms_decode"] * 1e6) if tm["ms_decode"] > 0 else None,
                h2d_gbs=st["bytes_h2d"] / (elapsed * 1e9))


def decode_kernels(T):
    """Names of the decode expert kernels the library launches for T tokens:
    the streaming variants up to 16 tokens per call, else the others."""
    if T <= 16:
        return "gateup_stream_kernel", "down_stream_kernel"
    return "gateup_decode_kernel", "down_decode_kernel"


def roofline_entry(name, gbs, us, nbytes, launches):
    return {"kernel": name, "bound": "hbm",
            "achieved": None if gbs is None else round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": None if gbs is None else round(gbs / HBM_PEAK_GBS, 4),
            "launches": launches, "avg_launch_us": round(us, 3), "bytes_per_launch": round(nbytes)}


def run_dsv4(prefill_steps, decode_steps, decode_warmup, seed=0):
    """The DeepSeek-V4-Flash-shaped stack on one engine: prefill of all
    layers per step (layer uploads included), then T=1 decode through the
    global LRU (13.4 MB experts: HBM-bound, not cache-resident)."""
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
        eng.prefill(xs, ys)
        torch.cuda.synchronize()
        eng.reset_stats()
        eng.set_timing(True)
        t0 = time.perf_counter()
        for _ in range(prefill_steps):
            eng.prefill(xs, ys)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        tm = eng.get_timing()
        eng.set_timing(False)
        el = t1 - t0
        layers = prefill_steps * sh.layers
        # algorithmic flops per layer: 3 matrices of H x I per (token, expert),
        # k routed experts plus the shared one, 2 flops per multiply-add
        flops_layer = 2 * 3 * sh.H * sh.I * T * (sh.k + (1 if sh.shared else 0))
        nl = max(tm["n_prefill"], 1)
        gemm_ms = tm["ms_prefill"] / nl
        gu_ms, dn_ms = tm["ms_prefill_gateup"] / nl, tm["ms_prefill_down"] / nl
        tflops = flops_layer / (gemm_ms * 1e9)
        upload = sh.E * sh.expert_bytes() * layers
        out["prefill"] = {
            "workload": wp.name, "T": T, "layers": sh.layers, "steps": prefill_steps,
            "tokens_per_s_end_to_end": round(T * prefill_steps / el, 1),
            "ms_per_step": round(1e3 * el / prefill_steps, 2),
            "gemm_ms_per_layer": round(gemm_ms, 4),
            "gemm_launches": 2 * tm["n_prefill"],
            "tokens_per_s_gemm_only": round(T / (gemm_ms * 1e-3) / sh.layers, 1),
            "flops_per_layer": flops_layer,
            "mfma_tflops": round(tflops, 1),
            "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            # matrix-core busy share by counters (profiles/mfma_busy_*.md)
            "mfma_busy_counters": mfma_busy_from_profile(),
            "gateup_prefill_kernel": {"avg_us": round(1e3 * gu_ms, 1),
                                      "tflops": round(2 * flops_layer / 3 / (gu_ms * 1e9), 1)},
            "down_prefill_kernel": {"avg_us": round(1e3 * dn_ms, 1),
                                    "tflops": round(flops_layer / 3 / (dn_ms * 1e9), 1)},
            "pcie_h2d_gbs": round(upload / (el * 1e9), 2)}
    if decode_steps > 0:
        r = run_decode(wd, 1, decode_steps, decode_warmup, seed, eng=eng)
        out["dsv4_decode_T1"] = {
            "tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 4),
            "hit_rate": round(r["hit_rate"], 4), "h2d_gbs": round(r["h2d_gbs"], 2),
            "roofline": [roofline_entry(decode_kernels(1)[0], r["gateup_gbs"], r["gateup_us"],
                                        r["gateup_bytes"], r["launches"]),
                         roofline_entry(decode_kernels(1)[1], r["down_gbs"], r["down_us"],
                                        r["down_bytes"], r["launches"])]}
    eng.close()
    return out


def cpu_baseline(wl, T, seconds):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import oracle
    from tests import harness as hz
    from workload import gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    sh = wl.shape
    model = hz.Model(sh)
    sets = [gen.zipf_sets(sh, l, T, 64, wl.zipf_s, wl.overlap, 0) if wl.zipf_s else None
            for l in range(sh.layers)]
    cache = oracle.SlotCache(wl.cache_slots, sh.E)
    t0 = time.perf_counter()
    done = 0
    while time.perf_counter() - t0 < seconds and done < 64:
        for l in range(sh.layers):
            x = gen.bf16_bits_to_f32(gen.tokens(sh, l, done, T, 0))
            bias = gen.bias_from_sets(sets[l][done], sh.E) if sets[l] is not None else None
            _, ids, g = model.route(l, x, bias)
            cache.lookup(l, oracle.permutation(ids, sh.E)["unique"])
            model.layer_out(l, x, ids, g)
        done += 1
    el = time.perf_counter() - t0
    return {"value": round(T * done / el, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} steps x T={T} of {wl.name} (routing, LRU simulation, per-token "
                      f"fp64 expert loops) in {el:.1f}s"}


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


def mfma_busy_from_profile():
    """Matrix-core busy share (SQ_VALU_MFMA_BUSY_CYCLES per SIMD over
    GRBM_GUI_ACTIVE per XCD) of the two prefill GEMMs from the committed
    counter summary, or None."""
    f = profile_fields("mfma_busy_prefill_dsv4_T4096.md")
    if f is None:
        return None
    try:
        return {k: float(f["busy_" + k]) for k in ("gateup_prefill_kernel", "down_prefill_kernel")}
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


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    from workload import gen
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.policy_study > 0:
        print(json.dumps(policy_study(a.policy_study, min(a.warmup, a.policy_study))), flush=True)
        return
    wl = gen.WORKLOADS[a.workload]
    if a.weights != "mxfp4":
        from dataclasses import replace
        wl = replace(wl, name=f"{wl.name}_{a.weights}", shape=replace(wl.shape, weights=a.weights))
    T = a.T or max(wl.Ts)
    res = run_decode(wl, T, a.steps, a.warmup)
    extra = {}
    for t in [int(v) for v in a.extra_T.split(",") if v.strip()]:
        if t != T and t in wl.Ts:
            r = run_decode(wl, t, a.steps, a.warmup)
            extra[f"T={t}"] = {"tokens_per_s": round(r["tokens_per_s"], 1),
                               "ms_per_step": round(r["ms_per_step"], 4),
                               "hit_rate": round(r["hit_rate"], 4),
                               "gateup_gbs": r["gateup_gbs"] and round(r["gateup_gbs"], 1),
                               "down_gbs": r["down_gbs"] and round(r["down_gbs"], 1),
                               "h2d_gbs": round(r["h2d_gbs"], 2)}
    graph = {}
    if not wl.resize:
        for t in [int(v) for v in a.graph_T.split(",") if v.strip()]:
            if t in wl.Ts:
                r = run_decode_graph(wl, t, a.steps, a.warmup)
                graph[f"T={t}"] = {"tokens_per_s": round(r["tokens_per_s"], 1),
                                   "ms_per_step": round(r["ms_per_step"], 4),
                                   "hit_rate": round(r["hit_rate"], 4)}
    sh = wl.shape
    kgu, kdn = decode_kernels(T)
    roof = roofline_entry(kgu, res["gateup_gbs"], res["gateup_us"], res["gateup_bytes"],
                          res["launches"])
    roof["traffic"] = traffic_from_profile(kgu, f"{wl.name}_T{T}")
    roof["other_kernels"] = [roofline_entry(kdn, res["down_gbs"], res["down_us"],
                                            res["down_bytes"], res["launches"])]
    roof["expert_ffn_pair_gbs"] = res["ffn_gbs"] and round(res["ffn_gbs"], 1)
    line = {
        "metric": "MoE-layer decode tokens/s",
        "value": round(res["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "H": sh.H, "I": sh.I, "E": sh.E, "k": sh.k,
                   "layers": sh.layers, "shared_expert": sh.shared,
                   "cache_slots": wl.cache_slots, "staging_slots": wl.staging_slots,
                   "weights": ("MXFP4 (E2M1 + E8M0/32)" if sh.weights == "mxfp4" else sh.weights),
                   "zipf_s": wl.zipf_s,
                   "overlap": wl.overlap},
        "roofline": roof,
        "cache": {"hit_rate": round(res["hit_rate"], 4), **{k: res["stats"][k] for k in
                  ("lookups", "hits", "fills", "bypasses", "evictions")}},
        "pcie_h2d_gbs": round(res["h2d_gbs"], 2),
        "other_T": extra,
    }
    if graph:
        line["graph_replay"] = graph
    if a.weights == "mxfp4" and (a.prefill_steps > 0 or a.dsv4_decode_steps > 0):
        line.update(run_dsv4(a.prefill_steps, a.dsv4_decode_steps, max(a.dsv4_decode_steps // 4, 1)))
    if a.calibrate_copy_mb > 0:
        calibrate_copy(a.calibrate_copy_mb)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, T, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
