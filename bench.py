"""Benchmark of the routed MoE expert-layer forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--T T]
                [--prefill-steps P]

A step is one decode call per layer of the workload (router, top-k, dispatch,
cache lookup, miss fills, expert FFN, combine) for a batch of T tokens, with
all inputs already resident in HBM.  Default workload: the 35B-A3B-shaped
decode layer (H=2048, E=256, top-8, I=512, MXFP4 experts, bf16 activations,
64-slot LRU from a cold start, Zipf(1.1) routing with 60% step overlap), T=16.
The line also carries the prefill leg: the DeepSeek-V4-Flash-shaped stack
(4 layers, H=4096, I=2048, E=256, top-6 + shared, T=4096) with whole-layer
uploads from the pinned pool, its grouped-GEMM time and MFMA utilisation.
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
    ap.add_argument("--prefill-steps", type=int, default=3,
                    help="prefill passes of the DeepSeek-V4-Flash-shaped stack (0: skip)")
    return ap.parse_args()


def ffn_bytes(sh, lookups, calls, pairs, T_total):
    """Algorithmic bytes of the expert FFN kernels over `calls` calls:
    every looked-up expert's MXFP4 weights once (plus the shared expert per
    call), the token rows read, the h rows written and read (bf16), and the
    expert output rows written (fp32)."""
    from workload import gen  # noqa: F401
    b_e = sh.expert_bytes()
    rows = pairs + (T_total if sh.shared else 0)
    weights = (lookups + (calls if sh.shared else 0)) * b_e
    acts = T_total * sh.H * 2 + rows * sh.I * 2 * 2 + rows * sh.H * 4
    return weights + acts


def make_engine(sh, T, cache_slots, staging_slots, prefill_tokens=0):
    from expert_offload_serving_amd import MoEEngine
    return MoEEngine(sh.H, sh.I, sh.E, sh.k, n_layers=sh.layers, has_shared=sh.shared,
                     renormalize=sh.renormalize, max_tokens=T, cache_slots=cache_slots,
                     staging_slots=staging_slots, max_prefill_tokens=prefill_tokens)


def load_weights(eng, sh, seed=0):
    from workload import gen
    for l in range(sh.layers):
        eng.set_router(l, gen.router_weights(sh, l, seed))
        for e in range(sh.E):
            eng.set_expert(l, e, gen.expert_weights(sh, l, e, seed))
        if sh.shared:
            eng.set_expert(l, -1, gen.expert_weights(sh, l, -1, seed))


def bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def run_decode(wl, T, steps, warmup, seed=0):
    import torch
    from workload import gen

    sh = wl.shape
    eng = make_engine(sh, T, wl.cache_slots, wl.staging_slots)
    load_weights(eng, sh, seed)
    n = min(wl.steps, steps + warmup)
    dev = torch.device("cuda")
    xs, bs = [], []
    for l in range(sh.layers):
        sets = gen.zipf_sets(sh, l, T, n, wl.zipf_s, wl.overlap, seed) if wl.zipf_s else None
        xs.append(torch.stack([bf16_dev(gen.tokens(sh, l, s, T, seed)) for s in range(n)]))
        bs.append(torch.from_numpy(np.stack([gen.bias_from_sets(sets[s], sh.E) for s in range(n)])).to(dev)
                  if sets is not None else None)
    y = torch.empty((T, sh.H), dtype=torch.int16, device=dev)
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
    eng.set_timing(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(warmup, warmup + steps):
        do_step(s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tm = eng.get_timing()
    st = eng.stats()
    eng.close()
    elapsed = t1 - t0
    calls = steps * sh.layers
    pairs = calls * T * sh.k
    fb = ffn_bytes(sh, st["lookups"], calls, pairs, calls * T)
    ms_ffn = tm["ms_decode"]
    return dict(T=T, steps=steps, elapsed_s=elapsed, tokens_per_s=T * steps / elapsed,
                ms_per_step=1e3 * elapsed / steps, stats=st,
                hit_rate=st["hits"] / max(st["lookups"], 1),
                ffn_launches=tm["n_decode"], ffn_ms_total=ms_ffn,
                ffn_bytes_total=fb,
                ffn_gbs=fb / (ms_ffn * 1e6) if ms_ffn > 0 else None,
                h2d_gbs=st["bytes_h2d"] / (elapsed * 1e9))


def run_prefill(wl, steps, warmup, seed=0):
    """Prefill of the whole layer stack per step (layer uploads included)."""
    import torch
    from workload import gen
    sh = wl.shape
    T = wl.Ts[0]
    eng = make_engine(sh, 1, 0, sh.k, prefill_tokens=T)
    load_weights(eng, sh, seed)
    xs = [bf16_dev(gen.tokens(sh, l, 0, T, seed)) for l in range(sh.layers)]
    ys = [torch.empty((T, sh.H), dtype=torch.int16, device="cuda") for _ in range(sh.layers)]
    for _ in range(warmup):
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
    eng.close()
    el = t1 - t0
    layers = steps * sh.layers
    # algorithmic flops per layer: 3 matrices of H x I per (token, expert),
    # k routed experts plus the shared one, 2 flops per multiply-add
    flops_layer = 2 * 3 * sh.H * sh.I * T * (sh.k + (1 if sh.shared else 0))
    gemm_ms = tm["ms_prefill"] / max(tm["n_prefill"], 1)
    tflops = flops_layer / (gemm_ms * 1e9)
    upload = sh.E * sh.expert_bytes() * layers
    return {"workload": wl.name, "T": T, "layers": sh.layers, "steps": steps,
            "tokens_per_s_end_to_end": round(T * steps / el, 1),
            "ms_per_step": round(1e3 * el / steps, 2),
            "gemm_ms_per_layer": round(gemm_ms, 4),
            "gemm_launches": tm["n_prefill"],
            "tokens_per_s_gemm_only": round(T / (gemm_ms * 1e-3) / sh.layers, 1),
            "flops_per_layer": flops_layer,
            "mfma_tflops": round(tflops, 1),
            "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "pcie_h2d_gbs": round(upload / (el * 1e9), 2)}


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


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    from workload import gen
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = gen.WORKLOADS[a.workload]
    T = a.T or max(wl.Ts)
    res = run_decode(wl, T, a.steps, a.warmup)
    extra = {}
    for t in [int(v) for v in a.extra_T.split(",") if v.strip()]:
        if t != T and t in wl.Ts:
            r = run_decode(wl, t, a.steps, a.warmup)
            extra[f"T={t}"] = {k: r[k] for k in ("tokens_per_s", "ms_per_step", "hit_rate", "ffn_gbs",
                                                 "h2d_gbs")}
    sh = wl.shape
    achieved = res["ffn_gbs"]
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
                   "weights": "MXFP4 (E2M1 + E8M0/32)", "zipf_s": wl.zipf_s,
                   "overlap": wl.overlap},
        "roofline": {
            "kernel": "expert FFN (gate/up+SwiGLU and down kernels)",
            "bound": "hbm",
            "achieved": None if achieved is None else round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": None if achieved is None else round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "launches": res["ffn_launches"],
            "avg_launch_us": round(1e3 * res["ffn_ms_total"] / max(res["ffn_launches"], 1), 3),
            "bytes_per_launch": round(res["ffn_bytes_total"] / max(res["ffn_launches"], 1)),
        },
        "cache": {"hit_rate": round(res["hit_rate"], 4), **{k: res["stats"][k] for k in
                  ("lookups", "hits", "fills", "bypasses", "evictions")}},
        "pcie_h2d_gbs": round(res["h2d_gbs"], 2),
        "other_T": extra,
    }
    if a.prefill_steps > 0:
        line["prefill"] = run_prefill(gen.WORKLOADS["dsv4_prefill"], a.prefill_steps, 1)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, T, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
