"""Drive the HIP library (through its C ABI) and the CPU oracle on the same
seeded synthetic inputs.  Used by the GPU tests, smoke and bench."""
from __future__ import annotations

import os
from collections import OrderedDict
from dataclasses import replace
from typing import Optional

import numpy as np

import oracle
from oracle import experts as oexp
from workload import gen

RTOL_Y = 2e-2     # max |y - y_ref| <= RTOL_Y * rms(y_ref), per call
# Decode carries h between its kernels as bf16 hi + lo (~16 significant
# bits) and accumulates in fp32, so its fp32 result sits within ~1e-4 of the
# oracle; this tighter bar catches small indexing or scaling mistakes that
# the 2e-2 bar would hide.
RTOL_Y_DECODE = 1e-3
# Prefill carries h as bf16 plus a block-scaled fp6 remainder (about 2^-14 of
# each 32-column block's largest value).  A CPU emulation of that rounding
# gives 1.06e-3 at the E = 1024, top-16, H = I = 256 shape (the worst one the
# tests run) and 3e-4 at wide I; this bar sits above those with room to spare
# and still far below the 2e-2 contract, so a mis-scaled or misplaced piece
# of h fails it.
RTOL_Y_PREFILL = 4e-3
# The MXFP8 prefill mode against the oracle of the same mode: x's codes are
# decided exactly as the oracle decides them (bf16 input, power-of-two
# scale, nearest-even convert); h's can differ where the GPU's fp32 h and the
# oracle's fp64 h straddle a rounding boundary or a block's amax a power of
# two.  oracle.mx.moe_layer_mx_bound gives, per output element, the most those
# decisions and the kernel's fp32 arithmetic can move it; each element is
# held to its own allowance plus MX_ATOL_RMS x rms(y) for what that model of
# the arithmetic leaves out (the combine's bf16-free fp32 adds are in it).
MX_ATOL_RMS = 1e-5
# ... and against the plain layer: the stated accuracy of that mode on
# N(0,1) activations.  Two E4M3 roundings (x and h, about 3.6% rms each) give
# about 5.5% relative rms and up to 0.55 x rms max-abs on the test shapes
# (oracle.moe_layer_mx against oracle.moe_layer on the CPU).
RTOL_Y_MX_PLAIN = 0.8
RRMS_MX_PLAIN = 0.08
ATOL_G = 1e-6     # gates
TOL_SUM = 1e-6    # |sum(g) - 1| with renormalisation


def oracle_rows(model: "Model", layer: int, xf: np.ndarray, ids: np.ndarray, g: np.ndarray,
                tokens, workers: Optional[int] = None, layer_fn=None) -> np.ndarray:
    """Oracle outputs of the listed token rows of one layer, through
    oracle.moe_layer.  Every expert those rows use is dequantised once, and
    the rows are split over worker threads (numpy releases the GIL in the
    dequantisation and in the products; each thread's BLAS keeps to one
    thread), so that a few hundred rows of a 256-expert layer take seconds
    instead of many minutes.  layer_fn: the oracle layer to evaluate
    (oracle.moe_layer by default; oracle.moe_layer_mx for the MXFP8 prefill
    mode; oracle.mx.moe_layer_mx_bound, whose (y, flip, arith) come back as
    a tuple).  Returns [len(tokens)][H] in the order given."""
    import concurrent.futures
    from threadpoolctl import threadpool_limits
    tokens = list(tokens)
    sh = model.shape
    workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    need = sorted({int(ids[t, j]) for t in tokens for j in range(sh.k)})
    if sh.shared:
        need.append(-1)
    with threadpool_limits(1), concurrent.futures.ThreadPoolExecutor(workers) as ex:
        mats = dict(zip(need, ex.map(lambda e: oexp.dequant_expert(model.expert(layer, e)),
                                     need)))
        shared = mats.pop(-1, None)
        chunks = [tokens[i::workers] for i in range(workers) if tokens[i::workers]]

        fn = layer_fn or oracle.moe_layer

        def run(rows):
            return fn(xf[rows], ids[rows], g[rows], mats.__getitem__, shared=shared)
        outs = list(ex.map(run, chunks))
    multi = isinstance(outs[0], tuple)
    parts = []
    for m in range(len(outs[0]) if multi else 1):
        y = {}
        for rows, out in zip(chunks, outs):
            o = out[m] if multi else out
            for i, t in enumerate(rows):
                y[t] = o[i]
        parts.append(np.stack([y[t] for t in tokens]))
    return tuple(parts) if multi else parts[0]


def bf16_dev(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def bf16_host(t) -> np.ndarray:
    return gen.bf16_bits_to_f32(t.cpu().numpy().view(np.uint16))


class Model:
    """Weights of a workload's layer stack: uploaded to an engine, and
    dequantised on demand for the oracle (bounded cache)."""

    def __init__(self, shape: gen.Shape, seed: int = 0, cache_entries: int = 32):
        self.shape = shape
        self.seed = seed
        self.routers = [gen.router_weights(shape, l, seed) for l in range(shape.layers)]
        self._mats = OrderedDict()
        self._cap = cache_entries

    def expert(self, layer: int, e: int):
        return gen.expert_weights_of(self.shape, layer, e, self.seed)

    def mats(self, layer: int, e: int):
        key = (layer, e)
        if key in self._mats:
            self._mats.move_to_end(key)
            return self._mats[key]
        m = oexp.dequant_expert(self.expert(layer, e))
        self._mats[key] = m
        if len(self._mats) > self._cap:
            self._mats.popitem(last=False)
        return m

    def load(self, eng):
        for l in range(self.shape.layers):
            eng.set_router(l, self.routers[l])
            for e in range(self.shape.E):
                eng.set_expert(l, e, self.expert(l, e))
            if self.shape.shared:
                eng.set_expert(l, -1, self.expert(l, -1))

    # oracle
    def route(self, layer, x, bias):
        return oracle.route(x, self.routers[layer], self.shape.k, bias, self.shape.renormalize)

    def layer_out(self, layer, x, ids, g, tokens=None):
        sh = self.mats(layer, -1) if self.shape.shared else None
        return oracle.moe_layer(x, ids, g, lambda e: self.mats(layer, e), shared=sh, tokens=tokens)


def make_engine(shape: gen.Shape, max_tokens: int, cache_slots: int, staging_slots: int,
                max_prefill_tokens: int = 0, cache_policy: str = "global",
                prefill_format: str = "bf16"):
    from expert_offload_serving_amd import MoEEngine
    return MoEEngine(shape.H, shape.I, shape.E, shape.k, n_layers=shape.layers,
                     has_shared=shape.shared, renormalize=shape.renormalize,
                     max_tokens=max_tokens, cache_slots=cache_slots,
                     staging_slots=staging_slots, max_prefill_tokens=max_prefill_tokens,
                     cache_policy=cache_policy, weight_format=shape.weights,
                     prefill_format=prefill_format)


def check_rounding(y_bf16, y32, what=""):
    """The bf16 output must be the fp32 result rounded to nearest even."""
    bits = y_bf16.cpu().numpy().view(np.uint16)
    want = gen.f32_to_bf16_bits(y32.cpu().numpy())
    assert np.array_equal(bits, want), f"{what}: bf16 output is not RNE of the fp32 result"


def check_y_mx(y_gpu: np.ndarray, ref, what=""):
    """Element-wise check of the MXFP8 prefill mode against
    oracle.mx.moe_layer_mx_bound's (y, flip, arith): |y_gpu - y| <= flip +
    arith + MX_ATOL_RMS x rms(y).  Returns (max |dy| / rms, max allowance /
    rms, fraction of elements whose |dy| needs the flip allowance)."""
    y, flip, arith = (np.asarray(a, dtype=np.float64) for a in ref)
    rms = float(np.sqrt(np.mean(y ** 2)))
    dy = np.abs(y_gpu.astype(np.float64) - y)
    base = arith + MX_ATOL_RMS * rms
    allow = flip + base
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    ratio = dy / allow
    i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert ratio[i] <= 1.0, (f"{what}: element {tuple(int(v) for v in i)} |dy| = {dy[i]:.4g} > "
                             f"allowance {allow[i]:.4g} (flip {flip[i]:.3g}, arith {arith[i]:.3g}, "
                             f"rms {rms:.4g})")
    return float(dy.max() / rms), float(allow.max() / rms), float(np.mean(dy > base))


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, rows=None, what="", rtol=RTOL_Y):
    """max |y - y_ref| <= RTOL_Y * rms(y_ref) over the checked rows; y_gpu is
    the fp32 combine result (before the bf16 rounding, checked separately)."""
    if rows is not None:
        y_gpu, y_ref = y_gpu[rows], y_ref[rows]
    rms = float(np.sqrt(np.mean(y_ref.astype(np.float64) ** 2)))
    err = float(np.max(np.abs(y_gpu.astype(np.float64) - y_ref)))
    assert err <= rtol * rms, f"{what}: max|dy| = {err:.4g} > {rtol} x rms {rms:.4g}"
    return err / rms


def valid_prefix(experts, E):
    """The entries of a lookup list the library acts on: those before the
    first one that is out of range or not above its predecessor."""
    out = []
    for e in experts:
        e = int(e)
        if e < 0 or e >= E or (out and e <= out[-1]):
            break
        out.append(e)
    return out


class DecodeRun:
    """Runs decode steps of one workload on the GPU and the oracle side by side."""

    def __init__(self, wl: gen.Workload, model: Model, T: int, cache_slots: Optional[int] = None,
                 staging_slots: Optional[int] = None, max_tokens: Optional[int] = None,
                 steps: Optional[int] = None, cache_policy: str = "global"):
        import torch
        self.wl, self.model, self.T = wl, model, T
        sh = wl.shape
        self.C = wl.cache_slots if cache_slots is None else cache_slots
        S = wl.staging_slots if staging_slots is None else staging_slots
        self.eng = make_engine(sh, max_tokens or T, self.C, S, cache_policy=cache_policy)
        model.load(self.eng)
        self.cache = oracle.SlotCache(self.C, sh.E, sh.layers, cache_policy)
        self.steps = wl.steps if steps is None else steps
        self.sets = ([gen.zipf_sets(sh, l, T, self.steps, wl.zipf_s, wl.overlap, model.seed)
                      for l in range(sh.layers)] if wl.zipf_s else None)
        self.dev = torch.device("cuda")
        self.ids = torch.empty((T, sh.k), dtype=torch.int32, device=self.dev)
        self.gates = torch.empty((T, sh.k), dtype=torch.float32, device=self.dev)
        self.y32 = torch.empty((T, sh.H), dtype=torch.float32, device=self.dev)
        if wl.preload_all:
            for l in range(sh.layers):
                self.preload(l, list(range(sh.E)))

    def preload(self, layer, experts):
        self.eng.cache_fill(layer, experts)
        self.cache.fill(layer, experts)

    def inputs(self, layer, step):
        sh = self.wl.shape
        xb = gen.tokens(sh, layer, step, self.T, self.model.seed)
        bias = gen.bias_from_sets(self.sets[layer][step], sh.E) if self.sets else None
        return xb, bias

    def step(self, layer, step, check_out=False, check_state=True, out_tokens=None,
             prefetch=None, forward=None):
        """prefetch: (layer, experts) armed for this call (moe_set_prefetch),
        mirrored by the oracle cache's prefetch after the call's lookup.
        forward: the engine method to call (default eng.forward; another
        entry point's dispatch arrays are not the context's, so then only
        the cache state is compared)."""
        import torch
        sh = self.wl.shape
        xb, bias = self.inputs(layer, step)
        x = bf16_dev(xb)
        bdev = torch.from_numpy(bias).to(self.dev) if bias is not None else None
        if prefetch is not None:
            self.eng.set_prefetch(prefetch[0], torch.tensor(list(prefetch[1]), dtype=torch.int32,
                                                            device=self.dev))
        fwd = forward or self.eng.forward
        y = fwd(layer, x, bias=bdev, ids=self.ids, gates=self.gates, y32=self.y32)
        xf = gen.bf16_bits_to_f32(xb)
        lg, ids_ref, g_ref = self.model.route(layer, xf, bias)
        ids = self.ids.cpu().numpy()
        assert np.array_equal(ids, ids_ref), f"ids differ at layer {layer} step {step}"
        g = self.gates.cpu().numpy()
        assert np.max(np.abs(g - g_ref)) <= ATOL_G, f"gates differ at layer {layer} step {step}"
        if sh.renormalize:
            assert np.max(np.abs(g.astype(np.float64).sum(1) - 1)) <= TOL_SUM
        perm = oracle.permutation(ids_ref, sh.E)
        pinned = self.cache.clock
        slots_ref, fills, bypass = self.cache.lookup(layer, perm["unique"])
        if prefetch is not None:
            self.cache.prefetch(prefetch[0], valid_prefix(prefetch[1], sh.E), pinned)
        if check_state:
            if forward is None:
                d = self.eng.inspect_dispatch()
                for k in ("counts", "offsets", "sorted", "inv", "unique"):
                    assert np.array_equal(d[k], perm[k]), f"{k} differs at layer {layer} step {step}"
                assert d["slot"].tolist() == slots_ref, f"slots differ at layer {layer} step {step}"
            key, stamp, clock = self.eng.cache_snapshot()
            k_ref, s_ref, c_ref = self.cache.snapshot()
            assert key.tolist() == k_ref and stamp.tolist() == s_ref and clock == c_ref, \
                f"cache state differs at layer {layer} step {step}"
        err = None
        if check_out:
            what = f"layer {layer} step {step}"
            check_rounding(y, self.y32, what)
            y_ref = self.model.layer_out(layer, xf, ids_ref, g_ref, tokens=out_tokens)
            err = check_y(self.y32.cpu().numpy(), y_ref, rows=out_tokens, what=what)
            check_y(self.y32.cpu().numpy(), y_ref, rows=out_tokens, what=what + " (decode bar)",
                    rtol=RTOL_Y_DECODE)
        return y, err

    def close(self):
        self.eng.close()


def small_shape(**kw) -> gen.Shape:
    base = gen.Shape(H=256, I=512, E=8, k=2)
    return replace(base, **kw)


# Share of h codes the MXFP8 mode may take differently from the oracle's own
# choice (each such decision must still lie inside its allowance).  On
# gfx950 0.02-0.04% of them differ at the test shapes (the instruction's
# error flips only elements within about 1e-4 of a rounding boundary); a
# computation with every instruction at its largest measured error would
# flip about 1%, and a bf16-rounded h about 3%.
MX_FLIP_SHARE = 0.005


def check_mx_decisions(run: "PrefillRun", tokens=None, what=""):
    """The MXFP8 mode's quantisation decisions on the last layer of the last
    prefill call, read back with moe_inspect_prefill_mx:

    - x: every scale byte and every element value equal to the oracle's
      quantisation of the input (the decision is exact on both sides);
    - h: every element within its allowance, oracle.mx.mx_h_deviation of the
      oracle's h and expert_h_mx's interval (fp32 gate/up sums under the
      measured instruction model), and at most MX_FLIP_SHARE of them off the
      oracle's own choice;
    - y: the library's output equal, within the down product's and the
      combine's own arithmetic allowance, to the down product and combine
      of the h codes the library chose -- the choices are the witness that
      y is one of the mode's valid outputs.

    Returns (share of h codes off the oracle's choice, max |y - y_w| / rms)."""
    import concurrent.futures
    from threadpoolctl import threadpool_limits
    from oracle import mx as omx
    sh = run.shape
    layer = sh.layers - 1
    T, k = run.T, sh.k
    toks = list(range(T)) if tokens is None else sorted(tokens)
    ins = run.eng.inspect_prefill_mx()
    assert ins["T"] == T
    xf = gen.bf16_bits_to_f32(run.xb[layer]).astype(np.float64)
    xq_ref = omx.quantize_mxfp8(xf)
    assert np.array_equal(ins["xs"].astype(np.int64) - 127, omx.block_exponents(xf)), \
        f"{what}: x scale bytes differ"
    xq_gpu = omx.dequant_mxfp8(ins["xq"], ins["xs"])
    bad = np.argwhere(xq_gpu != xq_ref)
    assert len(bad) == 0, f"{what}: x codes differ at {bad[:4].tolist()}"
    _, (_, ids, g) = run.route(layer)
    perm = oracle.permutation(ids, sh.E)
    hq = omx.dequant_mxfp8(ins["hq"], ins["hs"])
    # (row, token, slot) per expert; slot -1 for the shared expert
    groups = {}
    for t in toks:
        for j in range(k):
            groups.setdefault(int(ids[t, j]), []).append((int(perm["inv"][t * k + j]), t, j))
        if sh.shared:
            groups.setdefault(-1, []).append((T * k + t, t, -1))

    def one(item):
        e, rows = item
        wg, wu, wd = oexp.dequant_expert(run.model.expert(layer, e))
        r = np.array([q[0] for q in rows])
        tt = np.array([q[1] for q in rows])
        h, dh = omx.expert_h_mx(xq_ref[tt], wg, wu)
        dev = omx.mx_h_deviation(h, dh)
        q = omx.quantize_mxfp8(h)
        off = np.abs(hq[r] - q)
        wd = wd.astype(np.float64)
        ye = hq[r] @ wd.T
        return (e, rows, int(np.sum(off > dev)), int(np.sum(off > 0)), off.size, ye,
                omx.mfma_dot_err(np.abs(hq[r]), np.abs(wd)))
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(1), concurrent.futures.ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(one, groups.items()))
    H = sh.H
    pos = {t: i for i, t in enumerate(toks)}
    y_w, allow, mag = (np.zeros((len(toks), H)) for _ in range(3))
    outside = differ = total = 0
    for e, rows, n_out, n_diff, n, ye, ae in res:
        outside += n_out
        differ += n_diff
        total += n
        for i, (_, t, j) in enumerate(rows):
            gj = 1.0 if j < 0 else float(g[t, j])
            y_w[pos[t]] += gj * ye[i]
            allow[pos[t]] += abs(gj) * ae[i] + (0.0 if j < 0 else ATOL_G * np.abs(ye[i]))
            mag[pos[t]] += np.abs(gj * ye[i])
    assert outside == 0, f"{what}: {outside} of {total} h decisions outside their allowance"
    share = differ / max(total, 1)
    assert share <= MX_FLIP_SHARE, f"{what}: {share:.2%} of h codes off the oracle's choice"
    allow += (k + 3) * 2.0 ** -24 * mag
    y = run.y32[layer].cpu().numpy()[toks].astype(np.float64)
    rms = float(np.sqrt(np.mean(y_w ** 2)))
    d = np.abs(y - y_w)
    i = np.unravel_index(int(np.argmax(d / allow)), d.shape)
    assert d[i] <= allow[i], (f"{what}: y at (token {toks[i[0]]}, col {i[1]}) is {d[i]:.4g} from the "
                              f"down product of the library's own h codes (allowance {allow[i]:.3g})")
    return share, float(d.max() / rms)


class PrefillRun:
    """Prefill of a layer stack: every layer gets its own seeded x [T][H]."""

    def __init__(self, shape: gen.Shape, T: int, seed: int = 0, model: Optional[Model] = None,
                 bias_sets=None, prefill_format: str = "bf16"):
        import torch
        self.shape, self.T = shape, T
        self.model = model or Model(shape, seed)
        self.eng = make_engine(shape, max_tokens=1, cache_slots=0, staging_slots=shape.k,
                               max_prefill_tokens=T, prefill_format=prefill_format)
        self.model.load(self.eng)
        L = shape.layers
        self.xb = [gen.tokens(shape, l, 0, T, self.model.seed) for l in range(L)]
        self.xs = [bf16_dev(b) for b in self.xb]
        self.bias = bias_sets
        self.bias_dev = (None if bias_sets is None else
                         [torch.from_numpy(b).to("cuda") for b in bias_sets])
        self.ys = [torch.empty((T, shape.H), dtype=torch.int16, device="cuda") for _ in range(L)]
        self.y32 = [torch.empty((T, shape.H), dtype=torch.float32, device="cuda") for _ in range(L)]

    def run(self):
        import torch
        self.eng.prefill(self.xs, self.ys, biases=self.bias_dev, y32s=self.y32)
        torch.cuda.synchronize()

    def route(self, layer):
        xf = gen.bf16_bits_to_f32(self.xb[layer])
        b = None if self.bias is None else self.bias[layer]
        return xf, self.model.route(layer, xf, b)

    def check_routing(self, layer):
        """Routing and dispatch of one layer, read back from the library,
        against oracle.route and oracle.permutation: ids, counts, offsets,
        sorted and inv bit for bit, gates within ATOL_G.  Returns the oracle
        (x, ids, gates)."""
        xf, (lg, ids_ref, g_ref) = self.route(layer)
        d = self.eng.inspect_prefill(layer)
        assert d["T"] == self.T
        assert np.array_equal(d["ids"], ids_ref), f"prefill ids differ at layer {layer}"
        assert np.max(np.abs(d["gates"] - g_ref)) <= ATOL_G, f"prefill gates at layer {layer}"
        if self.shape.renormalize:
            assert np.max(np.abs(d["gates"].astype(np.float64).sum(1) - 1)) <= TOL_SUM
        perm = oracle.permutation(ids_ref, self.shape.E)
        for k in ("counts", "offsets", "sorted", "inv"):
            assert np.array_equal(d[k], perm[k]), f"prefill {k} differs at layer {layer}"
        return xf, ids_ref, g_ref

    def close(self):
        self.eng.close()
