"""A Python handle on one libmoe context (argument marshalling only).

The library takes raw device addresses, so a wrong tensor (host memory, a
transposed view, the wrong element size, too few rows) would reach the GPU
unchecked.  Every tensor and array is therefore checked here first and
rejected with ValueError: device tensors must be CUDA, contiguous, of the
element type and shape the call documents; host weight arrays must have the
canonical shapes.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import binding as b

_BF16_TYPES = ("bfloat16", "int16", "uint16", "float16")


def check_device(name: str, t, dtypes: Sequence[str], shape: tuple, device=None):
    """t must be a contiguous CUDA tensor of one of `dtypes` (torch dtype
    names) with exactly `shape`, on `device` when given."""
    if t is None or not hasattr(t, "data_ptr") or not hasattr(t, "is_cuda"):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a CUDA tensor (got device {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, the other tensors are on {device}")
    dt = str(t.dtype).replace("torch.", "")
    if dt not in dtypes:
        raise ValueError(f"{name}: dtype {dt}, expected one of {tuple(dtypes)}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def check_host(name: str, a, shape: tuple):
    """a must be a host array with exactly `shape` (it is converted to the
    element type the library reads)."""
    if hasattr(a, "is_cuda") and a.is_cuda:
        raise ValueError(f"{name}: expected a host array, got a CUDA tensor")
    if tuple(np.shape(a)) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(np.shape(a))}, expected {tuple(shape)}")


def check_forward(H: int, E: int, k: int, max_tokens: int, x, bias, y, ids, gates, y32):
    """Arguments of one decode forward (moe_layer_forward)."""
    check_device("x", x, _BF16_TYPES, (x.shape[0] if hasattr(x, "shape") and len(x.shape) else -1, H))
    T = int(x.shape[0])
    if not 0 <= T <= max_tokens:
        raise ValueError(f"x: {T} tokens, the context takes at most {max_tokens}")
    dev = x.device
    check_device("y", y, _BF16_TYPES, (T, H), dev)
    if bias is not None:
        check_device("bias", bias, ("float32",), (T, E), dev)
    if ids is not None:
        check_device("ids", ids, ("int32",), (T, k), dev)
    if gates is not None:
        check_device("gates", gates, ("float32",), (T, k), dev)
    if y32 is not None:
        check_device("y32", y32, ("float32",), (T, H), dev)
    return T


def check_prefill(H: int, E: int, n_layers: int, max_prefill_tokens: int, xs, ys, biases, y32s):
    """Arguments of one prefill call (moe_prefill_forward)."""
    L = len(xs)
    if not 1 <= L <= n_layers:
        raise ValueError(f"{L} layers given, the context has {n_layers}")
    check_device("xs[0]", xs[0], _BF16_TYPES,
                 (xs[0].shape[0] if hasattr(xs[0], "shape") and len(xs[0].shape) else -1, H))
    T = int(xs[0].shape[0])
    if not 1 <= T <= max_prefill_tokens:
        raise ValueError(f"prefill of {T} tokens, the context takes 1..{max_prefill_tokens}")
    dev = xs[0].device
    for name, seq, dts, cols in (("xs", xs, _BF16_TYPES, H), ("ys", ys, _BF16_TYPES, H),
                                 ("biases", biases, ("float32",), E),
                                 ("y32s", y32s, ("float32",), H)):
        if seq is None:
            continue
        if len(seq) != L:
            raise ValueError(f"{name}: {len(seq)} entries for {L} layers")
        for l, t in enumerate(seq):
            if t is not None or name in ("xs", "ys"):
                check_device(f"{name}[{l}]", t, dts, (T, cols), dev)
    return T


class MoEEngine:
    """Owns a moe_ctx.  Device tensors are torch tensors on the current GPU."""

    def __init__(self, H: int, I: int, E: int, k: int, n_layers: int = 1,
                 has_shared: bool = False, renormalize: bool = True, max_tokens: int = 16,
                 cache_slots: int = 0, staging_slots: int = 0, max_prefill_tokens: int = 0,
                 cache_policy: str = "global", weight_format: str = "mxfp4",
                 prefill_format: str = "bf16"):
        self.H, self.I, self.E, self.k, self.L = H, I, E, k, n_layers
        self.has_shared = bool(has_shared)
        self.max_tokens = max_tokens
        self.max_prefill_tokens = max_prefill_tokens
        self.cache_policy = cache_policy
        self.weight_format = weight_format
        self.ctx = b.moe_create(hidden=H, inter=I, n_experts=E, top_k=k, n_layers=n_layers,
                                has_shared=int(has_shared), renormalize=int(renormalize),
                                max_tokens=max_tokens, cache_slots=cache_slots,
                                staging_slots=staging_slots,
                                max_prefill_tokens=max_prefill_tokens,
                                cache_policy=b.CACHE_POLICIES.index(cache_policy),
                                weight_format=b.WEIGHT_FORMATS.index(weight_format),
                                prefill_format=b.PREFILL_FORMATS.index(prefill_format))
        self.prefill_format = prefill_format

    # ---------------------------------------------------------------- weights
    def set_router(self, layer: int, w_router: np.ndarray):
        check_host("w_router", w_router, (self.H, self.E))
        b.moe_set_router(self.ctx, layer, np.ascontiguousarray(w_router, dtype=np.float32))

    def set_expert(self, layer: int, expert: int, w):
        """w has canonical MXFP4 arrays qg, qu, qd, sg, su, sd (uint8); bf16
        matrices wg, wu, wd (uint16 bit patterns) for a bf16 context; or, for
        an NVFP4 context, codes qg, qu, qd, E4M3 block scales sg, su, sd
        (one byte per 16) and fp32 matrix scales tg, tu, td."""
        H, I = self.H, self.I
        if self.weight_format == "nvfp4":
            shapes = {"qg": (I, H // 2), "qu": (I, H // 2), "qd": (H, I // 2),
                      "sg": (I, H // 16), "su": (I, H // 16), "sd": (H, I // 16)}
            for n, shp in shapes.items():
                check_host(n, getattr(w, n), shp)
            q = [np.ascontiguousarray(getattr(w, n), dtype=np.uint8) for n in ("qg", "qu", "qd")]
            # each scale array is followed by its matrix's fp32 scale
            sc = [np.concatenate([np.ascontiguousarray(getattr(w, n), dtype=np.uint8).ravel(),
                                  np.array([getattr(w, t)], dtype="<f4").view(np.uint8)])
                  for n, t in (("sg", "tg"), ("su", "tu"), ("sd", "td"))]
            b.moe_set_expert(self.ctx, layer, expert, *q, *sc)
            return
        if self.weight_format == "bf16":
            shapes = {"wg": (I, H), "wu": (I, H), "wd": (H, I)}
            for n, shp in shapes.items():
                check_host(n, getattr(w, n), shp)
            arrs = [np.ascontiguousarray(getattr(w, n), dtype=np.uint16) for n in shapes]
            b.moe_set_expert(self.ctx, layer, expert, *arrs, None, None, None)
            return
        shapes = {"qg": (I, H // 2), "qu": (I, H // 2), "qd": (H, I // 2),
                  "sg": (I, H // 32), "su": (I, H // 32), "sd": (H, I // 32)}
        for n, shp in shapes.items():
            check_host(n, getattr(w, n), shp)
        arrs = [np.ascontiguousarray(getattr(w, n), dtype=np.uint8) for n in shapes]
        b.moe_set_expert(self.ctx, layer, expert, *arrs)

    # ---------------------------------------------------------------- forward
    def forward(self, layer: int, x, bias=None, y=None, ids=None, gates=None, y32=None,
                stream=None):
        import torch
        if y is None and hasattr(x, "shape") and hasattr(x, "is_cuda"):
            y = torch.empty((int(x.shape[0]), self.H), dtype=x.dtype, device=x.device)
        T = check_forward(self.H, self.E, self.k, self.max_tokens, x, bias, y, ids, gates, y32)
        b.moe_layer_forward(self.ctx, layer, x, T, bias, y, y32, ids, gates, stream)
        return y

    def forward_noalloc(self, layer: int, x, y, bias=None, ids=None, gates=None, y32=None,
                        stream=None):
        """forward() through moe_layer_forward_noalloc: the library's fixed
        device scratch, no allocation (y must be given)."""
        T = check_forward(self.H, self.E, self.k, self.max_tokens, x, bias, y, ids, gates, y32)
        b.moe_layer_forward_noalloc(self.ctx, layer, x, T, bias, y, y32, ids, gates, stream)
        return y

    def prefill(self, xs: Sequence, ys: Sequence, biases: Optional[Sequence] = None,
                y32s: Optional[Sequence] = None, stream=None):
        T = check_prefill(self.H, self.E, self.L, self.max_prefill_tokens, xs, ys, biases, y32s)
        b.moe_prefill_forward(self.ctx, len(xs), xs, T, biases, ys, y32s, stream)
        return ys

    def set_prefill_format(self, fmt: str):
        """"bf16" (exact) or "mxfp8" (native-MX, quantised activations)."""
        b.moe_set_prefill_format(self.ctx, fmt)
        self.prefill_format = fmt

    # ------------------------------------------------------------------ cache
    def cache_lookup(self, layer, d_experts, d_n, d_slot, stream=None):
        b.expert_cache_lookup(self.ctx, layer, d_experts, d_n, d_slot, stream)

    def cache_fill(self, layer: int, experts: Sequence[int], stream=None):
        b.expert_cache_fill(self.ctx, layer, experts, stream)

    def cache_resize(self, new_slots: int, stream=None):
        b.expert_cache_resize(self.ctx, new_slots, stream)

    def cache_snapshot(self):
        return b.expert_cache_snapshot(self.ctx)

    def inspect_dispatch(self):
        return b.moe_inspect_dispatch(self.ctx, self.E, self.k, self.max_tokens)

    def inspect_prefill(self, layer: int):
        """Routing (ids, gates) and dispatch (counts, offsets, sorted, inv) of
        one layer of the last prefill call."""
        return b.moe_inspect_prefill(self.ctx, layer, self.E, self.k, self.max_prefill_tokens)

    def inspect_prefill_mx(self):
        """E4M3 codes and E8M0 scale bytes of x and h of the last layer of the
        last prefill call (MXFP8 mode only); h rows in that layer's permuted
        order, the shared expert's rows last."""
        return b.moe_inspect_prefill_mx(self.ctx, self.H, self.I, self.k, self.has_shared,
                                        self.max_prefill_tokens)

    def set_copy_overlap(self, mode: int):
        """-1 automatic (records of 4 MiB and more), 0 off, 1 on: whether
        decode copies run beside the resident experts' kernels."""
        b.moe_set_copy_overlap(self.ctx, mode)

    def set_prefetch(self, layer: int, experts=None):
        """Arm a prefetch of `layer`'s experts (a device int32 tensor,
        ascending and unique; None or empty disarms) for the next decode
        call.  The tensor must stay alive until that call has run."""
        if experts is None or (hasattr(experts, "numel") and experts.numel() == 0):
            b.moe_set_prefetch(self.ctx, layer, None, 0)
            self._prefetch_list = None
            return
        n = int(experts.shape[0]) if hasattr(experts, "shape") and len(experts.shape) == 1 else -1
        check_device("experts", experts, ("int32",), (n,))
        b.moe_set_prefetch(self.ctx, layer, experts.data_ptr(), experts.numel())
        self._prefetch_list = experts  # kept until replaced

    def set_debug(self, sync: bool = False, fail_next_fill: bool = False):
        """Synchronise and check every stage; make the next copy step fail
        (the context then refuses cache work until cache_reset)."""
        b.moe_set_debug(self.ctx, (b.DEBUG_SYNC if sync else 0) |
                        (b.DEBUG_FAIL_NEXT_FILL if fail_next_fill else 0))

    def cache_reset(self):
        """Empty the expert cache (clock and counters kept)."""
        b.expert_cache_reset(self.ctx)

    def stats(self) -> dict:
        return b.moe_get_stats(self.ctx)

    def reset_stats(self):
        b.moe_reset_stats(self.ctx)

    def set_timing(self, enable: bool):
        b.moe_set_timing(self.ctx, enable)

    def get_timing(self) -> dict:
        """Summed kernel times (ms) since the last call, per decode kernel
        and per prefill stage, with the record counts."""
        return b.moe_get_timing(self.ctx)

    def close(self):
        if self.ctx:
            b.moe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
