"""A Python handle on one libmoe context (argument marshalling only)."""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import binding as b


class MoEEngine:
    """Owns a moe_ctx.  Device tensors are torch tensors on the current GPU."""

    def __init__(self, H: int, I: int, E: int, k: int, n_layers: int = 1,
                 has_shared: bool = False, renormalize: bool = True, max_tokens: int = 16,
                 cache_slots: int = 0, staging_slots: int = 0, max_prefill_tokens: int = 0,
                 cache_policy: str = "global", weight_format: str = "mxfp4"):
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
                                weight_format=b.WEIGHT_FORMATS.index(weight_format))

    # ---------------------------------------------------------------- weights
    def set_router(self, layer: int, w_router: np.ndarray):
        b.moe_set_router(self.ctx, layer, np.ascontiguousarray(w_router, dtype=np.float32))

    def set_expert(self, layer: int, expert: int, w):
        """w has canonical MXFP4 arrays qg, qu, qd, sg, su, sd (uint8), or
        bf16 matrices wg, wu, wd (uint16 bit patterns) for a bf16 context."""
        if self.weight_format == "bf16":
            arrs = [np.ascontiguousarray(getattr(w, n), dtype=np.uint16) for n in ("wg", "wu", "wd")]
            b.moe_set_expert(self.ctx, layer, expert, *arrs, None, None, None)
            return
        arrs = [np.ascontiguousarray(getattr(w, n), dtype=np.uint8)
                for n in ("qg", "qu", "qd", "sg", "su", "sd")]
        b.moe_set_expert(self.ctx, layer, expert, *arrs)

    # ---------------------------------------------------------------- forward
    def forward(self, layer: int, x, bias=None, y=None, ids=None, gates=None, y32=None,
                stream=None):
        import torch
        T = int(x.shape[0])
        if y is None:
            y = torch.empty((T, self.H), dtype=x.dtype, device=x.device)
        b.moe_layer_forward(self.ctx, layer, x, T, bias, y, y32, ids, gates, stream)
        return y

    def prefill(self, xs: Sequence, ys: Sequence, biases: Optional[Sequence] = None,
                y32s: Optional[Sequence] = None, stream=None):
        T = int(xs[0].shape[0])
        b.moe_prefill_forward(self.ctx, len(xs), xs, T, biases, ys, y32s, stream)
        return ys

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

    def inspect_prefill(self):
        """(ids, gates) of the last layer of the last prefill call."""
        return b.moe_inspect_prefill(self.ctx, self.k, self.max_prefill_tokens)

    def stats(self) -> dict:
        return b.moe_get_stats(self.ctx)

    def reset_stats(self):
        b.moe_reset_stats(self.ctx)

    def set_timing(self, enable: bool):
        b.moe_set_timing(self.ctx, enable)

    def get_timing(self) -> dict:
        """Summed event times (ms) since the last call, in total and per
        expert kernel (gate/up, down), for decode calls and prefill layers."""
        return b.moe_get_timing_split(self.ctx)

    def close(self):
        if self.ctx:
            b.moe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
