"""Mutation checks for the oracle's pins (no GPU).

Each case plants one plausible mistake in the CPU oracle (or in the bf16
rounding the output checks use): a dropped term, a flipped sign, a wrong
index or block size, a transposed operand, a wrong tie rule or slot order.
The mistake is applied with monkeypatch to this process's copy of the
module, and the pins that guard that part of the oracle are run against
it: at least one of them must fail.  A mutation that every pin accepts
would mean the pins do not fix that detail of the oracle.
"""
import numpy as np
import pytest

import oracle
from oracle import cache as ocache
from oracle import dispatch as odispatch
from oracle import experts as oexperts
from oracle import mx as omx
from oracle import mxfp4 as omxfp4
from oracle import nvfp4 as onvfp4
from oracle import router as orouter
from workload import gen

from tests import test_bf16_rounding as p_bf16
from tests import test_oracle_cache as p_cache
from tests import test_oracle_dispatch as p_dispatch
from tests import test_oracle_experts as p_experts
from tests import test_oracle_mx as p_mx
from tests import test_oracle_mxfp4 as p_mxfp4
from tests import test_oracle_nvfp4 as p_nvfp4
from tests import test_oracle_router as p_router


# ----------------------------------------------------------- planted mistakes
def m_nibbles_high_first(mp):
    def unpack(packed):
        p = np.asarray(packed, dtype=np.uint8)
        out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
        out[..., 0::2] = p >> 4
        out[..., 1::2] = p & 0x0F
        return out
    mp.setattr(omxfp4, "unpack_nibbles", unpack)


def m_scale_bias_126(mp):
    good = omxfp4.dequant
    mp.setattr(omxfp4, "dequant", lambda q, s: good(q, s) * np.float32(2.0))
    mp.setattr(oexperts, "dequant", omxfp4.dequant)


def m_sign_dropped(mp):
    mp.setattr(omxfp4, "E2M1_VALUES", np.abs(omxfp4.E2M1_VALUES))


def m_block_of_16(mp):
    def dequant(packed, scales):
        vals = omxfp4.decode_e2m1(omxfp4.unpack_nibbles(packed))
        s = np.asarray(scales).astype(np.int32) - 127
        e = np.repeat(s, 16, axis=1)
        e = np.concatenate([e, e], axis=1)[:, :vals.shape[1]]
        return (vals * np.ldexp(np.float32(1.0), e)).astype(np.float32)
    mp.setattr(omxfp4, "dequant", dequant)
    mp.setattr(oexperts, "dequant", dequant)


def m_logits_drop_bias(mp):
    good = orouter.logits
    mp.setattr(orouter, "logits", lambda x, w, bias=None: good(x, w))


def m_logits_reversed_k(mp):
    good = orouter.logits
    mp.setattr(orouter, "logits",
               lambda x, w, bias=None: good(np.asarray(x)[:, ::-1], w, bias))


def m_logits_fp32_accumulation(mp):
    def logits(x, w, bias=None):
        acc = np.asarray(x, np.float32) @ np.asarray(w, np.float32)
        if bias is not None:
            acc = acc + np.asarray(bias, np.float32)
        return acc.astype(np.float32)
    mp.setattr(orouter, "logits", logits)


def m_topk_ties_to_higher_id(mp):
    def topk(lg, k):
        T, E = lg.shape
        out = np.empty((T, k), dtype=np.int32)
        for t in range(T):
            out[t] = np.lexsort((-np.arange(E), -lg[t].astype(np.float64)))[:k]
        return out
    mp.setattr(orouter, "topk", topk)


def m_gates_not_renormalised(mp):
    good = orouter.gates
    mp.setattr(orouter, "gates", lambda lg, ids, renormalize=True: good(lg, ids, False))


def m_gates_sign_flipped(mp):
    good = orouter.gates
    mp.setattr(orouter, "gates",
               lambda lg, ids, renormalize=True: good(-np.asarray(lg), ids, renormalize))


def m_permutation_unstable(mp):
    good = odispatch.permutation

    def permutation(ids, E):
        p = good(ids, E)
        srt = p["sorted"].copy()
        for e in range(E):
            a, b = p["offsets"][e], p["offsets"][e + 1]
            srt[a:b] = srt[a:b][::-1]
        inv = np.empty_like(srt)
        inv[srt] = np.arange(srt.size, dtype=srt.dtype)
        return dict(p, sorted=srt, inv=inv)
    mp.setattr(odispatch, "permutation", permutation)


def m_offsets_inclusive(mp):
    good = odispatch.permutation

    def permutation(ids, E):
        p = good(ids, E)
        off = p["offsets"].copy()
        off[:-1] = off[1:]
        return dict(p, offsets=off)
    mp.setattr(odispatch, "permutation", permutation)


def _ffn(act):
    def expert_ffn(x_t, wg, wu, wd):
        return act(np.asarray(x_t, np.float64), wg.astype(np.float64), wu.astype(np.float64),
                   wd.astype(np.float64))
    return expert_ffn


def m_silu_sign(mp):
    mp.setattr(oexperts, "expert_ffn",
               _ffn(lambda x, g, u, d: d @ ((g @ x) / (1 + np.exp(g @ x)) * (u @ x))))


def m_gate_up_swapped(mp):
    mp.setattr(oexperts, "expert_ffn",
               _ffn(lambda x, g, u, d: d @ ((u @ x) / (1 + np.exp(-(u @ x))) * (g @ x))))


def m_up_dropped(mp):
    mp.setattr(oexperts, "expert_ffn",
               _ffn(lambda x, g, u, d: d @ ((g @ x) / (1 + np.exp(-(g @ x))))))


def m_down_transposed(mp):
    mp.setattr(oexperts, "expert_ffn",
               _ffn(lambda x, g, u, d: d.T @ ((g @ x) / (1 + np.exp(-(g @ x))) * (u @ x))))


def m_combine_drops_gates(mp):
    def moe_layer(x, ids, g, get_expert, shared=None, tokens=None):
        return _plain_moe(x, ids, np.ones_like(g), get_expert, shared, tokens)
    mp.setattr(oexperts, "moe_layer", moe_layer)


def m_combine_first_gate_only(mp):
    def moe_layer(x, ids, g, get_expert, shared=None, tokens=None):
        return _plain_moe(x, ids, np.repeat(np.asarray(g)[:, :1], ids.shape[1], 1), get_expert,
                          shared, tokens)
    mp.setattr(oexperts, "moe_layer", moe_layer)


def m_combine_drops_shared(mp):
    def moe_layer(x, ids, g, get_expert, shared=None, tokens=None):
        return _plain_moe(x, ids, g, get_expert, None, tokens)
    mp.setattr(oexperts, "moe_layer", moe_layer)


def _plain_moe(x, ids, g, get_expert, shared, tokens):
    T, k = ids.shape
    y = np.full((T, x.shape[1]), np.nan)
    for t in (range(T) if tokens is None else tokens):
        acc = np.zeros(x.shape[1])
        for j in range(k):
            acc += float(g[t, j]) * oexperts.expert_ffn(x[t], *get_expert(int(ids[t, j])))
        if shared is not None:
            acc += oexperts.expert_ffn(x[t], *shared)
        y[t] = acc
    return y


def m_resize_highest_free_first(mp):
    def resize(self, new_capacity):
        C = self.capacity
        if new_capacity >= C:
            self.key += [-1] * (new_capacity - C)
            self.stamp += [0] * (new_capacity - C)
            return [], []
        evicted = []
        occ = sorted((self.stamp[s], s) for s in range(C) if self.key[s] >= 0)
        n = len(occ)
        for _, s in occ:
            if n <= new_capacity:
                break
            evicted.append(self.key[s])
            self.key[s], self.stamp[s] = -1, 0
            n -= 1
        moves = []
        free = [s for s in range(new_capacity) if self.key[s] < 0]
        for s in range(new_capacity, C):
            if self.key[s] >= 0:
                d = free.pop()                      # the planted mistake
                self.key[d], self.stamp[d] = self.key[s], self.stamp[s]
                moves.append((s, d))
        del self.key[new_capacity:]
        del self.stamp[new_capacity:]
        return moves, evicted
    mp.setattr(ocache.SlotCache, "resize", resize)


def m_resize_evicts_most_recent(mp):
    good = ocache.SlotCache.resize

    def resize(self, new_capacity):
        # negate the stamps so the eviction order reverses, then restore them
        self.stamp = [-s if k >= 0 else 0 for s, k in zip(self.stamp, self.key)]
        moves, evicted = good(self, new_capacity)
        self.stamp = [-s if s else 0 for s in self.stamp]
        return moves, evicted
    mp.setattr(ocache.SlotCache, "resize", resize)


def m_reset_keeps_most_recent(mp):
    def reset(self):
        keep = max(range(self.capacity), key=lambda s: self.stamp[s])
        k, st = self.key[keep], self.stamp[keep]
        n = sum(1 for x in self.key if x >= 0)
        self.key = [-1] * self.capacity
        self.stamp = [0] * self.capacity
        self.key[keep], self.stamp[keep] = k, st
        return n
    mp.setattr(ocache.SlotCache, "reset", reset)


def m_reset_rewinds_clock(mp):
    good = ocache.SlotCache.reset

    def reset(self):
        n = good(self)
        self.clock = 0
        return n
    mp.setattr(ocache.SlotCache, "reset", reset)


def m_lookup_hits_not_pinned(mp):
    def lookup(self, layer, experts, insert=None):
        # victims may include slots hit earlier in the same call
        if insert is None:
            insert = self.policy != "static"
        experts = [int(e) for e in experts]
        keys = [layer * self.E + e for e in experts]
        slots = [None] * len(keys)
        misses = []
        for i, kk in enumerate(keys):
            s = self.slot_of(kk)
            if s is None:
                misses.append(i)
            else:
                self.clock += 1
                self.stamp[s] = self.clock
                slots[i] = s
                self.hits += 1
        rng = self.victim_range(layer)
        empty = [s for s in rng if self.key[s] < 0]
        old = sorted((self.stamp[s], s) for s in rng if self.key[s] >= 0)
        victims = empty + [s for _, s in old] if insert else []
        fills, bypass = [], []
        for r, i in enumerate(misses):
            if r < len(victims):
                s = victims[r]
                self.key[s] = keys[i]
                self.clock += 1
                self.stamp[s] = self.clock
                slots[i] = s
                fills.append((s, layer, experts[i]))
                self.fills += 1
            else:
                slots[i] = -1 - (r - len(victims))
                bypass.append((r - len(victims), layer, experts[i]))
                self.bypasses += 1
        return slots, fills, bypass
    mp.setattr(ocache.SlotCache, "lookup", lookup)


def m_lookup_victims_most_recent_first(mp):
    good = ocache.SlotCache.lookup

    def lookup(self, layer, experts, insert=None):
        # reverse the recency of the occupied slots before the call
        occ = sorted((s for s in range(self.capacity) if self.key[s] >= 0),
                     key=lambda s: self.stamp[s])
        vals = [self.stamp[s] for s in occ]
        for s, v in zip(occ, reversed(vals)):
            self.stamp[s] = v
        return good(self, layer, experts, insert)
    mp.setattr(ocache.SlotCache, "lookup", lookup)


def m_prefetch_ignores_pinning(mp):
    good = ocache.SlotCache.prefetch

    def prefetch(self, layer, experts, pinned):
        return good(self, layer, experts, self.clock)
    mp.setattr(ocache.SlotCache, "prefetch", prefetch)


def m_prefetch_hits_not_stamped(mp):
    good = ocache.SlotCache.prefetch

    def prefetch(self, layer, experts, pinned):
        keys = {layer * self.E + int(e) for e in experts}
        kept = {s: self.stamp[s] for s in range(self.capacity) if self.key[s] in keys}
        fills = good(self, layer, experts, pinned)
        for s, st in kept.items():
            if self.key[s] in keys:
                self.stamp[s] = st
        return fills
    mp.setattr(ocache.SlotCache, "prefetch", prefetch)


def m_prefetch_victims_by_index(mp):
    def prefetch(self, layer, experts, pinned):
        experts = [int(e) for e in experts]
        misses = []
        for e in experts:
            kk = layer * self.E + e
            s = self.slot_of(kk)
            if s is None:
                misses.append(kk)
            else:
                self.clock += 1
                self.stamp[s] = self.clock
        victims = [s for s in range(self.capacity)
                   if self.key[s] < 0 or (self.stamp[s] <= pinned and self.key[s] not in
                                          {layer * self.E + x for x in experts})]
        fills = []
        for kk, s in zip(misses, victims):
            self.key[s] = kk
            self.clock += 1
            self.stamp[s] = self.clock
            fills.append((s, layer, kk - layer * self.E))
        return fills
    mp.setattr(ocache.SlotCache, "prefetch", prefetch)


def m_bf16_truncates(mp):
    def trunc(a):
        u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
        return (u >> np.uint32(16)).astype(np.uint16)
    mp.setattr(gen, "f32_to_bf16_bits", trunc)


def m_bf16_ties_away(mp):
    def away(a):
        u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
        return ((u + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)
    mp.setattr(gen, "f32_to_bf16_bits", away)


def m_mx_scale_off_by_one(mp):
    good = omx.block_exponents
    mp.setattr(omx, "block_exponents", lambda v: good(v) + 1)


def m_mx_truncates(mp):
    def round_trunc(t):
        t = np.asarray(t, dtype=np.float64)
        a = np.abs(t)
        with np.errstate(divide="ignore"):
            e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
        step = np.ldexp(1.0, (e - 3).astype(np.int64))
        return np.copysign(np.minimum(np.floor(a / step) * step, 448.0), t)
    mp.setattr(omx, "round_e4m3", round_trunc)


def m_mx_no_clamp(mp):
    def round_noclamp(t):
        t = np.asarray(t, dtype=np.float64)
        a = np.abs(t)
        with np.errstate(divide="ignore"):
            e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
        step = np.ldexp(1.0, (e - 3).astype(np.int64))
        return np.copysign(np.round(a / step) * step, t)
    mp.setattr(omx, "round_e4m3", round_noclamp)


def m_mx_block_of_16(mp):
    def quant16(v):
        v = np.asarray(v, dtype=np.float64)
        b = v.reshape(v.shape[:-1] + (v.shape[-1] // 16, 16))
        amax = np.max(np.abs(b), axis=-1)
        with np.errstate(divide="ignore"):
            e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
        sc = np.repeat(np.ldexp(1.0, e.astype(np.int64)), 16, axis=-1)
        return omx.round_e4m3(v / sc) * sc
    mp.setattr(omx, "quantize_mxfp8", quant16)


def m_mx_h_not_quantised(mp):
    def ffn(xq_t, wg, wu, wd):
        x = np.asarray(xq_t, dtype=np.float64)
        a, b = wg.astype(np.float64) @ x, wu.astype(np.float64) @ x
        return wd.astype(np.float64) @ (a / (1.0 + np.exp(-a)) * b)
    mp.setattr(omx, "expert_ffn_mx", ffn)


def _mx_deviation_variant(upper_only=False, ref_exponent_only=False):
    def dev_fn(h, dh):
        h, dh = np.asarray(h, np.float64), np.asarray(dh, np.float64)
        q_ref = omx.quantize_mxfp8(h)
        nb = h.shape[-1] // 32
        hb, db_, qb = (a.reshape(a.shape[:-1] + (nb, 32)) for a in (h, dh, q_ref))
        dev = np.zeros_like(hb)
        e_ref = omx.block_exponents(h)
        amax_lo = np.max(np.maximum(np.abs(hb) - db_, 0.0), axis=-1)
        amax_hi = np.max(np.abs(hb) + db_, axis=-1)
        for idx in np.ndindex(e_ref.shape):
            if ref_exponent_only:
                es = [int(e_ref[idx])]
            else:
                lo_e = -127 if amax_lo[idx] == 0 else int(np.floor(np.log2(amax_lo[idx]))) - 8
                es = range(max(lo_e, -127), int(np.floor(np.log2(amax_hi[idx]))) - 8 + 1)
            for e in es:
                s = np.ldexp(1.0, e)
                up = np.abs(omx.round_e4m3((hb[idx] + db_[idx]) / s) * s - qb[idx])
                dn = np.abs(omx.round_e4m3((hb[idx] - db_[idx]) / s) * s - qb[idx])
                dev[idx] = np.maximum(dev[idx], up if upper_only else np.maximum(up, dn))
        return dev.reshape(h.shape)
    return dev_fn


def m_mx_bound_upper_end_only(mp):
    mp.setattr(omx, "mx_h_deviation", _mx_deviation_variant(upper_only=True))


def m_mx_bound_fixed_exponent(mp):
    mp.setattr(omx, "mx_h_deviation", _mx_deviation_variant(ref_exponent_only=True))


def m_mx_bound_drops_up_error(mp):
    def bound(xq, wg, wu, wd, h_rel, dot_err=omx.mfma_dot_err):
        x = np.atleast_2d(np.asarray(xq, np.float64))
        wg, wu, wd = (np.asarray(w, np.float64) for w in (wg, wu, wd))
        a, b = x @ wg.T, x @ wu.T
        da = dot_err(np.abs(x), np.abs(wg))
        silu = a / (1.0 + np.exp(-a))
        h = silu * b
        dh = omx.SILU_LIP * da * np.abs(b) + h_rel * np.abs(h)
        hq = omx.quantize_mxfp8(h)
        out = (hq @ wd.T, omx.mx_h_deviation(h, dh) @ np.abs(wd).T,
               dot_err(np.abs(hq), np.abs(wd)))
        return tuple(o[0] for o in out) if np.ndim(xq) == 1 else out
    mp.setattr(omx, "expert_ffn_mx_bound", bound)


def m_nv_block_of_32(mp):
    def dequant(packed, scales, matrix_scale):
        vals = omxfp4.decode_e2m1(omxfp4.unpack_nibbles(packed)).astype(np.float64)
        s = np.repeat(onvfp4.e4m3_values(scales)[..., ::2], 32, axis=-1)
        return vals * s * float(np.float32(matrix_scale))
    mp.setattr(onvfp4, "dequant", dequant)


def m_nv_matrix_scale_ignored(mp):
    good = onvfp4.dequant
    mp.setattr(onvfp4, "dequant", lambda p, s, t: good(p, s, 1.0))


def m_nv_e4m3_mantissa_dropped(mp):
    good = onvfp4.e4m3_values
    mp.setattr(onvfp4, "e4m3_values", lambda c: good(np.asarray(c) & 0xF8))


# --------------------------------------------------------- pins to run
MXFP4_PINS = [p_mxfp4.test_e2m1_table_matches_spec_fixture,
              p_mxfp4.test_e2m1_table_matches_bitfield_closed_form,
              p_mxfp4.test_nibble_order_low_first, p_mxfp4.test_dequant_all_codes_all_scales,
              p_mxfp4.test_dequant_constant_block, p_mxfp4.test_dequant_block_boundary_and_rows]
ROUTER_PINS = [p_router.test_logits_are_exact_sum_rounded_once,
               p_router.test_uniform_logits_pick_lowest_ids_equal_gates,
               p_router.test_duplicated_columns_tie_to_lower_id,
               p_router.test_topk_against_python_sort, p_router.test_forced_bias_selects_the_set,
               p_router.test_two_expert_gate_closed_form,
               lambda: p_router.test_gates_sum_to_one_and_match_softmax(3)]
DISPATCH_PINS = [lambda: p_dispatch.test_permutation_matches_numpy(37, 6, 256),
                 lambda: p_dispatch.test_permutation_matches_numpy(4, 2, 8)]
EXPERT_PINS = [lambda: p_experts.test_tiny_layer_equals_dense_masked_reference(0, False, 512),
               lambda: p_experts.test_tiny_layer_equals_dense_masked_reference(4, True, 256),
               p_experts.test_zero_gate_weights_leave_only_shared,
               p_experts.test_identity_down_projection_returns_swiglu,
               p_experts.test_all_ones_closed_form]
CACHE_PINS = [p_cache.test_matches_textbook_lru_when_unique_set_fits,
              lambda: p_cache.test_brute_force_against_recency_list(3, 1, 2, 5),
              p_cache.test_bypass_when_unique_set_exceeds_capacity,
              p_cache.test_resize_invariants, p_cache.test_resize_hand_computed_slot_numbering,
              lambda: p_cache.test_resize_brute_force_against_rank_model(4, 3, 3),
              p_cache.test_reset_is_a_fresh_cache_at_the_same_clock,
              p_cache.test_prefetch_hand_computed, p_cache.test_prefetch_into_empty_slots_ascending,
              lambda: [p_cache.test_prefetch_matches_brute_force(s) for s in range(6)],
              p_cache.test_prefetch_with_nothing_pinned_is_a_lookup]
MX_PINS = [p_mx.test_e4m3_fields, p_mx.test_round_e4m3_is_nearest_with_ties_to_even,
           p_mx.test_block_scale_rule, p_mx.test_quantize_closed_forms,
           p_mx.test_mx_layer_equals_plain_layer_on_representable_inputs,
           p_mx.test_mx_layer_near_plain_layer]
MX_BOUND_PINS = [p_mx.test_bound_with_zero_allowance_is_the_mx_layer, p_mx.test_mfma_dot_err_closed_form,
                 lambda: p_mx.test_bound_covers_every_kernel_inside_the_allowance(0),
                 p_mx.test_bound_covers_the_up_error_when_the_gate_sum_does_not_cancel,
                 p_mx.test_h_deviation_brute_force_on_small_blocks,
                 lambda: p_mx.test_decision_allowance_rejects_sloppy_kernels(256, 256),
                 p_mx.test_layer_bound_sums_the_experts]
NV_PINS = [p_nvfp4.test_e4m3_decoding_matches_torch_float8,
           p_nvfp4.test_block_of_16_and_matrix_scale,
           p_nvfp4.test_power_of_two_scales_reduce_to_mxfp4,
           p_nvfp4.test_mantissa_scales_are_exact_products,
           p_nvfp4.test_expert_dequant_uses_each_matrix_scale]
BF16_PINS = [p_bf16.test_ties_go_to_even, p_bf16.test_special_values_match_torch,
             p_bf16.test_random_values_match_torch]

MUTATIONS = [
    (m_nibbles_high_first, MXFP4_PINS + EXPERT_PINS),
    (m_scale_bias_126, MXFP4_PINS),
    (m_sign_dropped, MXFP4_PINS),
    (m_block_of_16, MXFP4_PINS),
    (m_logits_drop_bias, ROUTER_PINS),
    (m_logits_reversed_k, ROUTER_PINS),
    (m_logits_fp32_accumulation, ROUTER_PINS),
    (m_topk_ties_to_higher_id, ROUTER_PINS),
    (m_gates_not_renormalised, ROUTER_PINS),
    (m_gates_sign_flipped, ROUTER_PINS),
    (m_permutation_unstable, DISPATCH_PINS),
    (m_offsets_inclusive, DISPATCH_PINS),
    (m_silu_sign, EXPERT_PINS),
    (m_gate_up_swapped, EXPERT_PINS),
    (m_up_dropped, EXPERT_PINS),
    (m_down_transposed, EXPERT_PINS),
    (m_combine_drops_gates, EXPERT_PINS),
    (m_combine_first_gate_only, EXPERT_PINS),
    (m_combine_drops_shared, EXPERT_PINS),
    (m_resize_highest_free_first, CACHE_PINS),
    (m_resize_evicts_most_recent, CACHE_PINS),
    (m_lookup_hits_not_pinned, CACHE_PINS),
    (m_reset_keeps_most_recent, CACHE_PINS),
    (m_reset_rewinds_clock, CACHE_PINS),
    (m_lookup_victims_most_recent_first, CACHE_PINS),
    (m_prefetch_ignores_pinning, CACHE_PINS),
    (m_prefetch_hits_not_stamped, CACHE_PINS),
    (m_prefetch_victims_by_index, CACHE_PINS),
    (m_mx_scale_off_by_one, MX_PINS),
    (m_mx_truncates, MX_PINS),
    (m_mx_no_clamp, MX_PINS),
    (m_mx_block_of_16, MX_PINS),
    (m_mx_h_not_quantised, MX_PINS),
    (m_mx_bound_upper_end_only, MX_BOUND_PINS),
    (m_mx_bound_fixed_exponent, MX_BOUND_PINS),
    (m_mx_bound_drops_up_error, MX_BOUND_PINS),
    (m_nv_block_of_32, NV_PINS),
    (m_nv_matrix_scale_ignored, NV_PINS),
    (m_nv_e4m3_mantissa_dropped, NV_PINS),
    (m_bf16_truncates, BF16_PINS),
    (m_bf16_ties_away, BF16_PINS),
]


def _caught(pins):
    """Names of the pins that fail (any exception counts: a planted mistake
    that makes a pin crash is caught too)."""
    failed = []
    for pin in pins:
        try:
            pin()
        except Exception as exc:  # noqa: BLE001
            failed.append(f"{getattr(pin, '__name__', 'pin')}: {type(exc).__name__}")
    return failed


@pytest.mark.parametrize("mutate,pins", MUTATIONS, ids=[m.__name__ for m, _ in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, mutate, pins):
    assert not _caught(pins), "a pin fails on the unmodified oracle"
    with monkeypatch.context() as mp:
        mutate(mp)
        failed = _caught(pins)
    assert failed, f"no pin catches {mutate.__name__}"


def test_pins_pass_again_after_the_mutations():
    """monkeypatch restored every module: the plain oracle passes its pins."""
    assert oracle.router.topk is orouter.topk
    for pins in (MXFP4_PINS, ROUTER_PINS, DISPATCH_PINS, EXPERT_PINS, CACHE_PINS, MX_PINS,
                 MX_BOUND_PINS, NV_PINS, BF16_PINS):
        assert not _caught(pins)
