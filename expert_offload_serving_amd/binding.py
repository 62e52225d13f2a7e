"""ctypes binding of libmoe (include/moe.h): same names, marshalling only.

Device buffers are passed as torch tensors (their data_ptr) or raw integer
addresses; host arrays as numpy arrays.  Streams default to torch's current
stream.  Every failing call raises MoEError with the library's status and
message.  If libmoe.so has not been built this module fails to import:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

STATUS = {0: "OK", -1: "INVALID_ARG", -2: "OOM", -3: "HIP", -4: "CAPACITY", -5: "STATE",
          -6: "UNSUPPORTED"}


class MoEError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{func}: {self.name}: {message}")


class moe_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "inter", "n_experts", "top_k", "n_layers", "has_shared", "renormalize",
        "max_tokens", "cache_slots", "staging_slots", "max_prefill_tokens", "cache_policy",
        "weight_format", "prefill_format")]


class moe_timing(ctypes.Structure):
    _fields_ = [("n_decode", ctypes.c_int32), ("n_prefill", ctypes.c_int32),
                ("n_decode_split", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("decode_ms", ctypes.c_double * 6), ("prefill_ms", ctypes.c_double * 4)]


DECODE_KERNELS = ("router", "finalize", "fill", "gateup", "down", "combine")
PREFILL_STAGES = ("routing", "gateup", "down", "combine")


class moe_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "forward_calls", "lookups", "hits", "fills", "bypasses", "evictions", "bytes_h2d",
        "bytes_d2d", "resizes", "prefill_layers", "prefetch_lookups", "prefetch_hits",
        "prefetch_fills")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_expert_bytes": (ctypes.c_size_t, [_I32, _I32]),
    "moe_create": (_I32, [ctypes.POINTER(moe_config), ctypes.POINTER(_P)]),
    "moe_destroy": (_I32, [_P]),
    "moe_set_router": (_I32, [_P, _I32, _P]),
    "moe_set_expert": (_I32, [_P, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "moe_set_layer": (_I32, [_P, _I32, _P, _P, _P, _P, _P]),
    "moe_layer_forward": (_I32, [_P, _I32, _P, _I32, _P, _P, _P, _P, _P, _P]),
    "moe_layer_forward_noalloc": (_I32, [_P, _I32, _P, _I32, _P, _P, _P, _P, _P, _P]),
    "moe_prefill_forward": (_I32, [_P, _I32, _P, _I32, _P, _P, _P, _P]),
    "moe_set_prefill_format": (_I32, [_P, _I32]),
    "expert_cache_lookup": (_I32, [_P, _I32, _P, _P, _P, _P]),
    "expert_cache_fill": (_I32, [_P, _I32, _P, _I32, _P]),
    "expert_cache_resize": (_I32, [_P, _I32, _P]),
    "expert_cache_snapshot": (_I32, [_P, _I32, _P, _P, _P, _P]),
    "moe_inspect_dispatch": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_inspect_prefill": (_I32, [_P, _I32, _P, _P, _P, _P, _P, _P, _P]),
    "moe_inspect_prefill_mx": (_I32, [_P, _P, _P, _P, _P, _P]),
    "moe_get_stats": (_I32, [_P, ctypes.POINTER(moe_stats)]),
    "moe_set_copy_overlap": (_I32, [_P, _I32]),
    "moe_set_prefetch": (_I32, [_P, _I32, _P, _I32]),
    "moe_set_debug": (_I32, [_P, _I32]),
    "expert_cache_reset": (_I32, [_P]),
    "moe_reset_stats": (_I32, [_P]),
    "moe_set_timing": (_I32, [_P, _I32]),
    "moe_get_timing": (_I32, [_P, ctypes.POINTER(moe_timing)]),
    "moe_probe_copy": (_I32, [_P, _P, ctypes.c_size_t, _P]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
            " (there is no fallback implementation)")
    # torch first: its bundled HIP runtime then satisfies libmoe's dependency
    # on libamdhip64, so the process holds one HIP runtime whichever module
    # the caller imports first (two runtimes of one soname leave torch
    # without devices).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int, func: str):
    if status != 0:
        raise MoEError(status, func, lib.moe_last_error().decode(errors="replace"))


def _ptr(obj) -> Optional[int]:
    """Address of a torch tensor, numpy array, int, or None."""
    if obj is None:
        return None
    if isinstance(obj, int):
        return obj
    if hasattr(obj, "data_ptr"):
        return obj.data_ptr()
    if isinstance(obj, np.ndarray):
        assert obj.flags["C_CONTIGUOUS"], "host arrays must be C-contiguous"
        return obj.ctypes.data
    raise TypeError(f"cannot take the address of {type(obj)}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


# ------------------------------------------------------------------ calls
def moe_expert_bytes(hidden: int, inter: int) -> int:
    return int(lib.moe_expert_bytes(hidden, inter))


# moe_config.cache_policy values, in enum order (MOE_CACHE_GLOBAL, ...)
CACHE_POLICIES = ("global", "per_layer", "static")
# moe_config.weight_format values, in enum order (MOE_WEIGHTS_MXFP4, ...)
WEIGHT_FORMATS = ("mxfp4", "bf16", "nvfp4")


def moe_create(**fields) -> int:
    cfg = moe_config(**fields)
    out = _P()
    _check(lib.moe_create(ctypes.byref(cfg), ctypes.byref(out)), "moe_create")
    return out.value


def moe_destroy(ctx: Optional[int]):
    _check(lib.moe_destroy(ctx), "moe_destroy")


def moe_set_router(ctx, layer, h_router: np.ndarray):
    _check(lib.moe_set_router(ctx, layer, _ptr(h_router)), "moe_set_router")


def moe_set_expert(ctx, layer, expert, qg, qu, qd, sg, su, sd):
    _check(lib.moe_set_expert(ctx, layer, expert, *(_ptr(a) for a in (qg, qu, qd, sg, su, sd))),
           "moe_set_expert")


def moe_set_layer(ctx, layer, h_router, h_q, h_s, h_shared_q=None, h_shared_s=None):
    _check(lib.moe_set_layer(ctx, layer, _ptr(h_router), _ptr(h_q), _ptr(h_s), _ptr(h_shared_q),
                             _ptr(h_shared_s)), "moe_set_layer")


def moe_layer_forward(ctx, layer, d_x, T, d_bias, d_y, d_y32=None, d_ids=None, d_gates=None,
                      stream=None):
    _check(lib.moe_layer_forward(ctx, layer, _ptr(d_x), T, _ptr(d_bias), _ptr(d_y), _ptr(d_y32),
                                 _ptr(d_ids), _ptr(d_gates), _stream(stream)), "moe_layer_forward")


def moe_layer_forward_noalloc(ctx, layer, d_x, T, d_bias, d_y, d_y32=None, d_ids=None,
                              d_gates=None, stream=None):
    _check(lib.moe_layer_forward_noalloc(ctx, layer, _ptr(d_x), T, _ptr(d_bias), _ptr(d_y),
                                         _ptr(d_y32), _ptr(d_ids), _ptr(d_gates),
                                         _stream(stream)), "moe_layer_forward_noalloc")


def moe_prefill_forward(ctx, n_layers, d_xs: Sequence, T, d_biases, d_ys: Sequence,
                        d_y32s: Optional[Sequence] = None, stream=None):
    def arr(seq):
        return None if seq is None else ctypes.cast((_P * n_layers)(*[_ptr(a) for a in seq]), _P)
    _check(lib.moe_prefill_forward(ctx, n_layers, arr(d_xs), T, arr(d_biases), arr(d_ys),
                                   arr(d_y32s), _stream(stream)), "moe_prefill_forward")


# moe_config.prefill_format values, in enum order (MOE_PREFILL_BF16, ...)
PREFILL_FORMATS = ("bf16", "mxfp8")


def moe_set_prefill_format(ctx, fmt: str):
    _check(lib.moe_set_prefill_format(ctx, PREFILL_FORMATS.index(fmt)), "moe_set_prefill_format")


def expert_cache_lookup(ctx, layer, d_experts, d_n, d_slot, stream=None):
    _check(lib.expert_cache_lookup(ctx, layer, _ptr(d_experts), _ptr(d_n), _ptr(d_slot),
                                   _stream(stream)), "expert_cache_lookup")


def expert_cache_fill(ctx, layer, h_experts: Sequence[int], stream=None):
    arr = np.ascontiguousarray(np.asarray(h_experts, dtype=np.int32))
    _check(lib.expert_cache_fill(ctx, layer, _ptr(arr) if arr.size else None, int(arr.size),
                                 _stream(stream)), "expert_cache_fill")


def expert_cache_resize(ctx, new_slots: int, stream=None):
    _check(lib.expert_cache_resize(ctx, new_slots, _stream(stream)), "expert_cache_resize")


def expert_cache_snapshot(ctx):
    """Returns (key int32[C], stamp uint64[C], clock)."""
    C = ctypes.c_int32()
    clock = ctypes.c_uint64()
    st = lib.expert_cache_snapshot(ctx, 0, None, None, ctypes.byref(clock), ctypes.byref(C))
    if st not in (0, -4):
        _check(st, "expert_cache_snapshot")
    key = np.empty(max(C.value, 1), np.int32)
    stamp = np.empty(max(C.value, 1), np.uint64)
    _check(lib.expert_cache_snapshot(ctx, C.value, _ptr(key), _ptr(stamp), ctypes.byref(clock),
                                     ctypes.byref(C)), "expert_cache_snapshot")
    return key[:C.value], stamp[:C.value], int(clock.value)


def moe_inspect_dispatch(ctx, E: int, k: int, T_max: int):
    T = ctypes.c_int32()
    nu = ctypes.c_int32()
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sorted_ = np.zeros(T_max * k, np.int32)
    inv = np.zeros(T_max * k, np.int32)
    unique = np.zeros(E, np.int32)
    slot = np.zeros(E, np.int32)
    _check(lib.moe_inspect_dispatch(ctx, ctypes.byref(T), _ptr(counts), _ptr(offsets),
                                    _ptr(sorted_), _ptr(inv), _ptr(unique), ctypes.byref(nu),
                                    _ptr(slot)), "moe_inspect_dispatch")
    n = T.value * k
    return dict(T=T.value, counts=counts, offsets=offsets, sorted=sorted_[:n], inv=inv[:n],
                unique=unique[:nu.value], slot=slot[:nu.value])


def moe_inspect_prefill(ctx, layer: int, E: int, k: int, T_max: int):
    T = ctypes.c_int32()
    ids = np.zeros(T_max * k, np.int32)
    gates = np.zeros(T_max * k, np.float32)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sorted_ = np.zeros(T_max * k, np.int32)
    inv = np.zeros(T_max * k, np.int32)
    _check(lib.moe_inspect_prefill(ctx, layer, ctypes.byref(T), _ptr(ids), _ptr(gates),
                                   _ptr(counts), _ptr(offsets), _ptr(sorted_), _ptr(inv)),
           "moe_inspect_prefill")
    n = T.value
    return dict(T=n, ids=ids[:n * k].reshape(n, k), gates=gates[:n * k].reshape(n, k),
                counts=counts, offsets=offsets, sorted=sorted_[:n * k], inv=inv[:n * k])


def moe_inspect_prefill_mx(ctx, H: int, I: int, k: int, shared: bool, T_max: int):
    T = ctypes.c_int32()
    rows_max = T_max * (k + 1)
    xq = np.zeros(T_max * H, np.uint8)
    xs = np.zeros(T_max * (H // 32), np.uint8)
    hq = np.zeros(rows_max * I, np.uint8)
    hs = np.zeros(rows_max * (I // 32), np.uint8)
    _check(lib.moe_inspect_prefill_mx(ctx, ctypes.byref(T), _ptr(xq), _ptr(xs), _ptr(hq), _ptr(hs)),
           "moe_inspect_prefill_mx")
    n = T.value
    R = n * k + (n if shared else 0)
    return dict(T=n, xq=xq[:n * H].reshape(n, H), xs=xs[:n * (H // 32)].reshape(n, H // 32),
                hq=hq[:R * I].reshape(R, I), hs=hs[:R * (I // 32)].reshape(R, I // 32))


def moe_set_copy_overlap(ctx, mode: int):
    _check(lib.moe_set_copy_overlap(ctx, int(mode)), "moe_set_copy_overlap")


def moe_set_prefetch(ctx, layer: int, d_experts, n: int):
    _check(lib.moe_set_prefetch(ctx, int(layer), d_experts, int(n)), "moe_set_prefetch")


DEBUG_SYNC, DEBUG_FAIL_NEXT_FILL = 1, 2


def moe_set_debug(ctx, flags: int):
    _check(lib.moe_set_debug(ctx, int(flags)), "moe_set_debug")


def expert_cache_reset(ctx):
    _check(lib.expert_cache_reset(ctx), "expert_cache_reset")


def moe_get_stats(ctx) -> dict:
    s = moe_stats()
    _check(lib.moe_get_stats(ctx, ctypes.byref(s)), "moe_get_stats")
    return s.as_dict()


def moe_reset_stats(ctx):
    _check(lib.moe_reset_stats(ctx), "moe_reset_stats")


def moe_set_timing(ctx, enable: bool):
    _check(lib.moe_set_timing(ctx, 1 if enable else 0), "moe_set_timing")


def moe_get_timing(ctx) -> dict:
    """Records and summed milliseconds per decode kernel and prefill stage."""
    t = moe_timing()
    _check(lib.moe_get_timing(ctx, ctypes.byref(t)), "moe_get_timing")
    return dict(n_decode=t.n_decode, n_prefill=t.n_prefill, n_decode_split=t.n_decode_split,
                decode_ms=dict(zip(DECODE_KERNELS, list(t.decode_ms))),
                prefill_ms=dict(zip(PREFILL_STAGES, list(t.prefill_ms))))


def moe_probe_copy(d_src, d_dst, n_bytes: int, stream=None):
    _check(lib.moe_probe_copy(_ptr(d_src), _ptr(d_dst), n_bytes, _stream(stream)),
           "moe_probe_copy")
