"""Expert SwiGLU FFN and the weighted combine, per token, per chosen expert.

Test infrastructure (see the package docstring).

The pages fix only that partial expert results are summed at the end with no
approximation (jansverre.net FreeToken article, section "Hva er
FreeToken?") and that DeepSeek-V4-Flash runs MXFP4 experts (same article,
section "Hvor raskt kjører modellene?").  Readings where they are silent:

* FFN: o = W_d (silu(W_g x) * (W_u x)), silu(z) = z / (1 + exp(-z)), no
  biases; W_g, W_u are [I][H], W_d is [H][I];
* combine: y_t = sum_j g[t, j] * o_{t,j} (+ o_{t,shared}); the shared expert
  is added with weight 1 and takes no part in top-k or renormalisation;
* all arithmetic here is fp64 on exactly dequantised weights.

Experts come as MXFP4 (codes and scales, decoded by ``mxfp4.dequant``) or as
bf16 matrices, the format the pages run the 35B-A3B model in (jansverre.net
FreeToken article, section "Hvor raskt kjører modellene?"); a bf16 value is
the fp32 number whose upper 16 bits are its bit pattern and whose lower 16
are zero.
"""
import numpy as np

from .mxfp4 import dequant


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their values as fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def dequant_expert(w):
    """Canonical expert (MXFP4 codes and scales, bf16 matrices, or NVFP4
    codes, block scales and matrix scales) -> (W_g, W_u, W_d), exact (fp32
    for MXFP4 and bf16, fp64 for NVFP4)."""
    if hasattr(w, "wg"):
        return bf16_values(w.wg), bf16_values(w.wu), bf16_values(w.wd)
    if hasattr(w, "tg"):
        from . import nvfp4
        return (nvfp4.dequant(w.qg, w.sg, w.tg), nvfp4.dequant(w.qu, w.su, w.tu),
                nvfp4.dequant(w.qd, w.sd, w.td))
    return dequant(w.qg, w.sg), dequant(w.qu, w.su), dequant(w.qd, w.sd)


def expert_ffn(x_t: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray):
    """One token through one expert, fp64.  x_t: [H]."""
    x = np.asarray(x_t, dtype=np.float64)
    a = wg.astype(np.float64) @ x
    b = wu.astype(np.float64) @ x
    # exp(-a) overflows to inf for a below about -709; a / inf is then -0,
    # which is silu's limit there, so the overflow is expected and silenced
    with np.errstate(over="ignore"):
        h = a / (1.0 + np.exp(-a)) * b
    return wd.astype(np.float64) @ h


def moe_layer(x: np.ndarray, ids: np.ndarray, g: np.ndarray, get_expert,
              shared=None, tokens=None):
    """y[t] = sum_j g[t,j] * FFN_{ids[t,j]}(x[t]) (+ FFN_shared(x[t])), fp64.

    x: [T][H] activation values; ids, g: [T][k]; get_expert(e) returns the
    dequantised (W_g, W_u, W_d) of routed expert e; shared: the same triple
    or None.  tokens: optional subset of token rows to evaluate (others are
    left as NaN) so that large batches can be sampled.
    """
    T, k = ids.shape
    H = x.shape[1]
    y = np.full((T, H), np.nan, dtype=np.float64)
    rows = range(T) if tokens is None else tokens
    for t in rows:
        acc = np.zeros(H, dtype=np.float64)
        for j in range(k):
            wg, wu, wd = get_expert(int(ids[t, j]))
            acc += float(g[t, j]) * expert_ffn(x[t], wg, wu, wd)
        if shared is not None:
            acc += expert_ffn(x[t], *shared)
        y[t] = acc
    return y
