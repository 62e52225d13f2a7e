"""Router: logits, top-k selection and gate weights.

Test infrastructure (see the package docstring).

The pages say only that each token activates a few of many experts (6 of 256
for DeepSeek-V4-Flash; aiforradalom.hu article, section "A Mixture-of-Experts
(MoE) kihívásai és a FreeToken megoldásai") and that offloading leaves the
router unchanged (jansverre.net FreeToken article, section "Hva er
FreeToken?").  Readings taken where they are silent:

* scores are a softmax over all E experts; selection is the top k logits;
* logits accumulate in fp64 and are rounded once to fp32 (any summation
  order gives the same fp32 value except within ~1e-14 of a rounding
  midpoint);
* ties order by lower expert id first; ids are listed best first;
* with renormalisation the k gates are the softmax restricted to the chosen
  experts (identical to full softmax then dividing by the chosen mass);
  without it they are the full-softmax probabilities of the chosen experts.
"""
import numpy as np


def logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """l[t, e] = fp32(sum_h x[t, h] * W_r[h, e] + bias[t, e]), fp64 inside.

    x: [T][H] activation values (bf16 values as floats); w_router: [H][E]
    fp32; bias: [T][E] fp32 or None.
    """
    acc = np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64)
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float64)
    return acc.astype(np.float32)


def topk(lg: np.ndarray, k: int) -> np.ndarray:
    """ids[t, :] = the k experts of largest logit, ordered by
    (logit descending, expert id ascending).  int32 [T][k]."""
    T, E = lg.shape
    out = np.empty((T, k), dtype=np.int32)
    ids = np.arange(E)
    for t in range(T):
        # lexsort: last key is primary -> primary -logit, secondary id
        order = np.lexsort((ids, -lg[t].astype(np.float64)))
        out[t] = order[:k]
    return out


def gates(lg: np.ndarray, ids: np.ndarray, renormalize: bool = True) -> np.ndarray:
    """Gate weights of the chosen experts, computed in fp64, stored fp32."""
    T, k = ids.shape
    g = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        l = lg[t].astype(np.float64)
        if renormalize:
            sel = l[ids[t]]
            z = np.exp(sel - sel[0])       # sel[0] is the largest logit
            g[t] = z / z.sum()
        else:
            z = np.exp(l - l.max())
            g[t] = z[ids[t]] / z.sum()
    return g.astype(np.float32)


def route(x, w_router, k, bias=None, renormalize=True):
    """Logits, ids and gates for one token batch."""
    lg = logits(x, w_router, bias)
    ids = topk(lg, k)
    return lg, ids, gates(lg, ids, renormalize)
