"""MXFP8 block quantisation of activations, and the expert layer computed on
block-quantised activations (the opt-in native-MX prefill mode).

Test infrastructure (see the package docstring).

The method computes the plain layer (oracle.experts).  The native-MX mode is
this build's opt-in variant: it meets the MXFP4 weights with activations in
the same family of formats (the pages run MXFP4 experts: jansverre.net
FreeToken article, section "Hvor raskt kjører modellene?"), so that both
expert matrices run on the scaled FP8 x FP4 matrix instructions.  What it
computes, stated here as the reference for that mode:

* x (each token row) and h (each (token, expert) row) are cut into blocks of
  32 consecutive elements along the reduction axis;
* each block gets one power-of-two scale 2^e with e = floor(log2(amax)) - 8,
  amax the block's largest magnitude (8 is E4M3's largest exponent: the OCP
  MX v1.0 rule), clamped to the E8M0 range [-127, 127]; an all-zero block
  takes e = -127;
* each element becomes an E4M3 value v / 2^e rounded to nearest, ties to
  even, on the E4M3 grid (bias 7, 3 mantissa bits, subnormals down to 2^-9),
  clamped to +-448 (E4M3's largest finite value);
* the layer is then the plain one on the dequantised x for the gate and up
  products and on the dequantised h for the down product, in fp64.

The E4M3 and E8M0 encodings are the OCP MX v1.0 specification's; the pages do
not spell them out.
"""
import numpy as np

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of E4M3's largest binade
E4M3_MIN_NORMAL_EXP = -6
E4M3_MANT_BITS = 3


def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3 code from its fields (sign, 4-bit exponent with
    bias 7, 3-bit mantissa); 0x7F and 0xFF are NaN."""
    code &= 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def round_e4m3(t: np.ndarray) -> np.ndarray:
    """t rounded to the nearest E4M3 value (ties to even), clamped to
    +-448.  fp64 in and out; every E4M3 value is exact in fp64."""
    t = np.asarray(t, dtype=np.float64)
    a = np.abs(t)
    # spacing of the E4M3 grid around |t|: 2^(e-3) in binade e >= -6, and the
    # subnormal spacing 2^-9 below 2^-6
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, E4M3_MIN_NORMAL_EXP)
    step = np.ldexp(1.0, (e - E4M3_MANT_BITS).astype(np.int64))
    q = np.round(a / step) * step          # numpy rounds halves to even
    q = np.minimum(q, E4M3_MAX)
    return np.copysign(q, t)


def block_exponents(v: np.ndarray) -> np.ndarray:
    """Scale exponent of each block of 32 along the last axis: floor(log2
    amax) - 8, clamped to [-127, 127]; -127 for an all-zero block."""
    v = np.asarray(v, dtype=np.float64)
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    amax = np.max(np.abs(blocks), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E4M3_EMAX
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_mxfp8(v: np.ndarray) -> np.ndarray:
    """v block-quantised to MXFP8 (E4M3 elements, one E8M0 scale per 32
    along the last axis) and dequantised again: the values the native-MX mode
    multiplies.  fp64."""
    v = np.asarray(v, dtype=np.float64)
    assert v.shape[-1] % 32 == 0
    e = block_exponents(v)
    scale = np.repeat(np.ldexp(1.0, e), 32, axis=-1)
    return round_e4m3(v / scale) * scale


def expert_ffn_mx(xq_t: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray):
    """One token through one expert with an already quantised input xq_t:
    the gate and up products on it, h quantised to MXFP8, the down product."""
    x = np.asarray(xq_t, dtype=np.float64)
    a = wg.astype(np.float64) @ x
    b = wu.astype(np.float64) @ x
    with np.errstate(over="ignore"):
        h = a / (1.0 + np.exp(-a)) * b
    return wd.astype(np.float64) @ quantize_mxfp8(h)


def moe_layer_mx(x: np.ndarray, ids: np.ndarray, g: np.ndarray, get_expert, shared=None,
                 tokens=None):
    """y[t] = sum_j g[t,j] * FFN_mx_{ids[t,j]}(Q(x[t])) (+ FFN_mx_shared), fp64:
    oracle.experts.moe_layer with every token row of x quantised to MXFP8 once
    and h quantised per (token, expert) inside each expert.  Routing is the
    caller's, on the unquantised x (the router is unchanged).  tokens: optional
    subset of rows to evaluate (the others are NaN)."""
    T, k = ids.shape
    H = x.shape[1]
    xq = quantize_mxfp8(np.asarray(x, dtype=np.float64))
    y = np.full((T, H), np.nan, dtype=np.float64)
    for t in (range(T) if tokens is None else tokens):
        acc = np.zeros(H, dtype=np.float64)
        for j in range(k):
            wg, wu, wd = get_expert(int(ids[t, j]))
            acc += float(g[t, j]) * expert_ffn_mx(xq[t], wg, wu, wd)
        if shared is not None:
            acc += expert_ffn_mx(xq[t], *shared)
        y[t] = acc
    return y
