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


def dequant_mxfp8(codes: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """Values of MXFP8 data: E4M3 codes [..., n] and E8M0 scale bytes
    [..., n/32] (exponent + 127), each code's value (e4m3_value) times two to
    its block's exponent.  fp64."""
    table = np.array([e4m3_value(c) for c in range(256)])
    codes = np.asarray(codes, dtype=np.uint8)
    e = np.asarray(scale_bytes, dtype=np.int64) - 127
    return table[codes] * np.repeat(np.ldexp(1.0, e), 32, axis=-1)


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


U32 = 2.0 ** -24   # unit roundoff of fp32
MFMA_ALIGN = 2.0 ** -10


def mfma_dot_err(ax: np.ndarray, aw: np.ndarray) -> np.ndarray:
    """Error allowance of dot products computed as chained 128-term scaled
    FP8 x FP4 matrix instructions accumulating in fp32: ax [n][K] and aw [I][K]
    are the operands' magnitudes; returns [n][I].

    Model (measured, not specified by the pages): one instruction's result
    lies within 2^-10 of its largest product magnitude from the exact sum of
    its 128 products (measured on gfx950 over 32768 random outputs whose
    codes span the whole E4M3 range: at most 2^-11.3, 99.9th percentile
    2^-11.8 -- the instruction aligns its products to the largest one rather
    than rounding once in fp32), and each add into the fp32 accumulator
    rounds once (2 u of the running sum of magnitudes per instruction,
    taken over the whole sum)."""
    ax = np.asarray(ax, dtype=np.float64)
    aw = np.asarray(aw, dtype=np.float64)
    K = ax.shape[-1]
    out = np.zeros((ax.shape[0], aw.shape[0]))
    for c in range(0, K, 128):
        out += np.max(ax[:, None, c:c + 128] * aw[None, :, c:c + 128], axis=-1)
    nc = (K + 127) // 128
    return MFMA_ALIGN * out + 2.0 * U32 * nc * (ax @ aw.T)


def mx_h_deviation(h: np.ndarray, dh: np.ndarray) -> np.ndarray:
    """For each element of h (rows of 32-blocks along the last axis), the
    largest change of its MXFP8-quantised value that a computation of h
    within +-dh of the exact value can cause: over every block exponent that
    the perturbed block amax can take and both ends of the element's
    interval (the rounding is monotone in the value, so its reachable
    values lie between those of the ends).  Zero where every value in the
    interval rounds like h itself under the one reachable exponent."""
    h = np.asarray(h, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    nb = h.shape[-1] // 32
    blk = h.shape[:-1] + (nb, 32)
    hb, db_ = h.reshape(blk), dh.reshape(blk)
    qb = quantize_mxfp8(h).reshape(blk)
    lob, hib = hb - db_, hb + db_

    def expo(a):
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(a > 0, a, 1.0))) - E4M3_EMAX
        return np.clip(np.where(a > 0, e, -127), -127, 127).astype(np.int64)

    e_lo = expo(np.max(np.maximum(np.abs(hb) - db_, 0.0), axis=-1))
    e_hi = expo(np.max(np.abs(hb) + db_, axis=-1))
    dev = np.zeros(blk)
    # every exponent from the smallest to the largest reachable amax's; a
    # block with a narrower range repeats its largest
    for d in range(int(np.max(e_hi - e_lo)) + 1 if e_lo.size else 0):
        s = np.ldexp(1.0, np.minimum(e_lo + d, e_hi))[..., None]
        dev = np.maximum(dev, np.maximum(np.abs(round_e4m3(lob / s) * s - qb),
                                         np.abs(round_e4m3(hib / s) * s - qb)))
    return dev.reshape(h.shape)


SILU_LIP = 1.1   # bound of |d/da (a * sigmoid(a))| over the reals (max ~1.0998)


def expert_h_mx(xq, wg, wu, h_rel: float = 2.0 ** -16, dot_err=mfma_dot_err):
    """h = silu(W_g xq) * (W_u xq) in fp64 for one row xq [H] or a batch [n][H]
    of already quantised inputs, with dh, the most a kernel computing gate
    and up within dot_err of the exact sums and h within h_rel of its
    magnitude on top can be off: the interval whose quantisation decisions
    mx_h_deviation spans.  Returns (h, dh), [n][I] (or [I] for one row)."""
    x = np.asarray(xq, dtype=np.float64)
    one = x.ndim == 1
    x = np.atleast_2d(x)
    wg, wu = np.asarray(wg, dtype=np.float64), np.asarray(wu, dtype=np.float64)
    ax = np.abs(x)
    a, b = x @ wg.T, x @ wu.T
    da, db = dot_err(ax, np.abs(wg)), dot_err(ax, np.abs(wu))
    with np.errstate(over="ignore"):
        silu = a / (1.0 + np.exp(-a))
    h = silu * b
    # |silu(a') b' - silu(a) b| <= L da (|b| + db) + |silu(a)| db for
    # |a' - a| <= da, |b' - b| <= db; the evaluation error on top is
    # relative to the computed value
    dh0 = SILU_LIP * da * (np.abs(b) + db) + np.abs(silu) * db
    dh = dh0 + h_rel * (np.abs(h) + dh0)
    return (h[0], dh[0]) if one else (h, dh)


def expert_ffn_mx_bound(xq, wg, wu, wd, h_rel: float, dot_err=mfma_dot_err):
    """Tokens through one expert in the native-MX mode (as expert_ffn_mx, for
    one row xq [H] or a batch [n][H] of already quantised inputs) with two
    allowances for a kernel that computes in fp32: flip, per output element,
    the most that the quantisation decisions on h can move it when gate and
    up are computed within dot_err of the exact sums and h = silu(gate) * up
    is evaluated within h_rel of its magnitude on top (expert_h_mx); arith,
    the error of the down product itself (dot_err of its operands).
    dot_err(|x|, |W|) gives the allowance of x @ W.T from the operands'
    magnitudes.  Returns (y, flip, arith), fp64, shaped like xq."""
    one = np.ndim(xq) == 1
    h, dh = expert_h_mx(np.atleast_2d(xq), wg, wu, h_rel=h_rel, dot_err=dot_err)
    wd = np.asarray(wd, dtype=np.float64)
    hq = quantize_mxfp8(h)
    awd = np.abs(wd)
    y = hq @ wd.T
    flip = mx_h_deviation(h, dh) @ awd.T
    arith = dot_err(np.abs(hq), awd)
    if one:
        return y[0], flip[0], arith[0]
    return y, flip, arith


def moe_layer_mx_bound(x, ids, g, get_expert, shared=None, tokens=None, h_rel: float = 2.0 ** -16,
                       dot_err=mfma_dot_err):
    """moe_layer_mx with the allowances of expert_ffn_mx_bound summed over
    each token's experts (weighted by |g|), plus the fp32 error of combining
    them ((k + 2) roundings of the sum of the parts' magnitudes).  A kernel
    of the native-MX mode that computes in fp32 under the stated arithmetic
    model gives, for every checked element, |y_kernel - y| <= flip + arith.
    Tokens are grouped by expert so that each expert's products run as one
    matrix product.  Returns (y, flip, arith), each [T][H] (rows outside
    tokens NaN)."""
    T, k = ids.shape
    H = x.shape[1]
    rows = np.arange(T) if tokens is None else np.asarray(list(tokens), dtype=np.int64)
    xq = quantize_mxfp8(np.asarray(x, dtype=np.float64)[rows])
    n = len(rows)
    acc, fl, ar, mag = (np.zeros((n, H)) for _ in range(4))
    sel = ids[rows]
    for e in np.unique(sel):
        r, j = np.nonzero(sel == e)
        ye, fe, ae = expert_ffn_mx_bound(xq[r], *get_expert(int(e)), h_rel=h_rel, dot_err=dot_err)
        gj = np.asarray(g, dtype=np.float64)[rows[r], j][:, None]
        np.add.at(acc, r, gj * ye)
        np.add.at(fl, r, np.abs(gj) * fe)
        np.add.at(ar, r, np.abs(gj) * ae)
        np.add.at(mag, r, np.abs(gj * ye))
    parts = k
    if shared is not None:
        ye, fe, ae = expert_ffn_mx_bound(xq, *shared, h_rel=h_rel, dot_err=dot_err)
        acc += ye
        fl += fe
        ar += ae
        mag += np.abs(ye)
        parts += 1
    y, flip, arith = (np.full((T, H), np.nan) for _ in range(3))
    y[rows], flip[rows] = acc, fl
    arith[rows] = ar + (parts + 2) * U32 * mag
    return y, flip, arith
