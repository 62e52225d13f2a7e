"""Seeded synthetic inputs for the routed MoE expert-layer forward.

This module draws inputs only: token activations, router weights, MXFP4
expert weights in their canonical packed form, and the Zipf routing traces
that bias the router.  It holds none of the layer's arithmetic (no
dequantisation, no routing, no expert math), so both the CPU oracle and the
HIP path may consume what it produces.

Workload shapes follow the synthetic stand-ins for the models the FreeToken
pages measure (Qwen3.6-35B-A3B, DeepSeek-V4-Flash, GLM-5.2; jansverre.net
page, sections "Hvor raskt kjører modellene?" and "Hvorfor er båndbredden
viktigere enn antall kjerner?").  No trained weights or real prompts are used.

Randomness: every array has its own PCG64 stream keyed by
(seed, purpose, layer, index, ...) through ``numpy.random.SeedSequence``'s
``spawn_key``, so any expert, step or layer can be regenerated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

# purpose tags for the SeedSequence spawn keys
_ROUTER, _EXPERT, _SHARED, _X, _TRACE, _PERM = 1, 2, 3, 4, 5, 6

#: additive router bias that forces a drawn expert set into the top-k
BIAS_STRENGTH = 32.0


@dataclass(frozen=True)
class Shape:
    """Shape of one MoE layer stack."""

    H: int          # hidden size
    I: int          # expert intermediate size
    E: int          # routed experts
    k: int          # experts per token
    layers: int = 1
    shared: bool = False      # one always-on shared expert per layer
    renormalize: bool = True  # renormalise the top-k gates to sum to 1
    weights: str = "mxfp4"    # expert format: "mxfp4", "bf16" or "nvfp4"

    def expert_bytes(self) -> int:
        """Bytes of one expert record in the library: 3 matrices, MXFP4 (4
        bits + 8 bits per 32), bf16 (16 bits) or NVFP4 (4 bits + 8 bits per
        16, and a 16-byte trailer holding the three fp32 matrix scales)."""
        if self.weights == "bf16":
            return 3 * self.H * self.I * 2
        if self.weights == "nvfp4":
            return 3 * self.H * self.I * 9 // 16 + 16
        return 3 * self.H * self.I * 17 // 32


@dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    Ts: Sequence[int]                 # token batch sizes run on this shape
    steps: int = 1
    cache_slots: int = 0              # HBM LRU slots (global across layers)
    staging_slots: int = 0
    zipf_s: Optional[float] = None    # None: no router bias
    overlap: float = 0.0              # expected fraction kept step to step
    resize: tuple = ()                # ((before_step, new_slots), ...)
    preload_all: bool = False         # every expert resident before step 0
    prefill: bool = False
    notes: str = ""


WORKLOADS = {
    "tiny": Workload(
        "tiny", Shape(H=256, I=512, E=8, k=2), Ts=(4,), steps=1,
        cache_slots=8, staging_slots=8, preload_all=True,
        notes="T=4 tokens, all 8 experts resident, no router bias"),
    "a3b_decode": Workload(
        "a3b_decode", Shape(H=2048, I=512, E=256, k=8), Ts=(1, 4, 16),
        steps=512, cache_slots=64, staging_slots=128, zipf_s=1.1, overlap=0.6,
        notes="35B-A3B-shaped decode layer, 64-slot LRU, cold start"),
    "dsv4_decode": Workload(
        "dsv4_decode", Shape(H=4096, I=2048, E=256, k=6, layers=4, shared=True),
        Ts=(1, 32), steps=512, cache_slots=256, staging_slots=192,
        zipf_s=1.1, overlap=0.5,
        notes="DeepSeek-V4-Flash-shaped decode, 4 layers, global LRU of "
              "25% of experts per layer"),
    "dsv4_prefill": Workload(
        "dsv4_prefill", Shape(H=4096, I=2048, E=256, k=6, layers=4, shared=True),
        Ts=(4096,), steps=1, prefill=True,
        notes="T=4096 prefill, near-uniform routing, double-buffered layer "
              "uploads"),
    "glm_decode": Workload(
        "glm_decode", Shape(H=6144, I=2048, E=256, k=8, layers=8, shared=True),
        Ts=(1,), steps=1024, cache_slots=1228, staging_slots=8,
        zipf_s=1.2, overlap=0.55, resize=((512, 614),),
        notes="GLM-5.2-shaped decode, 8 layers, cache resized 60% -> 30% of "
              "experts before step 512"),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


# ----------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs are finite.  This is how synthetic activations are stored.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# -------------------------------------------------------------------- draws
def tokens(shape: Shape, layer: int, step: int, T: int, seed: int = 0) -> np.ndarray:
    """Activations x ~ N(0, 1) rounded to bf16; uint16 bits [T][H]."""
    g = _rng(seed, _X, layer, step, T)
    return f32_to_bf16_bits(g.standard_normal((T, shape.H), dtype=np.float32))


def router_weights(shape: Shape, layer: int, seed: int = 0) -> np.ndarray:
    """Router matrix W_r ~ N(0, 0.02^2), fp32 [H][E] (E contiguous)."""
    g = _rng(seed, _ROUTER, layer)
    return (g.standard_normal((shape.H, shape.E), dtype=np.float32) * np.float32(0.02))


@dataclass
class ExpertWeights:
    """Canonical MXFP4 expert: rows are output features, K contiguous.

    q*: packed E2M1 codes, element 2i in the low nibble of byte i.
    s*: E8M0 scale bytes, one per 32 consecutive K elements of a row.
    gate/up: [I][H/2] and [I][H/32]; down: [H][I/2] and [H][I/32].
    """

    qg: np.ndarray
    qu: np.ndarray
    qd: np.ndarray
    sg: np.ndarray
    su: np.ndarray
    sd: np.ndarray


def expert_weights(shape: Shape, layer: int, expert: int, seed: int = 0,
                   scale_lo: int = 119, scale_hi: int = 123) -> ExpertWeights:
    """Uniform 4-bit codes; scale exponents uniform over integers [-8, -4].

    ``expert = -1`` draws the layer's shared expert.
    """
    H, I = shape.H, shape.I
    g = _rng(seed, _SHARED if expert < 0 else _EXPERT, layer, max(expert, 0))
    q = g.integers(0, 256, size=3 * H * I // 2, dtype=np.uint8)
    s = g.integers(scale_lo, scale_hi + 1, size=3 * H * I // 32, dtype=np.uint8)
    n2, n32 = H * I // 2, H * I // 32
    return ExpertWeights(
        qg=q[:n2].reshape(I, H // 2), qu=q[n2:2 * n2].reshape(I, H // 2),
        qd=q[2 * n2:].reshape(H, I // 2),
        sg=s[:n32].reshape(I, H // 32), su=s[n32:2 * n32].reshape(I, H // 32),
        sd=s[2 * n32:].reshape(H, I // 32))


def zipf_sets(shape: Shape, layer: int, T: int, steps: int, s: float,
              overlap: float, seed: int = 0) -> np.ndarray:
    """Expert sets S[step][row] of size k drawn for one layer.

    Popularity: a per-layer random ranking pi of the experts, with
    p(pi[r]) proportional to (r+1)^-s.  Step 0 draws k experts without
    replacement from p.  Each later step keeps m ~ Binomial(k, overlap) of the
    row's previous set (a uniform subset) and draws the other k-m from p
    restricted to experts outside the previous set.  Returns int32
    [steps][T][k], each row sorted ascending.
    """
    E, k = shape.E, shape.k
    perm = _rng(seed, _PERM, layer).permutation(E)
    p = np.empty(E, dtype=np.float64)
    p[perm] = (np.arange(E, dtype=np.float64) + 1.0) ** (-s)
    p /= p.sum()
    out = np.empty((steps, T, k), dtype=np.int32)
    for r in range(T):
        g = _rng(seed, _TRACE, layer, T, r)
        prev = np.sort(g.choice(E, size=k, replace=False, p=p))
        out[0, r] = prev
        for st in range(1, steps):
            m = int(g.binomial(k, overlap))
            keep = g.choice(prev, size=m, replace=False) if m else np.empty(0, np.int64)
            mask = np.ones(E, dtype=bool)
            mask[prev] = False
            q = np.where(mask, p, 0.0)
            q /= q.sum()
            new = g.choice(E, size=k - m, replace=False, p=q)
            prev = np.sort(np.concatenate([keep, new]).astype(np.int64))
            out[st, r] = prev
    return out


@dataclass
class ExpertWeightsBF16:
    """Canonical bf16 expert (bit patterns): rows are output features, K
    contiguous.  wg, wu: [I][H]; wd: [H][I]."""
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray


def expert_weights_bf16(shape: Shape, layer: int, expert: int, seed: int = 0,
                        sigma: float = 2.0 ** -5) -> ExpertWeightsBF16:
    """Normal weights N(0, sigma^2) rounded to bf16 (sigma near the typical
    magnitude of the MXFP4 draws).  ``expert = -1`` draws the shared expert."""
    H, I = shape.H, shape.I
    g = _rng(seed, _SHARED if expert < 0 else _EXPERT, layer, max(expert, 0), 16)
    w = f32_to_bf16_bits((g.standard_normal(3 * H * I) * sigma).astype(np.float32))
    n = H * I
    return ExpertWeightsBF16(wg=w[:n].reshape(I, H), wu=w[n:2 * n].reshape(I, H),
                             wd=w[2 * n:].reshape(H, I))


@dataclass
class ExpertWeightsNV:
    """Canonical NVFP4 expert: E2M1 codes qg, qu [I][H/2], qd [H][I/2] (as
    MXFP4); E4M3 block-scale bytes sg, su [I][H/16], sd [H][I/16]; fp32
    matrix scales tg, tu, td."""
    qg: np.ndarray
    qu: np.ndarray
    qd: np.ndarray
    sg: np.ndarray
    su: np.ndarray
    sd: np.ndarray
    tg: np.float32
    tu: np.float32
    td: np.float32


# E4M3 block-scale codes drawn: exponent fields 3..6 (2^-4 .. 2^-1) with any
# mantissa, so blocks span 0.0625 .. 0.9375; with matrix scales in [0.25,
# 0.5) the weights sit near the MXFP4 draws' magnitude (up to 6 * 2^-4)
NV_SCALE_CODES = np.arange(3 << 3, 7 << 3, dtype=np.uint8)


def expert_weights_nvfp4(shape: Shape, layer: int, expert: int, seed: int = 0,
                         scale_codes: np.ndarray = NV_SCALE_CODES) -> ExpertWeightsNV:
    """Uniform 4-bit codes, E4M3 block scales uniform over scale_codes, fp32
    matrix scales uniform in [0.25, 0.5).  ``expert = -1`` draws the shared
    expert."""
    H, I = shape.H, shape.I
    g = _rng(seed, _SHARED if expert < 0 else _EXPERT, layer, max(expert, 0), 4)
    q = g.integers(0, 256, size=3 * H * I // 2, dtype=np.uint8)
    sc = g.choice(np.asarray(scale_codes, dtype=np.uint8), size=3 * H * I // 16)
    t = (0.25 + 0.25 * g.random(3)).astype(np.float32)
    n2, n16 = H * I // 2, H * I // 16
    return ExpertWeightsNV(
        qg=q[:n2].reshape(I, H // 2), qu=q[n2:2 * n2].reshape(I, H // 2),
        qd=q[2 * n2:].reshape(H, I // 2),
        sg=sc[:n16].reshape(I, H // 16), su=sc[n16:2 * n16].reshape(I, H // 16),
        sd=sc[2 * n16:].reshape(H, I // 16), tg=t[0], tu=t[1], td=t[2])


def expert_weights_of(shape: Shape, layer: int, expert: int, seed: int = 0):
    """The expert in the shape's weight format."""
    if shape.weights == "bf16":
        return expert_weights_bf16(shape, layer, expert, seed)
    if shape.weights == "nvfp4":
        return expert_weights_nvfp4(shape, layer, expert, seed)
    return expert_weights(shape, layer, expert, seed)


def popularity_order(shape: Shape, layer: int, seed: int = 0) -> np.ndarray:
    """The layer's experts from most to least popular under zipf_sets's
    ranking pi (the same permutation)."""
    return _rng(seed, _PERM, layer).permutation(shape.E).astype(np.int32)


def bias_from_sets(sets_step: np.ndarray, E: int) -> np.ndarray:
    """Router bias [T][E] fp32: BIAS_STRENGTH on each row's drawn set."""
    T = sets_step.shape[0]
    b = np.zeros((T, E), dtype=np.float32)
    b[np.arange(T)[:, None], sets_step] = BIAS_STRENGTH
    return b


# ------------------------------------------------- wide scale-exponent inputs
def expert_weights_scaled(shape: Shape, layer: int, expert: int, seed: int = 0,
                          gu_block_exp: Optional[np.ndarray] = None,
                          dn_row_exp: Optional[np.ndarray] = None,
                          jitter: int = 2) -> ExpertWeights:
    """MXFP4 expert whose E8M0 scale bytes span a wide range of exponents.

    Codes are uniform over the 16 values.  Gate and up: the scale byte of
    (row r, K block b) is gu_block_exp[b] + j; down: the scale byte of (row
    r, any K block) is dn_row_exp[r] + j; j uniform over [-jitter, jitter],
    the result clipped to [0, 250].  A part given as None keeps the usual
    bytes 119..123.  ``expert = -1`` draws the shared expert.
    """
    H, I = shape.H, shape.I
    base = expert_weights(shape, layer, expert, seed)
    g = _rng(seed, _SHARED if expert < 0 else _EXPERT, layer, max(expert, 0), 250)

    def spread(centre_of_block, rows, blocks):
        j = g.integers(-jitter, jitter + 1, size=(rows, blocks))
        return np.clip(centre_of_block + j, 0, 250).astype(np.uint8)

    sg, su, sd = base.sg, base.su, base.sd
    if gu_block_exp is not None:
        c = np.asarray(gu_block_exp, dtype=np.int64)[None, :]
        sg, su = spread(c, I, H // 32), spread(c, I, H // 32)
    if dn_row_exp is not None:
        sd = spread(np.asarray(dn_row_exp, dtype=np.int64)[:, None], H, I // 32)
    return ExpertWeights(qg=base.qg, qu=base.qu, qd=base.qd, sg=sg, su=su, sd=sd)


def tokens_block_scaled(shape: Shape, layer: int, step: int, T: int,
                        block_shift: np.ndarray, seed: int = 0) -> np.ndarray:
    """Activations x[t, 32 b + i] = N(0, 1) * 2^block_shift[b], rounded to
    bf16 (values below 2^-126 land on bf16's subnormal grid); uint16 [T][H]."""
    g = _rng(seed, _X, layer, step, T, 250)
    z = g.standard_normal((T, shape.H)).astype(np.float64)
    z *= np.exp2(np.repeat(np.asarray(block_shift, dtype=np.float64), 32))[None, :]
    return f32_to_bf16_bits(z.astype(np.float32))
