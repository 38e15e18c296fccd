"""Seeded synthetic inputs for the quantized latent-MoE expert stage.

This module draws random numbers and lays them into buffers; it performs none
of the expert stage's arithmetic (no dequantization, no quantization of the
activations, no products).  Both the HIP path and the CPU oracle read what it
produces, so it is the one piece of code the two sides share.

Workload recipe (all draws from one ``numpy.random.default_rng(seed)`` stream,
in this order):

1. ``x``: T x L float32 standard normal (latent activations before they are
   rounded to q8_1; the rounding is done by the library or the oracle).
2. Router logits: T x E float64 standard normal.
3. Skewed workloads only: a random permutation gives every expert a rank
   1..E; popularity p_e is proportional to rank_e ** -s (Zipf, s = 1.1) and
   ln(p_e) is added to every token's logits.  ``n_masked`` experts with the
   lowest popularity get logit -inf, so no token routes to them.
4. Softmax over E, top-k (ties go to the lower expert index), the k weights
   renormalised to sum to one in float64 and stored as float32.
5. Gate/up weights, Q3_K blocks [E][2F][L/256] x 110 bytes: every byte
   uniform random (so the 2-bit low codes, the high-bit mask and the packed
   6-bit sub-block scales are uniform), then the fp16 super-block scale at
   bytes 108..109 drawn from U(0.005, 0.015).
6. Down weights, IQ4_NL blocks [E][L][F/32] x 18 bytes: the 16 code bytes
   uniform random (both 4-bit indices uniform), the fp16 block scale at bytes
   0..1 drawn from U(0.005, 0.015).

The Q3_K, IQ4_NL and q8_1 block layouts are ggml's (GGUF) formats; the pages
on the latent expert stage name them without restating them.

Latent D / U projection workloads (``DenseWorkload``; the dense projections
into and out of the latent rows, Q8_0 weights), one ``default_rng(seed)``
stream, in this order:

1. ``x``: T x H float32 standard normal (hidden rows that D reads once they
   are rounded to q8_1).
2. D weights, Q8_0 blocks [L][H/32] x 34 bytes: int8 codes uniform in
   -127..127, fp16 block scale at bytes 0..1 drawn from U(0.5, 1.5) * 2^-12
   (so a projected value has a standard deviation of order one).
3. ``z``: T x L float32 standard normal (latent rows that U reads, standing
   in for the expert stage's output, once rounded to q8_1).
4. U weights, Q8_0 blocks [H][L/32] x 34 bytes, drawn as in 2.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

Q3K_BLOCK_BYTES = 110      # 256 weights: hmask[32], qs[64], scales[12], fp16 d
Q3K_BLOCK_VALUES = 256
IQ4NL_BLOCK_BYTES = 18     # 32 weights: fp16 d, qs[16]
IQ4NL_BLOCK_VALUES = 32
Q8_1_BLOCK_BYTES = 36      # 32 values: fp16 d, fp16 s, int8 qs[32]
Q8_1_BLOCK_VALUES = 32
Q8_0_BLOCK_BYTES = 34      # 32 weights: fp16 d, int8 qs[32]
Q8_0_BLOCK_VALUES = 32


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and routing recipe of one expert-stage call."""
    name: str
    T: int          # tokens
    L: int          # latent dimension (multiple of 256)
    F: int          # expert FFN width (multiple of 32)
    E: int          # experts
    k: int          # experts per token
    zipf_s: float = 0.0   # 0 = no popularity skew
    n_masked: int = 0     # least-popular experts that receive no tokens
    seed: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the stage is specified on.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", T=32, L=256, F=512, E=8, k=2),
    "decode": Workload("decode", T=4, L=1024, F=2048, E=128, k=8),
    "mid_prefill": Workload("mid_prefill", T=512, L=1024, F=2048, E=64, k=8),
    "prefill_5k": Workload("prefill_5k", T=5268, L=1024, F=2048, E=128, k=8, zipf_s=1.1),
    "prefill_21k": Workload("prefill_21k", T=21000, L=1024, F=2048, E=128, k=8, zipf_s=1.1,
                            n_masked=8),
}


@dataclasses.dataclass
class Inputs:
    wl: Workload
    x: np.ndarray            # float32 [T, L]
    router_idx: np.ndarray   # int32 [T, k]
    router_w: np.ndarray     # float32 [T, k]
    gateup_q3k: np.ndarray   # uint8 [E, 2F, L/256, 110]
    down_iq4nl: np.ndarray   # uint8 [E, L, F/32, 18]
    router_logits: Optional[np.ndarray] = None  # float32 [T, E]: the logits of step 3, before the softmax


def _route(rng: np.random.Generator, wl: Workload) -> tuple:
    logits = rng.standard_normal((wl.T, wl.E))
    if wl.zipf_s > 0.0:
        rank = rng.permutation(wl.E) + 1
        pop = rank.astype(np.float64) ** (-wl.zipf_s)
        pop /= pop.sum()
        logits = logits + np.log(pop)[None, :]
        if wl.n_masked > 0:
            masked = np.argsort(pop, kind="stable")[: wl.n_masked]
            logits[:, masked] = -np.inf
    raw = logits.astype(np.float32)
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    # stable sort of -p: equal probabilities keep ascending expert order
    order = np.argsort(-p, axis=1, kind="stable")[:, : wl.k]
    top = np.take_along_axis(p, order, axis=1)
    top = top / top.sum(axis=1, keepdims=True)
    return order.astype(np.int32), top.astype(np.float32), raw


def make_routing_draws(wl: Workload, n: int) -> list:
    """n more draws of the workload's activations and routing (steps 1-4 of
    the recipe, x then logits, skew and top-k), each from a stream of its own
    (seed [seed, 8 + i]); the weights are not redrawn.  A timing that rotates
    among them finds no call's experts left in cache by the call before.
    Returns a list of (x float32 [T, L], router_idx int32 [T, k], router_w
    float32 [T, k])."""
    out = []
    for i in range(n):
        rng = np.random.default_rng([wl.seed, 8 + i])
        x = rng.standard_normal((wl.T, wl.L), dtype=np.float32)
        idx, w, _ = _route(rng, wl)
        out.append((x, idx, w))
    return out


def random_q3k(rng: np.random.Generator, shape: tuple) -> np.ndarray:
    """Uniform random Q3_K blocks with fp16 scales d ~ U(0.005, 0.015)."""
    b = rng.integers(0, 256, size=shape + (Q3K_BLOCK_BYTES,), dtype=np.uint8)
    d = rng.uniform(0.005, 0.015, size=shape).astype(np.float16)
    b[..., 108:110] = d.view(np.uint8).reshape(shape + (2,))
    return b


def random_iq4nl(rng: np.random.Generator, shape: tuple) -> np.ndarray:
    """Uniform random IQ4_NL blocks with fp16 scales d ~ U(0.005, 0.015)."""
    b = rng.integers(0, 256, size=shape + (IQ4NL_BLOCK_BYTES,), dtype=np.uint8)
    d = rng.uniform(0.005, 0.015, size=shape).astype(np.float16)
    b[..., 0:2] = d.view(np.uint8).reshape(shape + (2,))
    return b


def make_inputs(wl: Workload) -> Inputs:
    if wl.L % 256 or wl.F % 32 or not (1 <= wl.k <= wl.E) or wl.T < 0:
        raise ValueError(f"unsupported workload shape {wl}")
    rng = np.random.default_rng(wl.seed)
    x = rng.standard_normal((wl.T, wl.L), dtype=np.float32)
    idx, w, logits = _route(rng, wl)
    gu = random_q3k(rng, (wl.E, 2 * wl.F, wl.L // 256))
    dn = random_iq4nl(rng, (wl.E, wl.L, wl.F // 32))
    return Inputs(wl, x, idx, w, gu, dn, logits)


def make_gateup_q4_0(wl: Workload) -> np.ndarray:
    """The workload's gate/up weights as Q4_0 blocks, uint8 [E, 2F, L/32, 18]
    (nibble bytes uniform, d ~ U(0.5, 1.5) * 2^-8), from a stream of their own
    (seed [seed, 4]), so make_inputs' draws are unchanged and nothing is drawn
    unless they are asked for."""
    return random_q4_0(np.random.default_rng([wl.seed, 4]), (wl.E, 2 * wl.F, wl.L // 32))


def group_sizes(router_idx: np.ndarray, E: int) -> np.ndarray:
    """Tokens routed to each expert (ids outside [0, E) ignored)."""
    ids = router_idx.reshape(-1)
    ids = ids[(ids >= 0) & (ids < E)]
    return np.bincount(ids, minlength=E)


def workload(name: str, seed: Optional[int] = None) -> Workload:
    wl = WORKLOADS[name]
    return wl if seed is None else wl.replace(seed=seed)


@dataclasses.dataclass(frozen=True)
class DenseWorkload:
    """Shapes of the latent layer's dense projections: D maps hidden rows
    (width H) to latent rows (width L), U maps latent rows back to width H."""
    name: str
    T: int          # tokens
    H: int          # hidden width (multiple of 32)
    L: int          # latent width (multiple of 32)
    seed: int = 0

    def replace(self, **kw) -> "DenseWorkload":
        return dataclasses.replace(self, **kw)


DENSE_WORKLOADS: Dict[str, DenseWorkload] = {
    "du_tiny": DenseWorkload("du_tiny", T=37, H=512, L=256),
    "du_decode": DenseWorkload("du_decode", T=4, H=4096, L=1024),
    "du_prefill_5k": DenseWorkload("du_prefill_5k", T=5268, H=4096, L=1024),
}


@dataclasses.dataclass
class DenseInputs:
    wl: DenseWorkload
    x: np.ndarray        # float32 [T, H]
    d_q8_0: np.ndarray   # uint8 [L, H/32, 34]
    z: np.ndarray        # float32 [T, L]
    u_q8_0: np.ndarray   # uint8 [H, L/32, 34]
    d_q4_0: np.ndarray = None  # uint8 [L, H/32, 18]: D's weights as Q4_0 blocks (drawn after the rest)
    u_q4_0: np.ndarray = None  # uint8 [H, L/32, 18]


def random_q8_0(rng: np.random.Generator, shape: tuple) -> np.ndarray:
    """Q8_0 blocks with codes uniform in -127..127 and fp16 scales
    d ~ U(0.5, 1.5) * 2^-12."""
    b = np.empty(shape + (Q8_0_BLOCK_BYTES,), np.uint8)
    b[..., 2:] = rng.integers(-127, 128, size=shape + (32,), dtype=np.int8).view(np.uint8)
    d = (rng.uniform(0.5, 1.5, size=shape) * 2.0 ** -12).astype(np.float16)
    b[..., 0:2] = d.view(np.uint8).reshape(shape + (2,))
    return b


def random_q4_0(rng: np.random.Generator, shape: tuple) -> np.ndarray:
    """Q4_0 blocks (18 bytes: fp16 d, 16 bytes of nibbles) with the nibble
    bytes uniform and d ~ U(0.5, 1.5) * 2^-8."""
    b = np.empty(shape + (18,), np.uint8)
    b[..., 2:] = rng.integers(0, 256, size=shape + (16,), dtype=np.uint8)
    d = (rng.uniform(0.5, 1.5, size=shape) * 2.0 ** -8).astype(np.float16)
    b[..., 0:2] = d.view(np.uint8).reshape(shape + (2,))
    return b


def make_dense_inputs(wl: DenseWorkload) -> DenseInputs:
    if wl.H % 32 or wl.L % 32 or wl.H <= 0 or wl.L <= 0 or wl.T < 0:
        raise ValueError(f"unsupported dense workload shape {wl}")
    rng = np.random.default_rng(wl.seed)
    x = rng.standard_normal((wl.T, wl.H), dtype=np.float32)
    dw = random_q8_0(rng, (wl.L, wl.H // 32))
    z = rng.standard_normal((wl.T, wl.L), dtype=np.float32)
    uw = random_q8_0(rng, (wl.H, wl.L // 32))
    dw4 = random_q4_0(rng, (wl.L, wl.H // 32))
    uw4 = random_q4_0(rng, (wl.H, wl.L // 32))
    return DenseInputs(wl, x, dw, z, uw, dw4, uw4)
