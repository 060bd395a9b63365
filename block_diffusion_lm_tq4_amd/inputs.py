"""Seeded synthetic inputs shared by the tests, the oracle checks and the bench.

This module holds none of the layer's arithmetic: it only draws random numbers
and casts them to the input dtypes (fp32 weights, bf16 activations, router
outputs).  The bf16 cast of the activations uses torch's own conversion.

Workloads (shapes from the denoiser projections being served; the distributions
follow the model card, section *What "Config-I" means*, which reports the
format on Mamba-2, attention and 128-expert MoE tensors alike):

* ``linear_512x256``     W 512x256 ~ N(0, 0.02^2) seed 0, x 16x256 ~ N(0,1) seed 2
* ``dense_m16``          M=16 (one 16-token diffusion block), K=2688, N=8192
* ``moe_t16``            128 experts top-6, W1 1856x2688 / W2 2688x1856 per
                         expert, 16 tokens, router logits ~ N(0,1) seed 3
* ``moe_t1024_uniform``  64 sequences x 16 tokens = 1024 tokens, same layer
* ``moe_t1024_zipf``     same, expert popularity Zipf(s=1.1) via Gumbel top-6
* ``dense_m4096_t3``     M=4096, K=2688, N=8192, W = 0.02 * Student-t(nu=3)

Random numbers that the method itself draws (the rotation signs) are inputs
too: ``sign_bits()`` returns the 32 sign bits drawn from seed 1.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

N_EXPERTS = 128
TOPK = 6


@dataclass(frozen=True)
class DenseWorkload:
    name: str
    m: int
    k: int
    n: int
    weights: str = "gaussian"      # or "student_t3"


@dataclass(frozen=True)
class MoEWorkload:
    name: str
    t: int
    k: int = 2688
    n1: int = 1856
    n_experts: int = N_EXPERTS
    topk: int = TOPK
    routing: str = "uniform"       # or "zipf"


WORKLOADS = {
    "linear_512x256": DenseWorkload("linear_512x256", m=16, k=256, n=512),
    "dense_m16": DenseWorkload("dense_m16", m=16, k=2688, n=8192),
    "moe_t16": MoEWorkload("moe_t16", t=16),
    "moe_t1024_uniform": MoEWorkload("moe_t1024_uniform", t=1024),
    "moe_t1024_zipf": MoEWorkload("moe_t1024_zipf", t=1024, routing="zipf"),
    "dense_m4096_t3": DenseWorkload("dense_m4096_t3", m=4096, k=2688, n=8192,
                                    weights="student_t3"),
}


def sign_bits(seed: int = 1) -> int:
    """32 rotation sign bits: bit i set means s_i = -1."""
    bits = np.random.default_rng(seed).integers(0, 2, 32)
    return int(sum(int(b) << i for i, b in enumerate(bits)))


def weights(n: int, k: int, kind: str = "gaussian", seed=0,
            scale: float = 0.02) -> np.ndarray:
    """fp32 weights [n, k]: scale * N(0,1) or scale * Student-t(3)."""
    rng = np.random.default_rng(seed)
    if kind == "gaussian":
        w = rng.standard_normal((n, k))
    elif kind == "student_t3":
        w = rng.standard_t(3, size=(n, k))
    else:
        raise ValueError(kind)
    return (scale * w).astype(np.float32)


def expert_weights(e: int, which: int, n1: int = 1856, k: int = 2688) -> np.ndarray:
    """Expert e's up (which=1, [n1, k]) or down (which=2, [k, n1]) fp32 weights.

    Each matrix has its own seed sequence [0, e, which], so any expert can be
    regenerated alone.
    """
    shape = (n1, k) if which == 1 else (k, n1)
    rng = np.random.default_rng(np.random.SeedSequence([0, e, which]))
    return (0.02 * rng.standard_normal(shape)).astype(np.float32)


def activations_bf16(m: int, k: int, seed: int = 2) -> np.ndarray:
    """x ~ N(0,1) cast fp32 -> bf16 (torch's round-to-nearest-even); uint16 bits."""
    import torch
    x = np.random.default_rng(seed).standard_normal((m, k)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    return xb.view(torch.int16).numpy().view(np.uint16).copy()


def router_logits(t: int, n_experts: int = N_EXPERTS, routing: str = "uniform",
                  seed: int = 3, zipf_s: float = 1.1) -> np.ndarray:
    """Router logits [t, E] (fp64).

    uniform: i.i.d. N(0,1).  zipf: log p_e + Gumbel(0,1) with p_e proportional
    to (e+1)^-s, so the top-k of each row is a Plackett-Luce draw without
    replacement whose first pick follows Zipf(s) exactly (expert 0 hottest).
    """
    rng = np.random.default_rng(seed)
    if routing == "uniform":
        return rng.standard_normal((t, n_experts))
    if routing == "zipf":
        p = (np.arange(1, n_experts + 1, dtype=np.float64)) ** (-zipf_s)
        p /= p.sum()
        return np.log(p)[None, :] + rng.gumbel(size=(t, n_experts))
    raise ValueError(routing)


def route(logits: np.ndarray, topk: int = TOPK):
    """Router outside the layer: softmax over all experts, then the top-k.

    Ids are the k largest logits (ties to the lower expert id); gates are the
    softmax probabilities of those ids, not renormalized.  Returns
    (ids int32 [t, k], gates fp32 [t, k]).
    """
    lg = np.asarray(logits, dtype=np.float64)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ids = np.argsort(-lg, axis=1, kind="stable")[:, :topk].astype(np.int32)
    gates = np.take_along_axis(p, ids, axis=1).astype(np.float32)
    return ids, gates


def moe_routing(wl: MoEWorkload, seed: int = 3):
    """(ids, gates) for an MoE workload."""
    return route(router_logits(wl.t, wl.n_experts, wl.routing, seed), wl.topk)
