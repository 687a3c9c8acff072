"""Seeded synthetic inputs for the routed MoE layer.

Shared by the tests, the benchmark and the oracle's timing leg. This module
holds none of the method's arithmetic: it only draws float32 arrays (router
logits, activations, expert weights) from NumPy's PCG64 generator. Quantising
them is done separately by each side (the oracle's own quantiser, or the
library's quantise kernel), and the parity tests check the two agree.

Workloads (the pages run DeepSeek-V4.1-Flash and GLM-5.2 decode; those shapes
and weights are not available, so these synthetic shapes stand in for them):

  tiny     T=16,   H=512,  I=256,  E=8,   k=2, all local, MXFP4 weights
  decode   T in {1, 8, 32, 128}, H=7168, I=2048, E=256, k=8, experts 0..31
           local (one GPU's share of an expert-parallel layer), MXFP4 weights
  full     T=256,  H=6144, I=1536, E=128, k=8, logits + per-expert bias N(0,1)
  prefill  T=16384, H=2048, I=1408, E=64, k=6, Zipf(1.1) popularity,
           MXFP8 weights, transposed copy of h
  shared   decode at T=32 plus one always-on shared expert

Distributions: logits ~ N(0,1); x ~ N(0,1); W ~ N(0, 0.02^2) (std 0.02). The
prefill logits are ln p_e + Gumbel(0,1) with p_e proportional to (e+1)^-1.1:
top-k of such logits samples k experts without replacement in proportion to
p (the Gumbel-top-k identity), so expert e has popularity rank e+1.

Every array has its own stream, keyed by (seed, stream tag, index), so one
expert's weights can be drawn without drawing the others. Weights depend on
the workload's seed only (the decode sweep and the shared-expert workload use
one set of routed experts); logits and x also depend on T and on a routing
variant, so a benchmark can cycle through several routing draws over the same
weights.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

W_STD = 0.02

_TAG = {"logits": 1, "bias": 2, "x": 3, "w1": 4, "w2": 5, "sw1": 6, "sw2": 7}


@dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    I: int
    E: int            # total experts seen by the router
    k: int
    e0: int           # first local expert
    n_local: int      # local experts
    w_fmt: str        # "e2m1" (MXFP4) or "e4m3" (MXFP8)
    logit_kind: str   # "normal", "normal+bias", "zipf"
    shared: bool = False
    transpose: bool = False
    seed: int = 1000

    @property
    def G(self) -> int:
        return self.n_local + (1 if self.shared else 0)

    @property
    def R_max(self) -> int:
        return self.T * self.k + (self.T if self.shared else 0)


def config(name: str, T: int | None = None) -> Config:
    """The named workload; `T` overrides the token count (decode sweeps)."""
    if name == "tiny":
        c = Config("tiny", 16, 512, 256, 8, 2, 0, 8, "e2m1", "normal", seed=1000)
    elif name == "decode":
        T = 128 if T is None else T
        c = Config("decode", T, 7168, 2048, 256, 8, 0, 32, "e2m1", "normal", seed=1001)
    elif name == "full":
        c = Config("full", 256, 6144, 1536, 128, 8, 0, 128, "e2m1", "normal+bias", seed=1002)
    elif name == "prefill":
        c = Config("prefill", 16384, 2048, 1408, 64, 6, 0, 64, "e4m3", "zipf",
                   transpose=True, seed=1003)
    elif name == "shared":
        c = Config("shared", 32, 7168, 2048, 256, 8, 0, 32, "e2m1", "normal",
                   shared=True, seed=1001)       # the decode workload's routed experts
    else:
        raise KeyError(name)
    if T is not None and name != "decode":
        c = replace(c, T=T)
    return c


def _rng(seed: int, tag: str, *index: int) -> np.random.Generator:
    key = [seed, _TAG[tag], *index]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def logits(c: Config, variant: int = 0) -> np.ndarray:
    """Router logits, float32 [T, E]. `variant` selects one of several routing
    draws over the same weights (new logits and x, same experts)."""
    g = _rng(c.seed, "logits", c.T, variant)
    if c.logit_kind == "zipf":
        p = (np.arange(1, c.E + 1, dtype=np.float64)) ** -1.1
        p /= p.sum()
        return (np.log(p)[None, :] + g.gumbel(size=(c.T, c.E))).astype(np.float32)
    lg = g.standard_normal((c.T, c.E), dtype=np.float32)
    if c.logit_kind == "normal+bias":
        b = _rng(c.seed, "bias", 0).standard_normal(c.E, dtype=np.float32)
        lg = (lg + b[None, :]).astype(np.float32)
    return lg


def x(c: Config, variant: int = 0) -> np.ndarray:
    """Activations, float32 [T, H]."""
    return _rng(c.seed, "x", c.T, variant).standard_normal((c.T, c.H), dtype=np.float32)


def w1(c: Config, g: int) -> np.ndarray:
    """W1 of local expert g, float32 [2I, H]: rows [0, I) gate, [I, 2I) up."""
    return _rng(c.seed, "w1", g).standard_normal((2 * c.I, c.H), dtype=np.float32) * np.float32(W_STD)


def w2(c: Config, g: int) -> np.ndarray:
    """W2 of local expert g, float32 [H, I]."""
    return _rng(c.seed, "w2", g).standard_normal((c.H, c.I), dtype=np.float32) * np.float32(W_STD)


def shared_w1(c: Config) -> np.ndarray:
    return _rng(c.seed, "sw1", 0).standard_normal((2 * c.I, c.H), dtype=np.float32) * np.float32(W_STD)


def shared_w2(c: Config) -> np.ndarray:
    return _rng(c.seed, "sw2", 0).standard_normal((c.H, c.I), dtype=np.float32) * np.float32(W_STD)
