"""Seeded synthetic inputs for the A16W4 MoE layer.

Shared by the tests, the benchmark and the smoke check; it holds none of the
layer's arithmetic (no decode, routing, GEMM or quantization), only random
draws of the shapes and value distributions of the workloads:

* activations: float32 N(0, 1) cast to bf16 (torch's round-to-nearest-even
  cast), returned as uint16 bit patterns [T, H];
* router logits: float32 N(0, 1) [T, E], plus a +3.0 bias on a seeded set of
  8 "hot" experts for the skewed-routing variant;
* MXFP4 weights: uniform random bytes, so every e2m1 nibble is uniform over
  its 16 codes; w13 [E, 2I, H/2], w2 [E, H, I/2];
* e8m0 block scales: uniform integers in an inclusive range, one per 32
  elements along K: w13_scale [E, 2I, H/32], w2_scale [E, H, I/32].

Weight layouts follow create_weights of Mxfp4MoEMethod (vLLM mxfp4
quantization API page). Draw order per workload: hot set (if any), logits,
x, w13, w13_scale, w2, w2_scale, all from numpy Generator(PCG64(seed)).
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# The production expert-parallel shape validated on the MXFP4-to-int4 pull
# request page (Validation: model_dim, intermediate_dim, local experts, topk).
PROD = dict(H=3584, I=3072, E=112, topk=15)
# One rank's share of the same model under 8-way tensor parallelism instead:
# every expert (8 x 112), each with I / 8 = 384 (the same page's memory
# comparison runs TP8 without expert parallelism).
TP8 = dict(H=3584, I=384, E=896, topk=15)


@dataclass
class Spec:
    name: str
    T: int
    H: int
    I: int
    E: int
    topk: int
    seed: int
    scale_lo: int = 118
    scale_hi: int = 128
    hot: int = 0          # number of hot experts (skewed routing), 0 = none
    hot_bias: float = 3.0


@dataclass
class Workload:
    spec: Spec
    logits: np.ndarray            # float32 [T, E]
    x: np.ndarray                 # uint16 bf16 bits [T, H]
    w13: np.ndarray               # uint8 [E, 2I, H/2]
    w13_scale: np.ndarray         # uint8 [E, 2I, H/32]
    w2: np.ndarray                # uint8 [E, H, I/2]
    w2_scale: np.ndarray          # uint8 [E, H, I/32]
    hot_experts: Optional[np.ndarray] = field(default=None)


def specs():
    """Every named workload, keyed by name."""
    out = {
        "tiny": Spec("tiny", T=4, H=256, I=128, E=8, topk=2, seed=0,
                     scale_lo=120, scale_hi=130),
        "decode_t1": Spec("decode_t1", T=1, seed=1, **PROD),
        "prefill_t1024": Spec("prefill_t1024", T=1024, seed=3, **PROD),
        "int4_t16": Spec("int4_t16", T=16, seed=4, **PROD),
        "tp8_t1": Spec("tp8_t1", T=1, seed=5, **TP8),
    }
    for T in (4, 7, 16, 32):
        out[f"decode_t{T}"] = Spec(f"decode_t{T}", T=T, seed=100 + T, **PROD)
        out[f"skewed_t{T}"] = Spec(f"skewed_t{T}", T=T, seed=200 + T, hot=8, **PROD)
    return out


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns via torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _uniform_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def make(spec: Spec, T: Optional[int] = None, with_weights: bool = True) -> Workload:
    """Draw the workload. T overrides the token count (same seed)."""
    s = spec
    T = s.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(s.seed))
    hot = None
    if s.hot:
        hot = np.sort(rng.choice(s.E, size=s.hot, replace=False)).astype(np.int32)
    logits = rng.standard_normal((T, s.E), dtype=np.float32)
    if hot is not None:
        logits[:, hot] += np.float32(s.hot_bias)
    x = to_bf16_bits(rng.standard_normal((T, s.H), dtype=np.float32))
    if with_weights:
        w13 = _uniform_bytes(rng, (s.E, 2 * s.I, s.H // 2))
        w13_scale = rng.integers(s.scale_lo, s.scale_hi + 1, size=(s.E, 2 * s.I, s.H // 32),
                                 dtype=np.uint8)
        w2 = _uniform_bytes(rng, (s.E, s.H, s.I // 2))
        w2_scale = rng.integers(s.scale_lo, s.scale_hi + 1, size=(s.E, s.H, s.I // 32),
                                dtype=np.uint8)
    else:
        w13 = w13_scale = w2 = w2_scale = None
    return Workload(s, logits, x, w13, w13_scale, w2, w2_scale, hot)


def biases(E: int, H: int, I: int, seed: int, scale13: float = 64.0, scale2: float = 2.0 ** 19):
    """Expert biases as bf16 bit patterns (create_weights under has_bias):
    w13_bias [E, 2I] ~ N(0, scale13^2) and w2_bias [E, H] ~ N(0, scale2^2),
    drawn in that order from Generator(PCG64(seed)). The default scales
    are of the order of the GEMM outputs at the workloads' value
    distributions, so the biases change the results visibly."""
    rng = np.random.Generator(np.random.PCG64(seed))
    b13 = to_bf16_bits(rng.standard_normal((E, 2 * I), dtype=np.float32) * np.float32(scale13))
    b2 = to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(scale2))
    return b13, b2


def small(T, H, I, E, topk, seed, scale_lo=120, scale_hi=130, hot=0) -> Workload:
    """An ad-hoc small workload with the same distributions."""
    return make(Spec("adhoc", T=T, H=H, I=I, E=E, topk=topk, seed=seed,
                     scale_lo=scale_lo, scale_hi=scale_hi, hot=hot))
