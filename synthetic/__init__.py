"""Seeded synthetic inputs for the W4A16 decode workloads.

This module is the only thing the oracle side and the HIP side share.  It
draws random numbers and rounds them to bf16; it holds none of the product's
arithmetic (no unpacking, no dequantization, no sums).

Generator: numpy's PCG64 seeded through ``SeedSequence([seed, stream, *tag])``,
one independent stream per tensor role (``STREAM``) and per tag (layer index,
expert index, ...), so every tensor is reproducible on its own.

Value distributions (the workload descriptions of the decode shapes):
  * codes: uniform in 0..15, packed 8 per uint32 with the first code in the
    lowest nibble.  Eight independent uniform nibbles are exactly one uniform
    32-bit word, so a packed row is drawn directly as uniform uint32 words.
  * scale ~ U(0.002, 0.02), rounded to bf16 (nearest-even, torch's rounding).
  * bias = -8*scale + N(0, 0.001) in fp32 from the bf16 scale, then bf16
    (``bias="noise"``), or exactly -8*scale (``bias="exact"``, the LM-head
    distribution; -8*s is exact in bf16).
  * x ~ N(0, 1) rounded to bf16, rows independent.
  * routed ids: for each token, ``top_k`` distinct experts drawn uniformly
    without replacement.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

STREAM = {"qw": 11, "scales": 12, "biases": 13, "x": 14, "ids": 15, "codes": 16}


def rng(seed: int, role: str, *tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, STREAM[role], *tag])))


def bf16_bits(a) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16) using torch's nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (torch widening cast)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()


@dataclass
class QWeights:
    qw: np.ndarray       # uint32 [..., N, K/8]
    scales: np.ndarray   # uint16 (bf16 bits) [..., N, K/G]
    biases: np.ndarray   # uint16 (bf16 bits) [..., N, K/G]
    N: int
    K: int
    group: int

    @property
    def nbytes(self) -> int:
        return self.qw.nbytes + self.scales.nbytes + self.biases.nbytes


def quantized_weights(N: int, K: int, group: int = 64, seed: int = 0, tag=(), bias: str = "noise",
                      lead=()) -> QWeights:
    """Random packed weights of shape lead + [N, K]; tag selects independent streams."""
    tag = tuple(tag)
    shape_w = tuple(lead) + (N, K // 8)
    shape_g = tuple(lead) + (N, K // group)
    qw = rng(seed, "qw", *tag).integers(0, 2**32, size=shape_w, dtype=np.uint32)
    s = rng(seed, "scales", *tag).uniform(0.002, 0.02, size=shape_g).astype(np.float32)
    s_bits = bf16_bits(s)
    s_val = bf16_values(s_bits)
    if bias == "noise":
        noise = rng(seed, "biases", *tag).normal(0.0, 0.001, size=shape_g).astype(np.float32)
        b = (np.float32(-8.0) * s_val + noise).astype(np.float32)
    elif bias == "exact":
        b = (np.float32(-8.0) * s_val).astype(np.float32)
    else:
        raise ValueError(bias)
    return QWeights(qw, s_bits, bf16_bits(b), N, K, group)


def activations(M: int, K: int, seed: int = 0, tag=()) -> np.ndarray:
    """x ~ N(0,1) as bf16 bits, shape [M, K]."""
    x = rng(seed, "x", *tuple(tag)).standard_normal(size=(M, K)).astype(np.float32)
    return bf16_bits(x)


def expert_ids(M: int, top_k: int, E: int, seed: int = 0, tag=()) -> np.ndarray:
    """int32 [M, top_k]: per token, top_k distinct experts uniformly without replacement."""
    g = rng(seed, "ids", *tuple(tag))
    return np.stack([g.choice(E, size=top_k, replace=False) for _ in range(M)]).astype(np.int32)


def random_codes(N: int, K: int, seed: int = 0, tag=()) -> np.ndarray:
    """Unpacked uniform codes (uint8 [N, K], values 0..15) for layout tests."""
    return rng(seed, "codes", *tuple(tag)).integers(0, 16, size=(N, K), dtype=np.uint8)


# ---- the decode workloads ---------------------------------------------------------

GROUP = 64
HIDDEN = 2560

# Decode-shaped projections of a 2560-hidden transformer (N <- K).
PROJECTIONS = {
    "q": (2560, 2560),
    "k": (512, 2560),
    "v": (512, 2560),
    "o": (2560, 2560),
    "gate_up": (20480, 2560),
    "down": (2560, 10240),
}
# One decode layer applies q, k, v, o, gate_up, down in that order.
LAYER_ORDER = ("q", "k", "v", "o", "gate_up", "down")
VERIFY_M = (2, 3, 5)

TINY = dict(M=1, N=256, K=512)
LM_HEAD = dict(N=262144, K=2560, M=(1, 3))
SQUARE = dict(N=16384, K=16384, M=(1, 4, 8))
MOE = dict(E=64, N=6144, K=2048, top_k=8, M=(1, 8))

