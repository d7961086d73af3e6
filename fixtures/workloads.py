"""The five seeded synthetic workloads (shapes, value distributions, seeds).

Input recipes only: which generator draws which tensor with which seed.  No
layer arithmetic.  The residency choice of the partial-residency stack
(top experts by how often a Gumbel-top-k draw selects them) uses a library
arg-sort to count draws; it decides an input (the slot map), not an output.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import MXFP4, Q3K_Q4K, Q4K, Q5K, Q6K, Q8_0, TAG_SHARED_EXPERT, activations, expert_blob, logits_normal, logits_zipf, to_bf16_bits
from . import expert_blobs as _expert_blobs

SOFTMAX, SIGMOID = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: int
    H: int
    I: int
    E: int
    k: int
    T: int
    score: int = SOFTMAX
    renormalize: bool = True
    scale: float = 1.0
    x_bf16: bool = False
    zipf_s: float = 0.0          # 0: logits N(0,1); else Gumbel-perturbed Zipf(s)
    I_shared: int = 0            # 0: no shared expert; else a Q8_0 shared expert of this width
    weight_std: float = 0.02
    seed: int = 0
    layers: int = 1
    resident: int = 0            # 0: every expert resident (S = E); else S resident slots
    staging: int = 0             # extra slots for swaps
    count_tokens: int = 0        # tokens of the frequency count that picks the resident set
    tags: tuple = field(default_factory=tuple)


TINY = Workload("tiny Q8_0 MoE layer (H256 E8 k2 I128 T4)", Q8_0, 256, 128, 8, 2, 4)
QWEN3_DECODE_T1 = Workload("Qwen3-30B-A3B-shaped MoE layer, decode T=1", Q4K, 2048, 768, 128, 8, 1)
QWEN3_DECODE_T2 = Workload("Qwen3-30B-A3B-shaped MoE layer, decode T=2", Q4K, 2048, 768, 128, 8, 2)
QWEN3_PREFILL = Workload("Qwen3-30B-A3B-shaped MoE layer, prefill T=4096, Zipf(1.0) loads", Q4K, 2048, 768, 128, 8,
                         4096, x_bf16=True, zipf_s=1.0)
DSV3_DECODE_T2 = Workload("DeepSeek-V3-shaped MoE layer, decode T=2 (+shared Q8_0 expert)", Q4K, 7168, 2048, 256, 8,
                          2, score=SIGMOID, scale=2.5, I_shared=2048)
DSV3_DECODE_T4 = Workload("DeepSeek-V3-shaped MoE layer, decode T=4 (+shared Q8_0 expert)", Q4K, 7168, 2048, 256, 8,
                          4, score=SIGMOID, scale=2.5, I_shared=2048)
DSV3_STACK = Workload("58-layer DeepSeek-V3-shaped stack, 96 of 256 experts resident, decode T=2", Q4K, 7168, 2048,
                      256, 8, 2, score=SIGMOID, scale=2.5, I_shared=2048, zipf_s=1.1, layers=58, resident=96,
                      staging=8, count_tokens=10000)

# The same layers with MXFP4 routed experts (a card expert type of the engine;
# OCP MX encodings).  Weights: the same seeded normals, MXFP4-encoded.
QWEN3_MXFP4_DECODE_T2 = Workload("Qwen3-30B-A3B-shaped MoE layer, MXFP4 experts, decode T=2", MXFP4, 2048, 768, 128, 8,
                                 2)
DSV3_MXFP4_DECODE_T2 = Workload("DeepSeek-V3-shaped MoE layer, MXFP4 experts, decode T=2 (+shared Q8_0 expert)", MXFP4,
                                7168, 2048, 256, 8, 2, score=SIGMOID, scale=2.5, I_shared=2048)

# The DeepSeek-V3-shaped layer with the card experts of the engine's V4.1
# files: Q3_K gate and up, Q4_K down.
DSV3_Q3K_DECODE_T2 = Workload("DeepSeek-V3-shaped MoE layer, Q3_K gate/up + Q4_K down experts, decode T=2 "
                              "(+shared Q8_0 expert)", Q3K_Q4K, 7168, 2048, 256, 8, 2, score=SIGMOID, scale=2.5,
                              I_shared=2048)

QWEN3_Q3K_DECODE_T2 = Workload("Qwen3-30B-A3B-shaped MoE layer, Q3_K gate/up + Q4_K down experts, decode T=2",
                               Q3K_Q4K, 2048, 768, 128, 8, 2)

# Q5_K experts (a card expert type of the engine).
QWEN3_Q5K_DECODE_T2 = Workload("Qwen3-30B-A3B-shaped MoE layer, Q5_K experts, decode T=2", Q5K, 2048, 768, 128, 8, 2)
DSV3_Q5K_DECODE_T2 = Workload("DeepSeek-V3-shaped MoE layer, Q5_K experts, decode T=2 (+shared Q8_0 expert)", Q5K,
                              7168, 2048, 256, 8, 2, score=SIGMOID, scale=2.5, I_shared=2048)

# Q6_K experts (the top of the engine's card K-quant range).
QWEN3_Q6K_DECODE_T2 = Workload("Qwen3-30B-A3B-shaped MoE layer, Q6_K experts, decode T=2", Q6K, 2048, 768, 128, 8, 2)
DSV3_Q6K_DECODE_T2 = Workload("DeepSeek-V3-shaped MoE layer, Q6_K experts, decode T=2 (+shared Q8_0 expert)", Q6K,
                              7168, 2048, 256, 8, 2, score=SIGMOID, scale=2.5, I_shared=2048)

ALL = [TINY, QWEN3_DECODE_T1, QWEN3_DECODE_T2, QWEN3_PREFILL, DSV3_DECODE_T2, DSV3_DECODE_T4, DSV3_STACK,
       QWEN3_MXFP4_DECODE_T2, DSV3_MXFP4_DECODE_T2, DSV3_Q3K_DECODE_T2, QWEN3_Q5K_DECODE_T2, DSV3_Q5K_DECODE_T2,
       QWEN3_Q6K_DECODE_T2, DSV3_Q6K_DECODE_T2, QWEN3_Q3K_DECODE_T2]


def x_of(w: Workload, layer: int = 0, seed: int | None = None) -> np.ndarray:
    """Token activations: float32 [T, H], or bf16 bit patterns (uint16) for bf16 workloads."""
    x = activations(w.seed if seed is None else seed, layer, w.T, w.H)
    return to_bf16_bits(x) if w.x_bf16 else x


def x_f64(w: Workload, x: np.ndarray) -> np.ndarray:
    """The stored activations widened exactly to float64 (bf16 bits or float32)."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def logits_of(w: Workload, layer: int = 0, seed: int | None = None, T: int | None = None) -> np.ndarray:
    s = w.seed if seed is None else seed
    T = w.T if T is None else T
    if w.zipf_s:
        return logits_zipf(s, layer, T, w.E, w.zipf_s, perm_seed=w.seed)
    return logits_normal(s, layer, T, w.E)


def expert_blobs(w: Workload, experts=None, layer: int = 0) -> np.ndarray:
    """Canonical blobs [n, bytes] of the given experts (all E by default)."""
    experts = list(range(w.E)) if experts is None else list(experts)
    return _expert_blobs(w.fmt, w.seed, layer, experts, w.H, w.I, w.weight_std)


def shared_blob(w: Workload, layer: int = 0) -> np.ndarray | None:
    if not w.I_shared:
        return None
    return expert_blob(Q8_0, w.seed, layer, TAG_SHARED_EXPERT, w.H, w.I_shared, w.weight_std)


def frequency_resident_set(w: Workload, layer: int) -> np.ndarray:
    """Experts ranked by how often the layer's Zipf routing picks them over
    count_tokens draws (ties: lower id); the first `resident` are resident,
    slot r holding rank r."""
    lg = logits_zipf(w.seed + 1, layer, w.count_tokens, w.E, w.zipf_s, perm_seed=w.seed)
    top = np.argsort(-lg, axis=1, kind="stable")[:, :w.k]
    counts = np.bincount(top.ravel(), minlength=w.E)
    ranked = np.lexsort((np.arange(w.E), -counts))
    return ranked


def slot_map(w: Workload, layer: int = 0) -> tuple[np.ndarray, int]:
    """(slot_of_expert int32 [E], S) for the layer."""
    if not w.resident:
        return np.arange(w.E, dtype=np.int32), w.E
    ranked = frequency_resident_set(w, layer)
    soe = np.full(w.E, -1, dtype=np.int32)
    soe[ranked[:w.resident]] = np.arange(w.resident, dtype=np.int32)
    return soe, w.resident + w.staging
