"""Seeded synthetic inputs and the workload shapes.

This module draws random numbers and nothing else: it holds none of the
dispatch/combine arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it.  bf16 activations are produced by rounding fp32 normal
draws with torch's CPU conversion and are handed out as uint16 bit patterns.

Shapes follow the pages' MoE layers: hidden size 7168, top-8 of 256 experts
(DeepSeek-V3) or 384 experts (Kimi-K2), 128 tokens per rank for decode and
4096 for prefill ("Enabling trillion-parameter models on AWS EFA", Evaluation;
"Lower Latency and Higher Throughput with Multi-Node DeepSeek Deployment",
Expert Parallelism).  Real router logits and activations need trained weights;
standard-normal draws stand in for them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens held by the sending rank
    H: int          # hidden size
    E: int          # routed experts
    k: int          # experts per token
    N: int          # expert-parallel ranks (virtual, all in this GPU's HBM)
    C: int          # receive rows per rank; 0 = packed regions sized by counts
    score: int      # SCORE_SIGMOID or SCORE_SOFTMAX
    payload: str    # "bf16" or "fp8"
    expert: str     # "identity" or "scale" (per-expert scalar stand-in)
    zipf: float     # 0 = no popularity bias, else the Zipf exponent
    seed: int
    sources: int = 1  # source ranks dispatching at once (T tokens each)

    @property
    def L(self) -> int:
        return self.E // self.N

    @property
    def tokens(self) -> int:
        return self.T * self.sources

    @property
    def rows(self) -> int:
        return self.N * self.C if self.C > 0 else self.tokens * self.k


def _cap(T: int, k: int, E: int, N: int) -> int:
    # one sender's tight bound: a token lands at most min(k, E/N) times on a rank
    return T * min(k, E // N)


WORKLOADS = {
    "tiny": Workload("tiny", 16, 256, 8, 2, 2, _cap(16, 2, 8, 2), SCORE_SOFTMAX,
                     "bf16", "identity", 0.0, 1000),
    "dsv3_decode": Workload("dsv3_decode", 128, 7168, 256, 8, 32, _cap(128, 8, 256, 32),
                            SCORE_SIGMOID, "bf16", "scale", 0.0, 1001),
    "kimi_k2_decode": Workload("kimi_k2_decode", 128, 7168, 384, 8, 16, _cap(128, 8, 384, 16),
                               SCORE_SIGMOID, "bf16", "scale", 0.0, 1002),
    "skewed_prefill": Workload("skewed_prefill", 4096, 7168, 256, 8, 32, 0, SCORE_SIGMOID,
                               "bf16", "scale", 1.2, 1003),
    "fp8_payload": Workload("fp8_payload", 512, 7168, 256, 8, 32, _cap(512, 8, 256, 32),
                            SCORE_SIGMOID, "fp8", "scale", 0.0, 1004),
    # all 32 ranks of a DeepSeek-V3 EP32 decode step dispatching at once
    # (128 tokens each); packed receive regions sized by the exchanged counts
    "dsv3_world": Workload("dsv3_world", 128, 7168, 256, 8, 32, 0, SCORE_SIGMOID, "bf16",
                           "scale", 0.0, 1005, sources=32),
}
def with_tokens(w: Workload, T: int) -> Workload:
    """The workload at T tokens per source; a fixed capacity is resized with
    them (the same one-sender bound), packed regions stay packed."""
    if T < 1:
        raise ValueError(f"tokens must be positive, got {T}")
    return dataclasses.replace(w, T=T, C=_cap(T, w.k, w.E, w.N) if w.C > 0 else 0)


WORKLOAD_ORDER = ["tiny", "dsv3_decode", "kimi_k2_decode", "skewed_prefill", "fp8_payload"]


@dataclasses.dataclass
class Inputs:
    logits: np.ndarray            # float32 [T, E]
    bias: Optional[np.ndarray]    # float32 [E] or None
    x_bits: np.ndarray            # uint16 [T, H] (bf16 bit patterns)
    alpha: np.ndarray             # float32 [E] expert stand-in scalars


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with torch's CPU conversion; return the bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def generate(T: int, H: int, E: int, seed: int, expert: str = "scale",
             zipf: float = 0.0) -> Inputs:
    """Fixed draw order from PCG64(seed): logits ~ N(0,1) [T,E]; x ~ N(0,1)
    [T,H] then bf16; alpha ~ U[0.5,1.5) [E]; for a Zipf bias, a permutation of
    the experts giving each its popularity rank r (1 = hottest) and the bias
    -zipf * ln(r)."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    x = rng.standard_normal((T, H), dtype=np.float32)
    alpha = rng.uniform(0.5, 1.5, size=E).astype(np.float32)
    if expert == "identity":
        alpha = np.ones(E, np.float32)
    bias = None
    if zipf > 0.0:
        popularity_rank = rng.permutation(E).astype(np.float64) + 1.0
        bias = (-zipf * np.log(popularity_rank)).astype(np.float32)
    return Inputs(logits=logits, bias=bias, x_bits=bf16_bits_from_f32(x), alpha=alpha)


def generate_for(w: Workload) -> Inputs:
    return generate(w.tokens, w.H, w.E, w.seed, w.expert, w.zipf)


def random_ids(T: int, k: int, E: int, seed: int, distinct: bool = True,
               hot: Optional[int] = None) -> np.ndarray:
    """Expert ids [T,k] int32 drawn directly (for layout cases that need no
    router).  distinct: k different experts per token; hot: every token's slot
    0 goes to expert `hot` (a fully skewed column)."""
    rng = np.random.default_rng(seed)
    if distinct:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k))
    else:
        ids = rng.integers(0, E, size=(T, k))
    ids = np.asarray(ids, np.int32).reshape(T, k)
    if hot is not None and T:
        ids[:, 0] = hot
    return ids


def random_weights(T: int, k: int, seed: int) -> np.ndarray:
    """Positive fp32 weights [T,k] (not normalised)."""
    rng = np.random.default_rng(seed)
    return rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
