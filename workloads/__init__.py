"""Seeded synthetic inputs for the sparse MoE FFN layer.

This module holds no step of the layer's arithmetic: it only draws the
inputs (hidden states, gate weight, optional per-expert logit bias, expert
weights) for the five workloads and rounds them to bfloat16.  Both the CPU
oracle (tests) and the HIP path (tests, bench) consume exactly these arrays.

Recipe (one reading, applied to both sides):
  * ``rng = numpy.random.default_rng(seed)``; hidden states ``X ~ N(0, 1)``
    drawn first as float32, then the gate weight ``W_g[d, E]`` Xavier-uniform
    with gain 1 (bound ``sqrt(6 / (d + E))``, the gate init named in
    "Qwen2-MoE代码解析" (jsqmd.com/news/1061813) §3.1, detail 1), then the bias.
  * Expert ``e``'s ``W1[e]`` ([F, d], nn.Linear [out, in]) and ``W2[e]``
    ([d, F]) come from child streams ``SeedSequence([seed, 1, e])`` and
    ``SeedSequence([seed, 2, e])`` as ``0.02 * N(0, 1)`` so that experts can be
    drawn in parallel threads and the largest workload never needs an fp32
    copy of all weights at once.
  * Decode: step ``i``'s hidden states come from ``SeedSequence([seed, 1000+i])``.
  * bf16 workloads: every float tensor except the bias is rounded to bfloat16
    with round-to-nearest-even and handed over as its uint16 bit pattern.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "MoEInputs", "generate", "decode_step_hidden",
           "f32_to_bf16_bits", "bf16_bits_to_f32", "capacity_of"]


@dataclass(frozen=True)
class Workload:
    name: str
    T: int           # tokens (batch * seq flattened)
    d: int           # hidden size
    E: int           # number of experts
    k: int           # experts per token
    F: int           # expert FFN inner size
    dtype: str       # "f32" or "bf16"
    seed: int
    bias: str = "none"        # "none" | "zipf" | "normal"
    capacity: bool = False    # expert_capacity = ceil(T/E)*k when True
    steps: int = 1            # decode: number of fresh-hidden-state steps
    note: str = ""


# The five workloads: sizes, init distributions and seeds as stated with the
# layer's measurement plan.
WORKLOADS = {
    "tiny": Workload("tiny", T=64, d=128, E=8, k=2, F=256, dtype="f32", seed=0,
                     note="tiny fp32 layer"),
    "prefill": Workload("prefill", T=8192, d=2048, E=32, k=2, F=5632, dtype="bf16", seed=1,
                        note="batch 4 x seq 2048 prefill"),
    "decode": Workload("decode", T=8, d=3584, E=64, k=2, F=2560, dtype="bf16", seed=2, steps=100,
                       note="batch 8, one token each, 100 fresh steps"),
    "skewed": Workload("skewed", T=16384, d=4096, E=64, k=2, F=14336, dtype="bf16", seed=3,
                       bias="zipf", note="large prefill, Zipf-pmf logit bias"),
    "capacity": Workload("capacity", T=32768, d=2048, E=32, k=4, F=1408, dtype="bf16", seed=4,
                         bias="normal", capacity=True,
                         note="batch 16 x seq 2048, capacity-limited"),
}


def capacity_of(w: Workload) -> int:
    """expert_capacity for a workload: ceil(T/E)*k when capacity-limited, else -1 (dropless)."""
    if not w.capacity:
        return -1
    return -(-w.T // w.E) * w.k


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns.

    Finite inputs only (the generators never produce inf/nan)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = u + (np.uint32(0x7FFF) + lsb)
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class MoEInputs:
    """One workload's tensors.  For dtype "bf16" X, Wg, W1, W2 are uint16 bf16
    bit patterns; for "f32" they are float32.  ``bias`` is float32 or None."""
    workload: Workload
    X: np.ndarray                 # [T, d]
    Wg: np.ndarray                # [d, E]
    bias: Optional[np.ndarray]    # [E] or None
    W1: np.ndarray                # [E, F, d]
    W2: np.ndarray                # [E, d, F]
    expert_capacity: int = -1
    extra: dict = field(default_factory=dict)


def _round(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def _zipf_pmf_log_bias(E: int, s: float = 1.1, scale: float = 1.5) -> np.ndarray:
    """Per-expert logit bias 1.5 * log of the Zipf(s) pmf at rank e+1 (expert 0 is rank 1)."""
    ranks = np.arange(1, E + 1, dtype=np.float64)
    pmf = ranks ** (-s)
    pmf /= pmf.sum()
    return (scale * np.log(pmf)).astype(np.float32)


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(w: Workload | str, *, T: Optional[int] = None, experts: Optional[list] = None,
             threads: Optional[int] = None) -> MoEInputs:
    """Draw a workload's inputs.

    ``T`` overrides the token count (the hidden states are then the first T
    rows of the same stream, so a smaller T is a prefix of the full workload).
    ``experts`` restricts which experts' weights are drawn (others are left as
    zeros); draws are per expert, so the drawn ones are identical either way.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    T_full = w.T
    T_use = T_full if T is None else int(T)
    rng = np.random.default_rng(w.seed)
    if w.steps > 1:
        X = decode_step_hidden(w, 0)
    else:
        X = rng.standard_normal((T_full, w.d), dtype=np.float32)[:T_use]
    a = math.sqrt(6.0 / (w.d + w.E))
    Wg = rng.uniform(-a, a, size=(w.d, w.E)).astype(np.float32)
    if w.bias == "zipf":
        bias = _zipf_pmf_log_bias(w.E)
    elif w.bias == "normal":
        bias = rng.normal(0.0, 0.5, size=w.E).astype(np.float32)
    else:
        bias = None

    wdt = np.uint16 if w.dtype == "bf16" else np.float32
    W1 = np.zeros((w.E, w.F, w.d), dtype=wdt)
    W2 = np.zeros((w.E, w.d, w.F), dtype=wdt)
    todo = list(range(w.E)) if experts is None else sorted(set(int(e) for e in experts))

    def draw(e: int) -> None:
        g1 = np.random.default_rng(np.random.SeedSequence([w.seed, 1, e]))
        W1[e] = _round(g1.standard_normal((w.F, w.d), dtype=np.float32) * np.float32(0.02), w.dtype)
        g2 = np.random.default_rng(np.random.SeedSequence([w.seed, 2, e]))
        W2[e] = _round(g2.standard_normal((w.d, w.F), dtype=np.float32) * np.float32(0.02), w.dtype)

    nt = threads or _threads()
    if nt > 1 and len(todo) > 1:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(draw, todo))
    else:
        for e in todo:
            draw(e)
    return MoEInputs(w, _round(X, w.dtype), _round(Wg, w.dtype), bias, W1, W2,
                     expert_capacity=capacity_of(w) if T is None else
                     (-(-T_use // w.E) * w.k if w.capacity else -1))


def decode_step_hidden(w: Workload | str, step: int) -> np.ndarray:
    """Fresh hidden states [T, d] (float32, not yet rounded) for decode step ``step``."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    g = np.random.default_rng(np.random.SeedSequence([w.seed, 1000 + step]))
    return g.standard_normal((w.T, w.d), dtype=np.float32)


def decode_step_inputs(w: Workload | str, step: int) -> np.ndarray:
    """Decode step's hidden states rounded to the workload dtype."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return _round(decode_step_hidden(w, step), w.dtype)


def random_case(seed: int, T: int, d: int, E: int, k: int, F: int, dtype: str = "f32",
                capacity: int = -1, bias_scale: float = 0.0, x_scale: float = 1.0,
                w_scale: float = 0.02) -> MoEInputs:
    """A small seeded case of arbitrary shape (same distributions as the workloads)."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, d), dtype=np.float32) * np.float32(x_scale)
    a = math.sqrt(6.0 / (d + E))
    Wg = rng.uniform(-a, a, size=(d, E)).astype(np.float32)
    bias = (rng.normal(0.0, bias_scale, size=E).astype(np.float32) if bias_scale > 0 else None)
    W1 = rng.standard_normal((E, F, d), dtype=np.float32) * np.float32(w_scale)
    W2 = rng.standard_normal((E, d, F), dtype=np.float32) * np.float32(w_scale)
    wl = Workload(f"random{seed}", T=T, d=d, E=E, k=k, F=F, dtype=dtype, seed=seed)
    return MoEInputs(wl, _round(X, dtype), _round(Wg, dtype), bias, _round(W1, dtype), _round(W2, dtype),
                     expert_capacity=capacity)
