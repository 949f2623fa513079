"""CPU oracle for the sparse MoE FFN layer forward pass (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it.

Sources (the web pages this layer is taken from):
  [P2] "Qwen2-MoE代码解析：MoE架构原理、工程实现与部署避坑指南"
       (www.jsqmd.com/news/1061813; a copy at www.ksqn.cn/news/44933)
  [P3] Qwen2-MoE code walk-through, www.mlqm.cn/news/48291
  [P4] MoE / "GPT-4 activates 2%" article, www.wmrh.cn/news/106769

What the layer computes, step by step (each function below cites its step):
  router      logits = X W_g (+ b); p = softmax(logits / tau); top-k of p;
              renormalise the k weights to sum to 1        [P2 §3.1; P3 §3.2 steps 1-2;
                                                            temperature tau: P4 §5.2]
  statistics  mean probability and selection frequency per expert, and
              E * their dot product                         [P2 §3.3]
  capacity    C = ceil(T/E) * k; pairs beyond C per expert dropped [P3 §2.2],
              or rerouted to the token's next-best expert with room
              (drop_tokens = False)                             [P2 §3.4]
  dispatch    group (token, slot) pairs by expert              [P2 §3.1 detail 3; P4 §2.2]
  experts     per expert Linear -> GELU -> Linear              [P3 §2.2; P4 §2.2]
  combine     weighted sum of the k expert outputs per token   [P2 §3.1 detail 2]

Readings taken where the pages are silent (each also listed in the design notes):
  * top-k order: probability descending, ties to the lower expert id;
  * GELU is the tanh form 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)));
  * capacity drop priority is (slot rank, token index); renormalisation happens
    over the top-k before any drop and is not redone; a dropped pair adds zero;
  * expert_capacity < 0 means dropless; 0 drops every pair;
  * the dispatch order is stable by (expert, token) -- unique, since a token
    picks an expert at most once (rerouting keeps that true);
  * rerouting (drop_tokens = False): the capacity cut runs first, unchanged;
    then the pairs it would drop, in the same (slot rank, token index)
    priority, each move to the best-ranked expert of their token outside its
    top-k that still has room and that the token does not already use; a
    pair finding none is dropped; a moved pair keeps its renormalised weight.

Every computation is float64 on the already-rounded inputs (bf16 bit patterns
are widened exactly).  Parity of this module is pinned by tests/test_oracle.py
(closed forms, brute force, invariants and the pages' printed examples).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "as_f64", "gelu_tanh", "router_logits", "softmax", "topk_route", "route",
    "router_stats", "RouterStats",
    "expert_capacity_formula", "expert_capacity_from_factor", "capacity_keep", "expert_ranking",
    "reroute_overflow", "dispatch", "expert_ffn",
    "combine", "moe_forward", "dense_bruteforce", "Routing", "Dispatch",
]


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen an input to float64. ``dtype == "bf16"``: ``a`` holds uint16 bfloat16
    bit patterns, which are the upper 16 bits of the float32 of the same value."""
    if dtype == "bf16":
        u = np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- router
def router_logits(X: np.ndarray, Wg: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    """Gate projection: the gate is a bias-free Linear(hidden, num_experts)
    [P2 §3.1, detail 1]; an optional per-expert logit bias is added (the
    per-domain routing bias of [P3 §6]).  X: [T, d], Wg: [d, E] -> [T, E]."""
    logits = X @ Wg
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits


def softmax(logits: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    """Softmax over the expert axis [P2 §3.1; P3 §3.2 step 2]; max-subtracted.
    With a router temperature the logits are divided by it first [P4 §5.2:
    the router softmax's temperature, 1.0 by default; above 1 the
    probabilities flatten, below 1 they sharpen]."""
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    m = z.max(axis=-1, keepdims=True)
    z = np.exp(z - m)
    return z / z.sum(axis=-1, keepdims=True)


@dataclass
class Routing:
    logits: np.ndarray   # [T, E] float64
    probs: np.ndarray    # [T, E] float64
    ids: np.ndarray      # [T, k] int64, slot 0 = most probable
    weights: np.ndarray  # [T, k] float64, renormalised, rows sum to 1
    margin: np.ndarray   # [T] float64, smallest adjacent gap among the top-(k+1) probs


def topk_route(probs: np.ndarray, k: int):
    """Top-k selection [P2 §3.1] and renormalisation [P2 §3.1, detail 2].

    The experts of a token are ordered by (probability descending, expert id
    ascending) -- the tie rule is a reading; the pages leave it to topk.  The
    first k are the selected experts, in slot order.  Their probabilities are
    divided by their sum so the k weights add up to 1.
    Also returns each token's margin: the smallest gap between adjacent entries
    of the sorted top-(k+1) probabilities (top-k when k = E), the measure of
    how close the selection or its slot order is to a tie."""
    T, E = probs.shape
    ids = np.empty((T, k), dtype=np.int64)
    w = np.empty((T, k), dtype=np.float64)
    margin = np.empty(T, dtype=np.float64)
    expert = np.arange(E)
    for t in range(T):
        order = np.lexsort((expert, -probs[t]))      # primary: -p, secondary: id
        sel = order[:k]
        ids[t] = sel
        top = probs[t, sel]
        w[t] = top / top.sum()
        upto = order[:min(k + 1, E)]
        pv = probs[t, upto]
        margin[t] = np.min(pv[:-1] - pv[1:]) if len(pv) > 1 else np.inf
    return ids, w, margin


def route(X: np.ndarray, Wg: np.ndarray, bias: Optional[np.ndarray], k: int,
          temperature: float = 1.0) -> Routing:
    """The router, all steps: gate Linear, softmax (at the given temperature),
    top-k, renormalise."""
    logits = router_logits(X, Wg, bias)
    probs = softmax(logits, temperature)
    ids, w, margin = topk_route(probs, k)
    return Routing(logits, probs, ids, w, margin)


@dataclass
class RouterStats:
    prob_mean: np.ndarray  # [E] mean router probability of each expert over the tokens
    sel_freq: np.ndarray   # [E] fraction of the tokens whose top-k holds the expert
    aux: float             # E * sum_e prob_mean[e] * sel_freq[e]


def router_stats(probs: np.ndarray, ids: np.ndarray, E: int) -> RouterStats:
    """The load-balancing statistics of one batch [P2 §3.3, its
    load_balancing_loss listing]: the mean over tokens of the router
    probabilities (the soft "tendency" of the gate), the mean over tokens of
    the 0/1 top-k selection mask (the hard "outcome"), and their dot product
    times the number of experts (balanced routing gives products near 1/E per
    expert, so the value is then near k).  probs: [T, E]; ids: [T, k]."""
    probs = np.asarray(probs, dtype=np.float64)
    T = probs.shape[0]
    mask = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for e in ids[t]:
            mask[t, int(e)] = 1.0
    prob_mean = probs.mean(axis=0) if T else np.zeros(E)
    sel_freq = mask.mean(axis=0) if T else np.zeros(E)
    return RouterStats(prob_mean, sel_freq, float(E * np.sum(prob_mean * sel_freq)))


# --------------------------------------------------------------------------- dispatch
def expert_capacity_formula(T: int, E: int, k: int) -> int:
    """expert_capacity = ceil(total_tokens / num_experts) * num_experts_per_tok [P3 §2.2]."""
    return int(math.ceil(T / E)) * k


def expert_capacity_from_factor(batch: int, seq_len: int, E: int, k: int, factor: float = 2.0) -> int:
    """The capacity-factor form of the expert capacity [P2 §3.4]: with
    tokens_per_expert the mean number of tokens per expert (T / E, T = batch *
    seq_len), C = int((tokens_per_expert * k * factor) // E), at most T; the
    factor defaults to 2.0.  Autoregressive decoding (seq_len == 1) uses
    min(512, 2 * batch) instead [P2 §5.2, its generate-mode fix].  (The page
    prints C = 128 for batch 1, seq_len 32768, which this reading of
    tokens_per_expert reproduces at 32 experts and k = 2.)"""
    if seq_len == 1:
        return min(512, 2 * batch)
    T = batch * seq_len
    tokens_per_expert = T / E
    c = int((tokens_per_expert * k * factor) // E)
    return min(c, T)


def capacity_keep(ids: np.ndarray, E: int, capacity: int) -> np.ndarray:
    """Which (token, slot) pairs an expert keeps [P2 §3.4: tokens over an
    expert's capacity are dropped].  Reading: each expert takes its pairs in
    (slot rank, token index) order and keeps the first ``capacity`` of them.
    ``capacity < 0`` keeps everything.  Returns a bool mask [T, k]."""
    T, k = ids.shape
    keep = np.ones((T, k), dtype=bool)
    if capacity < 0:
        return keep
    taken = np.zeros(E, dtype=np.int64)
    for s in range(k):              # slot rank first ...
        for t in range(T):          # ... then token index
            e = ids[t, s]
            if taken[e] < capacity:
                taken[e] += 1
            else:
                keep[t, s] = False
    return keep


def expert_ranking(probs: np.ndarray):
    """Each token's experts in preference order: probability descending, ties
    to the lower expert id (the order the top-k takes its first k from)
    [P2 §3.1].  Returns (order [T, E] int64, margin [T] float64), the margin
    being the smallest gap between adjacent probabilities along the whole
    order -- how close the order is to a tie anywhere (inf when E = 1)."""
    T, E = probs.shape
    order = np.empty((T, E), dtype=np.int64)
    margin = np.full(T, np.inf)
    expert = np.arange(E)
    for t in range(T):
        o = np.lexsort((expert, -probs[t]))
        order[t] = o
        if E > 1:
            pv = probs[t, o]
            margin[t] = np.min(pv[:-1] - pv[1:])
    return order, margin


def reroute_overflow(ids: np.ndarray, order: np.ndarray, keep: np.ndarray, E: int,
                     capacity: int):
    """Over-capacity pairs routed to the next-best expert instead of dropped
    [P2 §3.4: with drop_tokens = False, tokens over capacity go to a
    sub-optimal expert rather than being discarded].

    Reading (the page gives the rule in one sentence): the capacity cut of
    ``capacity_keep`` stands -- a pair it keeps is never moved.  The pairs it
    drops are then taken in the same (slot rank, token index) priority; each
    walks its token's order past the top-k (positions k, k+1, ..., E-1) and
    takes the first expert that has fewer than ``capacity`` pairs and that
    its token does not already use (an earlier slot may have moved there); if
    there is none the pair stays dropped.  Weights are not touched.

    ids, keep: [T, k]; order: [T, E] (``expert_ranking``).  Returns
    (assigned [T, k] int64, keep [T, k] bool): the expert each pair ends at
    (its own id when it is not moved) and whether it is computed."""
    T, k = ids.shape
    assigned = np.array(ids, dtype=np.int64, copy=True)
    keep = np.array(keep, dtype=bool, copy=True)
    if capacity < 0:
        return assigned, keep
    load = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for s in range(k):
            if keep[t, s]:
                load[ids[t, s]] += 1
    for s in range(k):              # the drop priority: slot rank first ...
        for t in range(T):          # ... then token index
            if keep[t, s]:
                continue
            used = set(int(assigned[t, j]) for j in range(k) if j != s)
            for pos in range(k, E):
                e = int(order[t, pos])
                if load[e] < capacity and e not in used:
                    assigned[t, s] = e
                    keep[t, s] = True
                    load[e] += 1
                    break
    return assigned, keep


@dataclass
class Dispatch:
    counts: np.ndarray    # [E] int64, routed pairs per expert (before any drop)
    keep: np.ndarray      # [T, k] bool
    offsets: np.ndarray   # [E+1] int64, exclusive scan of kept counts
    perm: np.ndarray      # [N] int64, pair id t*k+s of each expert-ordered row
    inv_perm: np.ndarray  # [T*k] int64, row of pair t*k+s, -1 if dropped
    assigned: np.ndarray  # [T, k] int64, expert each pair is computed by (= ids unless rerouted)


def dispatch(ids: np.ndarray, E: int, capacity: int = -1,
             reroute_order: Optional[np.ndarray] = None) -> Dispatch:
    """Group the kept (token, slot) pairs by expert [P2 §3.1 detail 3: tokens
    are regrouped by expert id with a sort; P4 §2.2: the dispatcher gathers each
    expert's token slices].  Rows are ordered by (expert, token); offsets are
    the exclusive scan of the kept counts (no padding).  With
    ``reroute_order`` (the tokens' ``expert_ranking``) and a capacity, the
    pairs over capacity are rerouted (``reroute_overflow``) rather than
    dropped, and grouped under the expert they move to."""
    T, k = ids.shape
    counts = np.bincount(ids.reshape(-1), minlength=E).astype(np.int64)
    keep = capacity_keep(ids, E, capacity)
    assigned = np.array(ids, dtype=np.int64, copy=True)
    if reroute_order is not None:
        assigned, keep = reroute_overflow(ids, reroute_order, keep, E, capacity)
    t_idx, s_idx = np.nonzero(keep)                      # kept pairs
    e_idx = assigned[t_idx, s_idx]
    order = np.lexsort((t_idx, e_idx))                   # sort by expert, then token
    perm = (t_idx * k + s_idx)[order]
    kept = np.bincount(e_idx, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    inv_perm = np.full(T * k, -1, dtype=np.int64)
    inv_perm[perm] = np.arange(len(perm))
    return Dispatch(counts, keep, offsets, perm, inv_perm, assigned)


# --------------------------------------------------------------------------- experts
def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def expert_ffn(x: np.ndarray, W1e: np.ndarray, W2e: np.ndarray) -> np.ndarray:
    """One expert: Linear -> GELU -> Linear, no biases [P3 §2.2: each expert is a
    standard FFN; P4 §2.2: Linear-GELU-Linear].  Weights follow nn.Linear's
    [out, in] layout: W1e [F, d], W2e [d, F].  x: [n, d] -> [n, d]."""
    h = gelu_tanh(x @ W1e.T)
    return h @ W2e.T


# --------------------------------------------------------------------------- combine
def combine(tokens: np.ndarray, d: int, weights: np.ndarray, keep: np.ndarray,
            y_pairs: dict) -> np.ndarray:
    """Weighted sum of each token's kept expert outputs [P2 §3.1 detail 2: the
    renormalised weights weight the experts' outputs].  ``y_pairs[(t, s)]`` is
    the expert output of pair (t, s).  Returns one row per entry of ``tokens``;
    a token with no kept pair gets zeros."""
    out = np.zeros((len(tokens), d), dtype=np.float64)
    for i, t in enumerate(tokens):
        for s in range(weights.shape[1]):
            if keep[t, s]:
                out[i] += weights[t, s] * y_pairs[(int(t), s)]
    return out


# --------------------------------------------------------------------------- layer
def moe_forward(X, Wg, bias, W1, W2, k: int, capacity: int = -1, dtype: str = "f32",
                tokens: Optional[Sequence[int]] = None, reroute: bool = False):
    """The whole layer [P3 §3.2 steps 1-5].  ``reroute``: over-capacity pairs
    move to the next-best expert with room instead of being dropped [P2 §3.4].

    Inputs are the raw arrays of a workload (bf16 bit patterns when ``dtype`` is
    "bf16").  Routing and dispatch always cover all T tokens (the capacity cut
    depends on every token); the expert FFNs and the combine are evaluated only
    for ``tokens`` (default: all).  Returns (out [len(tokens), d] float64,
    Routing, Dispatch)."""
    Xf = as_f64(X, dtype)
    T, d = Xf.shape
    E = Wg.shape[1]
    r = route(Xf, as_f64(Wg, dtype), bias, k)
    order = expert_ranking(r.probs)[0] if reroute else None
    disp = dispatch(r.ids, E, capacity, order)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    need = {}
    for t in toks:
        for s in range(k):
            if disp.keep[t, s]:
                need.setdefault(int(disp.assigned[t, s]), []).append((int(t), s))
    y_pairs = {}
    for e, pairs in sorted(need.items()):
        W1e = as_f64(W1[e], dtype)
        W2e = as_f64(W2[e], dtype)
        xs = Xf[[t for t, _ in pairs]]
        ys = expert_ffn(xs, W1e, W2e)
        for (t, s), y in zip(pairs, ys):
            y_pairs[(t, s)] = y
    out = combine(toks, d, r.weights, disp.keep, y_pairs)
    return out, r, disp


def dense_bruteforce(X, Wg, bias, W1, W2, k: int, capacity: int = -1, dtype: str = "f32"):
    """Dense reference for tiny shapes: run every expert on every token, then
    mask with M[t, e] = w[t, s] if expert e sits in kept slot s of token t,
    else 0, and sum over experts.  The top-k set is found by enumerating all
    k-subsets of experts and taking the one with the largest total probability
    (ties to the lexicographically smallest id set); slot order by
    (probability desc, id asc); the capacity cut by an explicit stable sort of
    all pairs on (expert, slot, token)."""
    from itertools import combinations
    Xf = as_f64(X, dtype)
    T, d = Xf.shape
    E = Wg.shape[1]
    logits = Xf @ as_f64(Wg, dtype)
    if bias is not None:
        logits = logits + np.asarray(bias, np.float64)
    p = np.exp(logits - logits.max(1, keepdims=True))
    p = p / p.sum(1, keepdims=True)
    ids = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        best, best_val = None, -1.0
        for sub in combinations(range(E), k):
            v = sum(p[t, j] for j in sub)
            if v > best_val + 1e-15:
                best, best_val = sub, v
        ordered = sorted(best, key=lambda j: (-p[t, j], j))
        ids[t] = ordered
    w = np.take_along_axis(p, ids, 1)
    w = w / w.sum(1, keepdims=True)
    keep = np.ones((T, k), dtype=bool)
    if capacity >= 0:
        pairs = sorted(((int(ids[t, s]), s, t) for t in range(T) for s in range(k)))
        seen = {}
        for e, s, t in pairs:
            seen[e] = seen.get(e, 0) + 1
            if seen[e] > capacity:
                keep[t, s] = False
    M = np.zeros((T, E))
    for t in range(T):
        for s in range(k):
            if keep[t, s]:
                M[t, ids[t, s]] = w[t, s]
    out = np.zeros((T, d))
    for e in range(E):
        Ye = expert_ffn(Xf, as_f64(W1[e], dtype), as_f64(W2[e], dtype))
        out += M[:, e:e + 1] * Ye
    return out, ids, w, keep
