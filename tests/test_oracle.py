"""Pins of the CPU oracle against facts that do not come from the oracle itself:
values printed on the source pages (tests/golden), closed forms, brute force on
tiny inputs, library routines for the textbook special cases, and invariants.
CPU only."""
import json
import math
import os
from itertools import combinations

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _case(seed, T=24, d=32, E=6, k=2, F=48, capacity=-1, bias_scale=0.0, x_scale=1.0):
    return workloads.random_case(seed, T, d, E, k, F, "f32", capacity, bias_scale, x_scale, w_scale=0.2)


# ----------------------------------------------------------------- page examples
def test_renorm_printed_example():
    g = _golden("renorm_example.json")
    p = np.array([[0.3, 0.2, 0.15, 0.15, 0.1, 0.1]])
    ids, w, _ = oracle.topk_route(p, 2)
    assert ids.tolist() == [[0, 1]]
    assert p[0, ids[0]].sum() == pytest.approx(g["sum_before"], abs=1e-15)
    assert w[0].tolist() == pytest.approx(g["renormalised"], abs=1e-15)


def test_worked_count_prefill_shape():
    """Batch 4 x seq 2048 with k=2 routes 16384 pairs; with k=1, 8192."""
    g = _golden("worked_count.json")
    inp = workloads.generate("prefill", experts=[])
    assert inp.X.shape[0] == g["batch"] * g["seq_len"] == g["tokens"]
    X = oracle.as_f64(inp.X, "bf16")
    Wg = oracle.as_f64(inp.Wg, "bf16")
    for k, key in ((2, "pairs_k2"), (1, "pairs_k1")):
        r = oracle.route(X, Wg, None, k)
        disp = oracle.dispatch(r.ids, inp.Wg.shape[1])
        assert int(disp.counts.sum()) == g[key]
        assert len(disp.perm) == g[key]


def test_activation_rate_two_of_64():
    g = _golden("activation_rate.json")
    case = _case(7, T=40, d=16, E=g["num_experts"], k=g["num_experts_per_tok"])
    r = oracle.route(oracle.as_f64(case.X, "f32"), oracle.as_f64(case.Wg, "f32"), None, 2)
    for t in range(r.ids.shape[0]):
        assert len(set(r.ids[t].tolist())) == 2
    frac = r.ids.shape[1] / g["num_experts"]
    assert round(100 * frac, 1) == g["active_fraction_rounded_pct"]


def test_capacity_formula_golden():
    for c in _golden("capacity_formula.json")["cases"]:
        assert oracle.expert_capacity_formula(c["T"], c["E"], c["k"]) == c["C"]
    assert workloads.capacity_of(workloads.WORKLOADS["capacity"]) == 4096


def test_capacity_factor_golden():
    """The capacity-factor formula and the generate-mode override: the page's
    printed capacity (128 at batch 1, seq_len 32768) and hand computations."""
    for c in _golden("capacity_factor_example.json")["cases"]:
        assert oracle.expert_capacity_from_factor(c["batch"], c["seq_len"], c["E"], c["k"], c["factor"]) == c["C"]
    # never above the number of tokens; grows with the factor
    assert oracle.expert_capacity_from_factor(1, 8, 2, 2, 100.0) == 8
    assert oracle.expert_capacity_from_factor(16, 1024, 8, 2, 1.0) < oracle.expert_capacity_from_factor(16, 1024, 8, 2, 3.0)


def test_capacity_hand_case():
    g = _golden("capacity_hand_case.json")
    ids = np.array(g["ids"])
    d = oracle.dispatch(ids, g["E"], g["capacity"])
    assert d.keep.tolist() == g["keep"]
    assert d.counts.tolist() == g["counts"]
    assert d.offsets.tolist() == g["offsets"]
    assert d.perm.tolist() == g["perm"]
    assert d.inv_perm.tolist() == g["inv_perm"]


# ----------------------------------------------------------------- GELU
def test_gelu_matches_torch_tanh_gelu():
    x = np.linspace(-8, 8, 2001)
    ref = torch.nn.functional.gelu(torch.tensor(x, dtype=torch.float64), approximate="tanh").numpy()
    assert np.max(np.abs(oracle.gelu_tanh(x) - ref)) < 1e-14


def test_gelu_closed_forms():
    x = np.linspace(-5, 5, 101)
    g = oracle.gelu_tanh
    assert g(np.array([0.0]))[0] == 0.0
    # 0.5x(1+tanh(u(x))) with u odd  =>  g(x) - g(-x) = x
    assert np.max(np.abs(g(x) - g(-x) - x)) < 1e-14
    assert abs(g(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(g(np.array([-40.0]))[0]) < 1e-12
    # the tanh form stays within 1e-3 of the exact erf GELU
    exact = 0.5 * x * (1 + np.vectorize(math.erf)(x / math.sqrt(2)))
    assert np.max(np.abs(g(x) - exact)) < 1e-3


# ----------------------------------------------------------------- router
def test_router_logits_match_bias_free_linear():
    case = _case(1, E=5, bias_scale=0.7)
    X = oracle.as_f64(case.X, "f32")
    Wg = oracle.as_f64(case.Wg, "f32")
    lin = torch.nn.Linear(X.shape[1], Wg.shape[1], bias=True).double()
    with torch.no_grad():
        lin.weight.copy_(torch.tensor(Wg.T))
        lin.bias.copy_(torch.tensor(case.bias, dtype=torch.float64))
        ref = lin(torch.tensor(X)).numpy()
    assert np.max(np.abs(oracle.router_logits(X, Wg, case.bias) - ref)) < 1e-12
    p = oracle.softmax(ref)
    ref_p = torch.softmax(torch.tensor(ref), dim=-1).numpy()
    assert np.max(np.abs(p - ref_p)) < 1e-15


@pytest.mark.parametrize("seed,E,k", [(0, 4, 1), (1, 6, 2), (2, 8, 3), (3, 5, 5), (4, 7, 4)])
def test_topk_is_best_subset(seed, E, k):
    case = _case(seed, T=20, d=12, E=E, k=k, bias_scale=0.3)
    r = oracle.route(oracle.as_f64(case.X, "f32"), oracle.as_f64(case.Wg, "f32"), case.bias, k)
    for t in range(r.ids.shape[0]):
        best = max(combinations(range(E), k), key=lambda sub: sum(r.probs[t, j] for j in sub))
        assert set(r.ids[t].tolist()) == set(best)
        # slots in descending probability
        assert np.all(np.diff(r.probs[t, r.ids[t]]) <= 0)


def test_weights_closed_form_and_sum():
    case = _case(5, T=50, E=8, k=3, bias_scale=1.0)
    r = oracle.route(oracle.as_f64(case.X, "f32"), oracle.as_f64(case.Wg, "f32"), case.bias, 3)
    assert np.max(np.abs(r.weights.sum(1) - 1.0)) < 1e-12
    # the renormalised weights equal a softmax restricted to the selected logits
    sel = np.take_along_axis(r.logits, r.ids, 1)
    ref = np.exp(sel - sel.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    assert np.max(np.abs(r.weights - ref)) < 1e-14


def test_router_shift_invariance_and_huge_bias():
    case = _case(6, T=30, E=8, k=2)
    X = oracle.as_f64(case.X, "f32")
    Wg = oracle.as_f64(case.Wg, "f32")
    r0 = oracle.route(X, Wg, None, 2)
    r1 = oracle.route(X, Wg, np.full(8, 3.25), 2)
    assert (r0.ids == r1.ids).all()
    assert np.max(np.abs(r0.weights - r1.weights)) < 1e-14
    b = np.zeros(8)
    b[5] = 1e3
    r2 = oracle.route(X, Wg, b, 2)
    assert (r2.ids[:, 0] == 5).all()


def test_router_relabelling_equivariance():
    case = _case(8, T=30, E=7, k=3)
    X = oracle.as_f64(case.X, "f32")
    Wg = oracle.as_f64(case.Wg, "f32")
    pi = np.array([3, 0, 6, 1, 5, 2, 4])
    r = oracle.route(X, Wg, None, 3)
    rp = oracle.route(X, Wg[:, pi], None, 3)
    # new expert j is old expert pi[j]
    assert (pi[rp.ids] == r.ids).all()


def test_temperature_closed_forms():
    """Router temperature: softmax(l / tau).  Two experts: the logistic
    function of (l0 - l1) / tau; the selection does not depend on tau (> 0);
    the renormalised top-2 weight is the logistic function of the top-2 gap
    over tau; huge tau flattens to 1/E, tiny tau gives a one-hot."""
    l = np.array([[1.5, -0.5], [0.2, 0.7]])
    for tau in (0.5, 1.0, 2.0, 3.0):
        p = oracle.softmax(l, tau)
        for t in range(2):
            want0 = 1.0 / (1.0 + math.exp((l[t, 1] - l[t, 0]) / tau))
            assert abs(p[t, 0] - want0) < 1e-15 and abs(p[t, 1] - (1 - want0)) < 1e-15
    case = _case(12, T=40, E=8, k=2, bias_scale=0.5)
    X, Wg = oracle.as_f64(case.X, "f32"), oracle.as_f64(case.Wg, "f32")
    r1 = oracle.route(X, Wg, case.bias, 2)
    for tau in (0.25, 0.5, 2.0, 7.0):
        rt = oracle.route(X, Wg, case.bias, 2, temperature=tau)
        assert (rt.ids == r1.ids).all()
        top = np.take_along_axis(rt.logits, rt.ids, 1)
        want = 1.0 / (1.0 + np.exp((top[:, 1] - top[:, 0]) / tau))
        assert np.max(np.abs(rt.weights[:, 0] - want)) < 1e-14
    flat = oracle.softmax(r1.logits, 1e12)
    assert np.max(np.abs(flat - 1.0 / 8)) < 1e-10
    sharp = oracle.softmax(r1.logits, 1e-4)
    assert (np.argmax(sharp, 1) == r1.ids[:, 0]).all() and np.max(np.abs(sharp.max(1) - 1.0)) < 1e-12


def test_router_stats_properties():
    """Load-balancing statistics: the mean probabilities sum to 1, the
    selection frequencies to k; uniform logits give 1/E each and a value of
    exactly k; a balanced selection gives k whatever the probabilities; a
    collapse onto one expert at k = 1 with sharp probabilities gives E (the
    worst value)."""
    case = _case(13, T=64, E=8, k=3, bias_scale=1.0)
    X, Wg = oracle.as_f64(case.X, "f32"), oracle.as_f64(case.Wg, "f32")
    r = oracle.route(X, Wg, case.bias, 3)
    st = oracle.router_stats(r.probs, r.ids, 8)
    assert abs(st.prob_mean.sum() - 1.0) < 1e-12 and abs(st.sel_freq.sum() - 3.0) < 1e-12
    assert (st.sel_freq >= 0).all() and (st.sel_freq <= 1).all()
    # uniform logits
    ru = oracle.route(X, np.zeros_like(Wg), None, 3)
    su = oracle.router_stats(ru.probs, ru.ids, 8)
    assert np.max(np.abs(su.prob_mean - 1.0 / 8)) < 1e-15 and abs(su.aux - 3.0) < 1e-12
    # a balanced selection: 8 tokens, k = 2, each expert picked twice
    ids = np.array([[e, (e + 1) % 4] for e in range(4)] * 2)
    probs = np.random.default_rng(0).dirichlet(np.ones(4), size=8)
    assert abs(oracle.router_stats(probs, ids, 4).aux - 2.0) < 1e-12
    # collapse
    logits = np.tile(np.array([5.0, 0.0, -1.0, 0.5, 0.2]), (10, 1))
    rc_probs = oracle.softmax(logits, 1e-3)
    sc = oracle.router_stats(rc_probs, np.zeros((10, 1), dtype=np.int64), 5)
    assert abs(sc.aux - 5.0) < 1e-12
    # the value from the frequencies and probabilities of a hand case:
    # T = 2, E = 2, k = 1; token 0 picks expert 0 with p0 = s(1), token 1
    # picks expert 1 with p1 = s(2) (s the logistic function)
    s1, s2 = 1 / (1 + math.exp(-1.0)), 1 / (1 + math.exp(-2.0))
    hp = np.array([[s1, 1 - s1], [1 - s2, s2]])
    hs = oracle.router_stats(hp, np.array([[0], [1]]), 2)
    assert np.allclose(hs.prob_mean, [(s1 + 1 - s2) / 2, (1 - s1 + s2) / 2], atol=1e-15)
    assert np.allclose(hs.sel_freq, [0.5, 0.5]) and abs(hs.aux - 1.0) < 1e-15


def test_topk_ties_go_to_lower_id_and_margin():
    p = np.array([[0.25, 0.25, 0.25, 0.25],
                  [0.1, 0.4, 0.1, 0.4],
                  [0.5, 0.3, 0.15, 0.05]])
    ids, w, margin = oracle.topk_route(p, 2)
    assert ids.tolist() == [[0, 1], [1, 3], [0, 1]]
    assert margin[0] == 0.0 and margin[1] == 0.0
    assert margin[2] == pytest.approx(0.15)
    ids4, _, m4 = oracle.topk_route(p, 4)
    assert ids4[2].tolist() == [0, 1, 2, 3]
    assert m4[2] == pytest.approx(0.1)


# ----------------------------------------------------------------- dispatch
@pytest.mark.parametrize("seed,E,k,cap", [(0, 4, 1, -1), (1, 6, 2, -1), (2, 8, 3, 5), (3, 3, 2, 4), (4, 6, 2, 0)])
def test_dispatch_invariants(seed, E, k, cap):
    rng = np.random.default_rng(seed)
    T = 37
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    d = oracle.dispatch(ids, E, cap)
    assert int(d.counts.sum()) == T * k
    kept = np.bincount(ids[d.keep], minlength=E)
    if cap >= 0:
        assert (kept == np.minimum(d.counts, cap)).all()
    else:
        assert d.keep.all()
    assert (np.diff(d.offsets) == kept).all() and d.offsets[0] == 0
    N = int(d.offsets[-1])
    assert len(d.perm) == N == int(d.keep.sum())
    # bijection between kept pairs and rows
    assert (d.inv_perm[d.perm] == np.arange(N)).all()
    assert ((d.inv_perm >= 0) == d.keep.reshape(-1)).all()
    # rows strictly increasing in (expert, token)
    t = d.perm // k
    s = d.perm % k
    e = ids[t, s]
    key = e * T + t
    assert (np.diff(key) > 0).all()
    for j in range(E):
        assert (e[d.offsets[j]:d.offsets[j + 1]] == j).all()


def test_capacity_bruteforce_and_limits():
    rng = np.random.default_rng(11)
    T, E, k = 41, 5, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    for cap in (0, 1, 7, 20, 200):
        keep = oracle.capacity_keep(ids, E, cap)
        # brute force: sort all pairs on (expert, slot, token), cut each expert at cap
        pairs = sorted((int(ids[t, s]), s, t) for t in range(T) for s in range(k))
        ref = np.zeros((T, k), dtype=bool)
        n = {}
        for e, s, t in pairs:
            n[e] = n.get(e, 0) + 1
            ref[t, s] = n[e] <= cap
        assert (keep == ref).all()
    full = oracle.dispatch(ids, E, -1)
    big = oracle.dispatch(ids, E, int(full.counts.max()))
    assert (full.perm == big.perm).all() and (full.inv_perm == big.inv_perm).all()


# ----------------------------------------------------------------- rerouting
def _random_order_case(rng, T, E, k):
    """Random preferences: a strict order per token; ids are its first k."""
    order = np.stack([rng.permutation(E) for _ in range(T)])
    return order, order[:, :k].copy()


def test_reroute_hand_case():
    g = _golden("reroute_hand_case.json")
    logits = np.array(g["logits"], dtype=np.float64)
    p = oracle.softmax(logits)
    ids, _, _ = oracle.topk_route(p, g["k"])
    order, _ = oracle.expert_ranking(p)
    assert ids.tolist() == g["ids"] and order.tolist() == g["preference_order"]
    for c in g["cases"]:
        d = oracle.dispatch(ids, g["E"], c["capacity"], order)
        assert d.assigned.tolist() == c["assigned"]
        assert d.keep.tolist() == c["keep"]
        assert d.offsets.tolist() == c["offsets"] and d.perm.tolist() == c["perm"]
        assert d.counts.tolist() == np.bincount(ids.reshape(-1), minlength=g["E"]).tolist()


def test_expert_ranking_matches_topk_and_margin():
    rng = np.random.default_rng(5)
    p = oracle.softmax(rng.standard_normal((30, 7)))
    order, margin = oracle.expert_ranking(p)
    for k in (1, 3, 7):
        ids, _, _ = oracle.topk_route(p, k)
        assert (order[:, :k] == ids).all()
    for t in range(30):
        assert sorted(order[t].tolist()) == list(range(7))
        sp = np.sort(p[t])[::-1]
        assert margin[t] == pytest.approx(np.min(sp[:-1] - sp[1:]), abs=0)
        assert (np.diff(p[t, order[t]]) <= 0).all()


@pytest.mark.parametrize("seed,T,E,k,cap", [(0, 60, 8, 2, 9), (1, 50, 6, 3, 20), (2, 80, 5, 1, 10),
                                             (3, 40, 8, 4, 12), (4, 33, 4, 2, 0), (5, 70, 16, 2, 6)])
def test_reroute_invariants(seed, T, E, k, cap):
    """Necessary conditions of the rule, checked without its loop: the cut's
    kept pairs stay put; loads stay within capacity; a moved pair lands past
    its token's top-k on an expert its token uses once; every expert a moved
    pair passed over is full at the end (room only shrinks) or used by an
    earlier slot of its token; a pair left dropped finds every candidate so."""
    rng = np.random.default_rng(seed)
    order, ids = _random_order_case(rng, T, E, k)
    base = oracle.dispatch(ids, E, cap)
    d = oracle.dispatch(ids, E, cap, order)
    assert (d.assigned[base.keep] == ids[base.keep]).all() and d.keep[base.keep].all()
    load = np.bincount(d.assigned[d.keep], minlength=E)
    assert (load <= cap).all()
    assert (d.counts == base.counts).all()
    pos = np.argsort(order, axis=1)                      # pos[t, e]: place of e in t's order
    for t in range(T):
        live = [int(d.assigned[t, s]) for s in range(k) if d.keep[t, s]]
        assert len(set(live)) == len(live)
        for s in range(k):
            if base.keep[t, s]:
                continue
            earlier = {int(d.assigned[t, j]) for j in range(s) if d.keep[t, j]}
            stop = pos[t, d.assigned[t, s]] if d.keep[t, s] else E
            if d.keep[t, s]:
                assert stop >= k
            for q in range(k, stop):
                e = int(order[t, q])
                assert load[e] == cap or e in earlier
    # bijection and (expert, token) order of the rows, as for the plain cut
    N = int(d.keep.sum())
    assert d.offsets[-1] == N and (d.inv_perm[d.perm] == np.arange(N)).all()
    e_rows = d.assigned.reshape(-1)[d.perm]
    assert (np.diff(e_rows * T + d.perm // k) > 0).all()


def test_reroute_is_lexicographic_best_by_brute_force():
    """Taken in priority order, the moved pairs' places in their tokens'
    orders form the lexicographically smallest vector over every feasible
    placement (capacity per expert, a token on an expert at most once, any
    pair may stay dropped): enumerate all placements of tiny cases."""
    from itertools import product
    rng = np.random.default_rng(21)
    checked = 0
    for trial in range(40):
        T, E, k = int(rng.integers(2, 6)), int(rng.integers(2, 5)), 0
        k = int(rng.integers(1, E + 1))
        cap = int(rng.integers(0, 3))
        order, ids = _random_order_case(rng, T, E, k)
        keep0 = oracle.capacity_keep(ids, E, cap)
        dropped = [(t, s) for s in range(k) for t in range(T) if not keep0[t, s]]
        if len(dropped) > 7:
            continue
        load0 = np.bincount(ids[keep0], minlength=E)
        options = [[int(order[t, q]) for q in range(k, E)] + [None] for t, s in dropped]
        best = None
        for choice in product(*options):
            load = load0.copy()
            used = {t: set() for t in range(T)}
            ok = True
            for (t, s), e in zip(dropped, choice):
                if e is None:
                    continue
                load[e] += 1
                if load[e] > cap or e in used[t]:
                    ok = False
                    break
                used[t].add(e)
            if not ok:
                continue
            vec = tuple(E if e is None else int(np.where(order[t] == e)[0][0])
                        for (t, s), e in zip(dropped, choice))
            if best is None or vec < best[0]:
                best = (vec, choice)
        assigned, keep = oracle.reroute_overflow(ids, order, keep0, E, cap)
        for (t, s), e in zip(dropped, best[1]):
            assert keep[t, s] == (e is not None)
            if e is not None:
                assert assigned[t, s] == e
        checked += 1
    assert checked >= 20


def test_reroute_limits():
    rng = np.random.default_rng(8)
    T, E, k = 45, 6, 2
    order, ids = _random_order_case(rng, T, E, k)
    full = oracle.dispatch(ids, E, -1)
    # capacity at the largest load: nothing overflows, nothing moves
    d = oracle.dispatch(ids, E, int(full.counts.max()), order)
    assert (d.assigned == ids).all() and d.keep.all() and (d.perm == full.perm).all()
    # capacity 0: nothing has room, every pair stays dropped
    z = oracle.dispatch(ids, E, 0, order)
    assert not z.keep.any() and len(z.perm) == 0
    # k = E: no expert lies past the top-k, so rerouting is the plain cut
    order_e, ids_e = _random_order_case(rng, 20, 4, 4)
    a = oracle.dispatch(ids_e, 4, 7, order_e)
    b = oracle.dispatch(ids_e, 4, 7)
    assert (a.keep == b.keep).all() and (a.perm == b.perm).all()
    # total room T*k: with k = 1 every token finds an expert (one option per place)
    order1, ids1 = _random_order_case(rng, 40, 8, 1)
    c = oracle.dispatch(ids1, 8, 5, order1)
    assert c.keep.all() and (np.bincount(c.assigned[:, 0], minlength=8) == 5).all()


def test_reroute_layer_equals_dense_mask():
    """The rerouted layer equals every expert run on every token, masked by
    the moved pairs' weights (computed expert by expert, independently of the
    sparse grouping)."""
    case = _case(13, T=30, d=16, E=5, k=2, F=24, bias_scale=1.5)
    cap = 8
    out, r, d = oracle.moe_forward(case.X, case.Wg, case.bias, case.W1, case.W2, 2, cap, reroute=True)
    assert d.keep.sum() > oracle.dispatch(r.ids, 5, cap).keep.sum()  # some pairs did move
    Xf = oracle.as_f64(case.X, "f32")
    ref = np.zeros_like(out)
    for e in range(5):
        h = Xf @ oracle.as_f64(case.W1[e], "f32").T
        h = 0.5 * h * (1 + np.tanh(math.sqrt(2 / math.pi) * (h + 0.044715 * h ** 3)))
        ye = h @ oracle.as_f64(case.W2[e], "f32").T
        m = np.array([sum(r.weights[t, s] for s in range(2) if d.keep[t, s] and d.assigned[t, s] == e)
                      for t in range(30)])
        ref += m[:, None] * ye
    assert np.abs(out - ref).max() < 1e-12


# ----------------------------------------------------------------- expert FFN
def test_single_expert_is_dense_ffn():
    """E = 1, k = 1: the layer is the textbook FFN Linear-GELU-Linear."""
    case = _case(9, T=16, d=20, E=1, k=1, F=36)
    out, r, _ = oracle.moe_forward(case.X, case.Wg, None, case.W1, case.W2, 1)
    assert (r.weights == 1.0).all()
    ffn = torch.nn.Sequential(torch.nn.Linear(20, 36, bias=False), torch.nn.GELU(approximate="tanh"),
                              torch.nn.Linear(36, 20, bias=False)).double()
    with torch.no_grad():
        ffn[0].weight.copy_(torch.tensor(case.W1[0], dtype=torch.float64))
        ffn[2].weight.copy_(torch.tensor(case.W2[0], dtype=torch.float64))
        ref = ffn(torch.tensor(case.X, dtype=torch.float64)).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_linearity_in_w2():
    case = _case(10, E=4, k=2)
    o1, _, _ = oracle.moe_forward(case.X, case.Wg, None, case.W1, case.W2, 2)
    o2, _, _ = oracle.moe_forward(case.X, case.Wg, None, case.W1, case.W2 * np.float32(4.0), 2)
    assert np.max(np.abs(o2 - 4 * o1)) < 1e-12


# ----------------------------------------------------------------- whole layer
@pytest.mark.parametrize("seed,E,k,cap", [(0, 6, 2, -1), (1, 8, 3, -1), (2, 5, 1, -1),
                                          (3, 6, 2, 5), (4, 4, 3, 9), (5, 6, 2, 0)])
def test_sparse_equals_dense_bruteforce(seed, E, k, cap):
    case = _case(seed, T=24, d=16, E=E, k=k, F=24, bias_scale=0.5)
    out, r, disp = oracle.moe_forward(case.X, case.Wg, case.bias, case.W1, case.W2, k, cap)
    ref, ids, w, keep = oracle.dense_bruteforce(case.X, case.Wg, case.bias, case.W1, case.W2, k, cap)
    assert (r.ids == ids).all()
    assert np.max(np.abs(r.weights - w)) < 1e-14
    assert (disp.keep == keep).all()
    assert np.max(np.abs(out - ref)) < 1e-12
    if cap == 0:
        assert (out == 0).all()


def test_k_equals_E_is_soft_mixture():
    """With every expert selected, the layer is the full softmax-weighted mixture."""
    E = 5
    case = _case(12, T=18, d=14, E=E, k=E, F=22, bias_scale=0.4)
    out, r, _ = oracle.moe_forward(case.X, case.Wg, case.bias, case.W1, case.W2, E)
    X = torch.tensor(case.X, dtype=torch.float64)
    logits = X @ torch.tensor(case.Wg, dtype=torch.float64) + torch.tensor(case.bias, dtype=torch.float64)
    p = torch.softmax(logits, -1)
    ref = torch.zeros_like(X)
    for e in range(E):
        h = torch.nn.functional.gelu(X @ torch.tensor(case.W1[e], dtype=torch.float64).T, approximate="tanh")
        ref += p[:, e:e + 1] * (h @ torch.tensor(case.W2[e], dtype=torch.float64).T)
    assert np.max(np.abs(out - ref.numpy())) < 1e-12


def test_token_permutation_equivariance():
    case = _case(13, T=30, E=6, k=2)
    out, _, _ = oracle.moe_forward(case.X, case.Wg, None, case.W1, case.W2, 2)
    pi = np.random.default_rng(0).permutation(30)
    outp, _, _ = oracle.moe_forward(case.X[pi], case.Wg, None, case.W1, case.W2, 2)
    assert np.max(np.abs(outp - out[pi])) < 1e-13


def test_token_subset_matches_full():
    case = _case(14, T=40, E=6, k=2, capacity=9)
    full, _, _ = oracle.moe_forward(case.X, case.Wg, None, case.W1, case.W2, 2, 9)
    toks = [3, 17, 39, 0]
    part, _, _ = oracle.moe_forward(case.X, case.Wg, None, case.W1, case.W2, 2, 9, tokens=toks)
    assert np.max(np.abs(part - full[toks])) < 1e-13  # BLAS may block rows differently


# ----------------------------------------------------------------- inputs
def test_bf16_rounding_and_widening_match_torch():
    rng = np.random.default_rng(3)
    a = (rng.standard_normal(100000) * 3).astype(np.float32)
    bits = workloads.f32_to_bf16_bits(a)
    ref = torch.tensor(a).to(torch.bfloat16)
    assert np.array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(oracle.as_f64(bits, "bf16"), ref.double().numpy())


def test_workload_recipe():
    w = workloads.WORKLOADS["skewed"]
    inp = workloads.generate("tiny")
    a = math.sqrt(6 / (128 + 8))
    assert np.abs(inp.Wg).max() <= a
    b = workloads._zipf_pmf_log_bias(w.E)
    pmf = np.exp(b.astype(np.float64) / 1.5)
    assert abs(pmf.sum() - 1) < 1e-5
    assert np.all(np.diff(b) < 0)
    # expert draws do not depend on which experts are drawn
    full = workloads.generate("tiny")
    part = workloads.generate("tiny", experts=[3])
    assert np.array_equal(full.W1[3], part.W1[3]) and np.array_equal(full.W2[3], part.W2[3])
    # a smaller T is a prefix of the same stream
    pre = workloads.generate("tiny", T=10)
    assert np.array_equal(pre.X, full.X[:10])
