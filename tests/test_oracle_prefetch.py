"""Pins for the oracle's prefetching-tree construction and reaching weights (PreSTO Section 3.2
step (1) and Appendix C), and host parity of tav_prefetch_build / tav_prefetch_reach with it.

Pins (each rests on something other than the function it checks):
* SplitMix64's published first outputs for seed 0;
* Example 2's BFS tree (golden file, from the page) with its two sampled cuts;
* deferral: an infeasible acceptance child is created but not expanded, its sibling is;
* Lemma 1 = Lemma 2 = the traversal of Definition 1 enumerated path by path, on scored trees with
  rounded branch probabilities (Equation 10) and deferred nodes;
* Proposition 2: the dynamic program's value equals a brute-force maximum over every
  ancestor-closed subset of the candidates, and the sum of the largest predicted reaching weights;
* the Remark of Appendix C.2: a selection of |I| nodes issues |I| requests and yields a subtree of
  2|I| + 1 nodes; Condition 1 holds for every issued request;
* Equation 14 is the midpoint of Lemma 3's interval.

Host parity: the library's BFS trees are identical to the oracle's; its predictive trees reach the
dynamic program's optimum (identical trees when the optimum is unique), and at budgets the dynamic
program cannot reach (up to 62) its selection carries an optimality certificate: ancestor-closed,
made of candidates, and no candidate outside it has a larger predicted reaching weight than the
smallest inside it.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle.prefetch as op

HERE = os.path.dirname(os.path.abspath(__file__))
W_DEFAULT = [1.0, -3.0, -1.0, 2.5, 0.0, 0.0]


def _weights(seed):
    """Class weights representable in float32 (the library's parameter type)."""
    r = np.random.default_rng(seed)
    return [float(np.float32(x)) for x in r.normal(0.0, 1.5, 6)]


def test_splitmix64_known_outputs():
    x, outs = 0, []
    for _ in range(3):
        outs.append(op.splitmix64(x))
        x = (x + 0x9E3779B97F4A7C15) & op.MASK64
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_example2_bfs_golden():
    g = json.load(open(os.path.join(HERE, "golden", "presto_examples.json")))["example2"]
    drawn = {2: g["sampled_cuts"][0], 4: g["sampled_cuts"][1]}
    t = op.bfs_tree(g["T"], 2, 100, lambda h: drawn[h])
    assert t["parent"].tolist() == g["pf_parent"]
    assert t["is_accept"].tolist() == g["pf_is_accept"]
    assert t["request"].tolist() == g["pf_request"]
    assert t["cut"].tolist() == g["pf_cut"]
    assert t["request_cut"].tolist() == g["request_cuts"]


def test_bfs_deferral():
    # root cut 10; v1 (heap 2) cut 6 fits; v3 (heap 4, under v1) cut 9 > 6: deferred, not expanded;
    # v2 (heap 3, rejection child of the root, cut 10) is expanded next: heap 6 cut 2 fits
    cuts = {2: 6, 4: 9, 6: 2, 10: 1, 12: 0, 14: 5}
    t = op.bfs_tree(10, 3, 100, lambda h: cuts.get(h, 0))
    heap = t["heap"].tolist()
    req = dict(zip(heap, t["request"].tolist()))
    assert req[2] == 0 and req[4] == -1 and req[6] == 1
    assert 8 not in heap and 9 not in heap          # the deferred node has no children
    assert 5 in heap and 10 in heap                 # its sibling was expanded
    for h, c in zip(heap, t["cut"].tolist()):
        if h > 1 and req.get(h, -1) >= 0:
            assert c <= t["cut"].tolist()[heap.index(h // 2)]


def _scored(seed, rule, T=48, budget=9):
    cut_of = lambda h: op.splitmix_cut(seed, h, T)
    t = op.bfs_tree(T, budget, 20, cut_of) if rule == "bfs" else op.predictive_tree(T, budget, 20, cut_of, W_DEFAULT)
    r = np.random.default_rng(seed)
    R = len(t["request_cut"])
    la = np.log(np.clip(r.choice([0.001, 0.3, 0.7, 0.999, 1.0], R) * r.uniform(0.5, 1.0, R), 1e-6, 1.0))
    return t, la.astype(np.float32)


def _traversal_expectation(t, la, eps):
    """Definition 1's traversal, path by path: from the root, at an expanded node go to v+ with
    h(v+) and to v- with 1 - h(v+); count the expanded nodes visited; stop elsewhere."""
    par, acc_flag, req = t["parent"], t["is_accept"], t["request"]
    kids = {}
    for v in range(1, len(par)):
        kids.setdefault(int(par[v]), {})["a" if acc_flag[v] else "r"] = v

    def walk(v, prob, count):
        k = kids.get(v, {})
        a = k.get("a")
        if a is None or int(req[a]) < 0:
            return prob * count
        h = op.rounded_h(math.exp(float(la[int(req[a])])), eps)
        out = 0.0
        if h > 0:
            out += walk(a, prob * h, count + 1)
        if h < 1:
            out += walk(k["r"], prob * (1 - h), count + 1) if "r" in k else prob * (1 - h) * (count + 1)
        return out

    return walk(0, 1.0, 0)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("rule", ["bfs", "predictive"])
@pytest.mark.parametrize("eps", [0.0, 0.01, 0.3])
def test_lemma1_equals_lemma2_equals_traversal(seed, rule, eps):
    t, la = _scored(seed, rule)
    R, F, expanded = op.reaching_weights(t["parent"], t["is_accept"], t["request"], la, eps)
    F13 = op.transitions_recursive(t["parent"], t["is_accept"], t["request"], la, eps)
    assert abs(F - F13) < 1e-12
    assert abs(F - _traversal_expectation(t, la, eps)) < 1e-12


def test_equation10_rounding():
    assert op.rounded_h(0.01, 0.01) == 0.0 and op.rounded_h(0.99, 0.01) == 1.0
    assert op.rounded_h(0.5, 0.01) == 0.5 and op.rounded_h(0.0101, 0.01) == 0.0101
    assert op.rounded_h(1.0, 0.0) == 1.0 and op.rounded_h(0.0, 0.0) == 0.0


def test_equation14_is_lemma3_midpoint():
    for seed in range(10):
        w = _weights(seed)
        for frac in (0.0, 0.3, 0.77, 1.0):
            P = op.class_probs(w, frac)
            eps = 0.01
            lo = P[op.ACCEPT] + eps * P[op.UNCERTAIN]
            hi = P[op.ACCEPT] + (1 - eps) * P[op.UNCERTAIN]
            h = op.predicted_h(w, int(round(frac * 1000)), 1000)
            assert abs(h - 0.5 * (lo + hi)) < 1e-12 and 0.0 < h < 1.0


def _ancestor_closed_sets(C, max_size):
    """Every ancestor-closed set of candidate nodes of size <= max_size (grown from the root)."""
    out = {frozenset()}
    if not C.candidate(1):
        return out
    frontier = [frozenset([1])]
    seen = set(frontier)
    while frontier:
        s = frontier.pop()
        out.add(s)
        if len(s) == max_size:
            continue
        for h in s:
            for c in (2 * h, 2 * h + 1):
                if c not in s and C.candidate(c):
                    n = s | {c}
                    if n not in seen:
                        seen.add(n)
                        frontier.append(n)
    return out


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("budget,K", [(1, 5), (3, 5), (5, 6), (6, 3)])
def test_proposition2_dp_is_brute_force_optimum(seed, budget, K):
    T = 30
    w = _weights(100 + seed)
    cut_of = lambda h: op.splitmix_cut(seed, h, T)
    val, sel, C = op.dp_value(T, budget, K, cut_of, w)
    best = max(sum(C.reach(h) for h in s) for s in _ancestor_closed_sets(C, budget))
    assert abs(val - best) < 1e-12
    assert abs(sum(C.reach(h) for h in sel) - val) < 1e-12
    # every candidate within reach of the budget, by predicted reaching weight
    cands = [h for h in range(1, 1 << min(budget, K)) if C.candidate(h)]
    top = sorted((C.reach(h) for h in cands), reverse=True)[:budget]
    assert abs(sum(top) - val) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_predictive_tree_shape(seed):
    T, budget = 64, 8
    cut_of = lambda h: op.splitmix_cut(seed, h, T)
    t = op.predictive_tree(T, budget, 20, cut_of, _weights(seed))
    n_sel = len(t["selection"])
    assert len(t["request_cut"]) == n_sel and len(t["parent"]) == 2 * n_sel + 1
    heap = t["heap"].tolist()
    for i, h in enumerate(heap):
        if t["request"][i] >= 0:
            assert t["cut"][i] <= t["cut"][heap.index(h // 2)]      # Condition 1
        assert h.bit_length() - 1 <= budget


# ---------------------------------------------------------------------------------------------
# host parity: the library's builder against the oracle (no GPU: both are host code)
# ---------------------------------------------------------------------------------------------

def _lib():
    import tree_masked_verification_attn_amd as tav

    return tav


@pytest.mark.parametrize("seed", [10086, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("T,budget,K", [(8, 2, 10), (64, 8, 20), (4096, 32, 100), (100, 20, 4), (30, 62, 62)])
def test_bfs_parity(seed, T, budget, K):
    tav = _lib()
    got = tav.tav_prefetch_build(T, budget, K, tav.TAV_PREFETCH_BFS, seed, W_DEFAULT)
    want = op.bfs_tree(T, budget, K, lambda h: op.splitmix_cut(seed, h, T))
    for k in ("parent", "is_accept", "request", "cut", "heap", "request_cut"):
        np.testing.assert_array_equal(got[k], want[k], err_msg=k)
    F = op.predicted_transitions(want["parent"], want["is_accept"], want["request"], want["cut"], W_DEFAULT, T)
    assert abs(got["predicted_transitions"] - F) < 1e-9


@pytest.mark.parametrize("seed", [10086, 1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("T,budget,K", [(8, 2, 10), (64, 8, 20), (4096, 10, 100), (100, 9, 4)])
def test_predictive_parity_with_dynamic_program(seed, T, budget, K):
    tav = _lib()
    w = _weights(seed)
    got = tav.tav_prefetch_build(T, budget, K, tav.TAV_PREFETCH_PREDICTIVE, seed, w)
    want = op.predictive_tree(T, budget, K, lambda h: op.splitmix_cut(seed, h, T), w)
    assert abs(got["predicted_transitions"] - want["predicted_transitions"]) < 1e-9
    F = op.predicted_transitions(got["parent"], got["is_accept"], got["request"], got["cut"], w, T)
    assert abs(F - want["predicted_transitions"]) < 1e-9
    if got["heap"].tolist() != want["heap"].tolist():      # only when the optimum is not unique
        C = op._Candidates(T, K, lambda h: op.splitmix_cut(seed, h, T), w)
        vals = sorted(C.reach(h) for h in want["selection"])
        assert any(abs(a - b) < 1e-12 for a, b in itertools.combinations(vals, 2)) or len(vals) < budget
    else:
        for k in ("parent", "is_accept", "request", "cut", "request_cut"):
            np.testing.assert_array_equal(got[k], want[k], err_msg=k)


@pytest.mark.parametrize("seed", [10086, 1, 2, 3])
@pytest.mark.parametrize("T,budget,K", [(4096, 32, 100), (4096, 62, 62), (50, 40, 12)])
def test_predictive_optimality_certificate(seed, T, budget, K):
    tav = _lib()
    w = _weights(seed)
    got = tav.tav_prefetch_build(T, budget, K, tav.TAV_PREFETCH_PREDICTIVE, seed, w)
    C = op._Candidates(T, K, lambda h: op.splitmix_cut(seed, h, T), w)
    heap = got["heap"].tolist()
    sel = [h for i, h in enumerate(heap) if got["request"][i] >= 0]
    sel = [h // 2 for h in sel]                                 # expanded nodes: parents of requests
    assert len(sel) <= budget and all(C.candidate(h) for h in sel)
    ss = set(sel)
    assert all(h == 1 or h // 2 in ss for h in sel)             # ancestor-closed
    assert abs(sum(C.reach(h) for h in sel) - got["predicted_transitions"]) < 1e-9
    if len(sel) == budget:
        low = min(C.reach(h) for h in sel)
        frontier = [c for h in sel for c in (2 * h, 2 * h + 1) if c not in ss and C.candidate(c)]
        assert all(C.reach(c) <= low + 1e-12 for c in frontier)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("rule", ["bfs", "predictive"])
@pytest.mark.parametrize("eps", [0.0, 0.01, 0.2])
def test_reach_parity(seed, rule, eps):
    tav = _lib()
    t, la = _scored(seed, rule)
    reach, F = tav.tav_prefetch_reach(t["parent"], t["is_accept"], t["request"], la, eps)
    R, Fo, _ = op.reaching_weights(t["parent"], t["is_accept"], t["request"], la, eps)
    np.testing.assert_allclose(reach, R, rtol=1e-12, atol=1e-15)
    assert abs(F - Fo) < 1e-12


def test_builder_errors():
    tav = _lib()
    with pytest.raises(tav.TavError):
        tav.tav_prefetch_build(64, 0, 10, 0, 1, W_DEFAULT)
    with pytest.raises(tav.TavError):
        tav.tav_prefetch_build(64, 63, 10, 0, 1, W_DEFAULT)
    with pytest.raises(tav.TavError):
        tav.tav_prefetch_build(64, 4, 10, 7, 1, W_DEFAULT)
    with pytest.raises(tav.TavError):
        tav.tav_prefetch_build(64, 4, 10, 1, 1, [float("nan")] + W_DEFAULT[1:])
    with pytest.raises(tav.TavError):
        tav.tav_prefetch_build(64, 8, 10, 0, 1, W_DEFAULT, capacity=5)
