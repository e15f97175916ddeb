"""Pins for the oracle's verification walk.

* Losslessness by exact enumeration on tiny vocabularies: over the draft
  tree's own randomness (the sampled token Y ~ q~) and every accept/reject
  coin, the emitted tokens follow the target distribution -- RheoSampling
  Theorem 1 / Appendix C (Equation 6 at one layer, the product p(a) p(b|a) over
  two layers with global pruning), Progressive Tree Drafting Appendix F.
* The per-layer acceptance rate equals RheoSampling's closed form
  (Theorem 3, Appendix D.1 Equation 13).
* Special cases: q~ = p always accepts the sampled child; one sampled child per
  layer is standard speculative sampling with acceptance sum_x min(p, q)
  (RheoSampling Section 2.2, Figure 1); a one-hot target picks its token.
* The worked example of RheoSampling Table 1 (golden file) pins the hybrid-pool
  tree builder used to make the trees above.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle.verify import rheo_verify_sequence, inverse_cdf, node_terminal_stats
from workloads import gen

from enumerate_util import enumerate_outcomes

HERE = os.path.dirname(os.path.abspath(__file__))


def _dirichlet(rng, V, alpha=0.7):
    x = rng.gamma(alpha, size=V)
    x = np.maximum(x, 1e-3)
    return x / x.sum()


def _one_layer(p, q, K, m, R, hybrid=True):
    """Enumerate building a one-layer pool (R of K slots kept) and verifying it.
    Returns {first emitted token: probability} and P(a candidate is accepted)."""
    V = p.size

    def run(ch):
        par, tok, smp, draft_of, paths, _ = gen.build_rheo_tree(
            R, 1, 1, K, m, lambda d, r: hybrid,
            lambda path, cid: (q, q),
            lambda path, qt: ch.sample(None, qt))
        p_of = lambda v: p if v == 0 else np.full(V, 1.0 / V)
        qt_of = lambda v: draft_of.get(v)
        status, path, bonus = rheo_verify_sequence(par, tok, smp, p_of, qt_of, ch)
        if len(path) > 1:
            return int(tok[path[1]]), True
        return int(bonus), False

    dist = np.zeros(V)
    acc = 0.0
    for (t, accepted), pr in enumerate_outcomes(run):
        dist[t] += pr
        acc += pr if accepted else 0.0
    return dist, acc


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("K,m,R", [(3, 1, 3), (4, 0, 4), (4, 2, 4), (4, 1, 2), (3, 1, 1), (5, 2, 3)])
def test_one_layer_lossless(seed, K, m, R):
    rng = np.random.default_rng(seed)
    V = 6
    p = _dirichlet(rng, V)
    q = _dirichlet(rng, V)
    dist, _ = _one_layer(p, q, K, m, R)
    np.testing.assert_allclose(dist, p, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("n,m", [(3, 1), (4, 1), (4, 2), (5, 0), (2, 1)])
def test_acceptance_matches_theorem3(seed, n, m):
    """Equation 13 with a full pool of n candidates whose sampled slot survives."""
    rng = np.random.default_rng(100 + seed)
    V = 7
    p = _dirichlet(rng, V)
    q = _dirichlet(rng, V)
    _, acc = _one_layer(p, q, n, m, n)
    order = np.lexsort((np.arange(V), -q))
    lead = order[:m]
    qt = q.copy(); qt[lead] = 0.0; qt /= qt.sum()
    top_n1 = set(int(t) for t in order[: n - 1])
    x_n = int(order[n - 1])
    r = np.maximum(0.0, p - qt); r /= r.sum()
    closed = (sum(p[v] for v in top_n1)
              + sum(min(p[v], qt[v]) for v in range(V) if v not in top_n1)
              + r[x_n] * sum(max(0.0, qt[v] - p[v]) for v in top_n1))
    assert abs(acc - closed) < 1e-12


def test_sequential_rejection_selects_with_target_probability():
    """Progressive Tree Drafting Appendix F: with only deterministic children,
    child i is selected with probability P_i (and the fallback draw covers the rest)."""
    rng = np.random.default_rng(5)
    V = 8
    p = _dirichlet(rng, V)
    parent = np.array([-1, 0, 0, 0], np.int32)
    token = np.array([-1, 5, 2, 7])
    sampled = np.zeros(4, np.uint8)

    def run(ch):
        status, path, bonus = rheo_verify_sequence(
            parent, token, sampled, lambda v: p if v == 0 else np.full(V, 1 / V), lambda v: None, ch)
        return ("child", path[1]) if len(path) > 1 else ("bonus", bonus)

    res = enumerate_outcomes(run)
    for c in (1, 2, 3):
        assert abs(sum(pr for r, pr in res if r == ("child", c)) - p[token[c]]) < 1e-12
    for t in range(V):
        expect = 0.0 if t in (5, 2, 7) else p[t]
        assert abs(sum(pr for r, pr in res if r == ("bonus", t)) - expect) < 1e-12


def _path_tables(seed, V):
    cache = {}

    def table(kind, path):
        key = (kind, tuple(path))
        if key not in cache:
            r = np.random.default_rng([seed, 1 if kind == "p" else 2, len(path)] + [t + 3 for t in path])
            cache[key] = _dirichlet(r, V)
        return cache[key]
    return table


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("R", [3, 5, 8])
def test_two_layer_lossless_with_global_pruning(seed, R):
    V = 5
    table = _path_tables(seed, V)

    def run(ch):
        par, tok, smp, draft_of, paths, _ = gen.build_rheo_tree(
            R, 2, 2, 3, 1, lambda d, r: True,
            lambda path, cid: (table("q", path), table("q", path)),
            lambda path, qt: ch.sample(None, qt))
        p_of = lambda v: table("p", paths[v])
        status, path, bonus = rheo_verify_sequence(par, tok, smp, p_of, lambda v: draft_of.get(v), ch)
        emitted = [int(tok[v]) for v in path[1:]] + [int(bonus)]
        return tuple(emitted[:2])

    joint = np.zeros((V, V))
    for em, pr in enumerate_outcomes(run):
        if len(em) == 2:
            joint[em[0], em[1]] += pr
        else:                          # one token emitted: the next one comes from p(.|a)
            joint[em[0], :] += pr * table("p", [em[0]])
    expect = np.array([[table("p", [])[a] * table("p", [a])[b] for b in range(V)] for a in range(V)])
    np.testing.assert_allclose(joint, expect, rtol=0, atol=1e-12)


def test_qtilde_equal_to_p_always_accepts_sampled_child():
    rng = np.random.default_rng(9)
    V = 6
    p = _dirichlet(rng, V)
    parent = np.array([-1, 0, 0], np.int32)
    sampled = np.array([0, 1, 0], np.uint8)

    for y in range(V):
        token = np.array([-1, y, (y + 1) % V])
        res = enumerate_outcomes(lambda ch: rheo_verify_sequence(
            parent, token, sampled, lambda v: p, lambda v: p if v == 0 else None, ch)[1])
        assert all(path[:2] == [0, 1] for path, pr in res)


def test_chain_of_sampled_children_is_speculative_sampling():
    rng = np.random.default_rng(4)
    V = 7
    p = _dirichlet(rng, V)
    q = _dirichlet(rng, V)
    parent = np.array([-1, 0], np.int32)
    sampled = np.array([0, 1], np.uint8)

    def run(ch):
        y = ch.sample(None, q)                     # the draft token Y ~ q
        token = np.array([-1, y])
        return len(rheo_verify_sequence(parent, token, sampled, lambda v: p,
                                        lambda v: q if v == 0 else None, ch)[1]) > 1

    acc = sum(pr for a, pr in enumerate_outcomes(run) if a)
    assert abs(acc - np.minimum(p, q).sum()) < 1e-12


def test_one_hot_target_selects_that_child():
    V = 5
    p = np.zeros(V); p[3] = 1.0
    parent = np.array([-1, 0, 0, 0], np.int32)
    token = np.array([-1, 1, 3, 4])
    res = enumerate_outcomes(lambda ch: rheo_verify_sequence(
        parent, token, np.zeros(4, np.uint8), lambda v: p if v == 0 else np.full(V, .2),
        lambda v: None, ch)[1][:2])
    assert all(path == [0, 2] for path, pr in res)
    assert abs(sum(pr for path, pr in res) - 1.0) < 1e-12


def test_residual_mass_identity():
    """sum (p - q~)+ = sum (q~ - p)+ for any two distributions (RheoSampling Eq. 10)."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        p = _dirichlet(rng, 50); q = _dirichlet(rng, 50)
        assert abs(np.maximum(p - q, 0).sum() - np.maximum(q - p, 0).sum()) < 1e-14


def test_inverse_cdf_small_cases():
    w = np.array([0.0, 0.25, 0.25, 0.0, 0.5])
    assert inverse_cdf(w, 0.0)[0] == 1
    assert inverse_cdf(w, 0.2499)[0] == 1
    assert inverse_cdf(w, 0.25)[0] == 2          # cumsum must exceed u * total
    assert inverse_cdf(w, 0.5)[0] == 4
    assert inverse_cdf(w, 0.999999)[0] == 4
    assert inverse_cdf(w * 7.0, 0.3)[0] == 2     # scale-free


def test_rheo_table1_golden():
    g = json.load(open(os.path.join(HERE, "golden", "rheo_table1.json")))
    q = np.array(g["q"])
    for row in g["rows"]:
        override = None if row["proxy"] == "rheo" else g["adhoc_proxy"]
        par, tok, smp, draft_of, paths, _ = gen.build_rheo_tree(
            g["R"], 1, 1, g["K"], g["m"], lambda d, r: True, lambda path, cid: (q, q),
            lambda path, qt, y=row["Y"]: y, proxy_override=override)
        got = [("Y" if smp[v] else int(tok[v])) for v in range(1, len(tok))]
        assert got == row["survivors"]
        if 0 in draft_of:                         # the sampled slot survived: check q~
            for t, val in g["qtilde"].items():
                assert abs(draft_of[0][int(t)] - val) < 1e-12
        assert ("Y" in got) == (0 in draft_of)
    # Rheo proxy = min{q(x_1), z} = min{0.5, 0.5}
    assert abs(min(q[0], 1.0 - q[0]) - g["rheo_proxy"]) < 1e-15


def test_terminal_stats_agree_with_walk_end():
    """The per-node terminal draw equals the walk's draw when the walk ends there."""
    w = gen.tree_batch(21, B=2, prefix_len=[3, 4], tree="random", n_nodes=[12, 9], Hq=2, Hkv=1,
                       D=8, dtype="f32", V=300, temperature=0.8, max_depth=4)
    res = oracle.verify_workload(w)
    for b, r in enumerate(res):
        s = int(w.node_offsets[b])
        v = r["path"][-1]
        kids = [c for c in range(1, w.node_offsets[b + 1] - s) if w.parent[s + c] == v]
        det = [int(w.token[s + c]) for c in kids if not w.sampled[s + c]]
        dr = int(w.draft_row[s + v])
        qt = None if dr < 0 else w.draft[dr]
        M, S, Z, tok, _ = node_terminal_stats(w.logits[s + v], w.temperature[b], qt, det,
                                              w.uniforms[s + v, 1])
        assert tok == r["bonus"]


def _truncated(q, k):
    """RheoSampling Section 3.2's sparse draft: the draft's logits kept at their k largest
    entries before the softmax, i.e. q restricted to its top-k tokens and renormalised."""
    keep = np.lexsort((np.arange(q.size), -q))[:k]
    out = np.zeros_like(q)
    out[keep] = q[keep]
    return out / out.sum()


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("K,m,R,k", [(3, 1, 3, 3), (4, 0, 4, 2), (4, 2, 3, 4), (3, 1, 2, 4), (4, 1, 4, 5)])
def test_one_layer_lossless_with_truncated_draft(seed, K, m, R, k):
    """Verification with the truncated draft (tokens outside the support have q~ = 0, so the
    residual (p - q~)+ keeps all their target mass) is still lossless: the emitted token follows
    p exactly (RheoSampling Section 3.2: losslessness holds when verification uses the same
    truncated distribution the draft was sampled from)."""
    rng = np.random.default_rng(200 + seed)
    V = 7
    p = _dirichlet(rng, V)
    q = _truncated(_dirichlet(rng, V), k)
    dist, _ = _one_layer(p, q, K, m, R)
    np.testing.assert_allclose(dist, p, rtol=0, atol=1e-12)


@pytest.mark.parametrize("tree", ["random", "eagle"])
def test_sparse_rows_equal_their_dense_scatter(tree):
    """The oracle's sparse draft rows are exactly the dense rows with zeros off the support: the
    walk on a workload with sparse rows and on the same workload with each row scattered into a
    dense one takes the same decisions and draws the same tokens."""
    extra = {"max_depth": 4, "hybrid": "all", "draft_peak": (4.0, 7.0)} if tree == "eagle" else {}
    w = gen.tree_batch(17, B=3, prefix_len=[5, 6, 7], tree=tree, n_nodes=[12, 20, 9], Hq=2, Hkv=1, D=8,
                       dtype="f32", V=700, temperature=0.8, draft_support=24, **extra)
    assert w.draft_k == 24 and w.draft is None
    assert (np.diff(w.draft_idx, axis=1) > 0).all()
    sparse = oracle.verify_workload(w)
    dense = np.zeros((w.draft_idx.shape[0], w.V), np.float32)
    for r in range(dense.shape[0]):
        dense[r, w.draft_idx[r]] = w.draft_val[r]
        assert np.count_nonzero(dense[r]) <= 24
    w.draft, w.draft_k, w.draft_idx, w.draft_val = dense, 0, None, None
    for a, b in zip(sparse, oracle.verify_workload(w)):
        assert a["path"] == b["path"] and a["bonus"] == b["bonus"]
        np.testing.assert_array_equal(a["status"], b["status"])
