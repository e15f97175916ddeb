"""Pins for the oracle's draft-tree construction (RheoSampling Sections 2.1 and 3.2, Appendix C).

* Table 1 (golden file): q = (.5, .3, .2), K = 3, m = 1, R = 2 -- with the Rheo proxy min{q(x_1), z}
  the survivors are {A, Y} whatever Y is; with the ad-hoc proxy .25 and Y = C they are {A, B};
* Lemma 4: the sampled token's proxy is at least q(x_{m+1}), hence at least every fill's proxy;
* Lemma 5 and the tie-break: path scores never rise from parent to child and the pruned tree is
  ancestor-closed (checked inside prune);
* Theorem 1 (losslessness), by exact enumeration: over the sampled token Y (each Y with
  probability q~(Y), through the builder's inverse CDF) and every accept/reject coin of the
  verification, the first emitted token follows the target p -- with the sparse draft (support
  smaller than the vocabulary) as well;
* the same pools and trees as the input generator's builder when nothing is truncated.
"""

import json
import os

import numpy as np
import pytest

import oracle.draft_tree as odt
import oracle.verify as ov
from enumerate_util import enumerate_outcomes
from workloads import gen

HERE = os.path.dirname(os.path.abspath(__file__))


def test_table1_golden():
    g = json.load(open(os.path.join(HERE, "golden", "rheo_table1.json")))
    q = np.array(g["q"])
    z = np.log(q)
    names = ["A", "B", "C"]
    for row in g["rows"]:
        override = None if row["proxy"] == "rheo" else g["adhoc_proxy"]
        y = names.index(row["Y"]) if isinstance(row["Y"], str) else int(row["Y"])
        qt = {1: 0.6, 2: 0.4}
        u = 0.3 if y == 1 else 0.8                      # inside Y's step of the tail CDF (B, C)
        t = odt.DraftTreeBuilder(3, 1, 1, g["K"], g["m"], "all", 3, g["R"], proxy_override=override)
        t.expand(1, [z], [u])
        parent, token, sampled, cids, rows = t.prune()
        got = ["Y" if sampled[v] else int(token[v]) for v in range(1, len(token))]
        assert got == row["survivors"], (row, got)
        if rows[0] is not None:
            ids, vals = rows[0]
            for tok, val in g["qtilde"].items():
                assert abs(vals[list(ids).index(int(tok))] - val) < 1e-12
            assert abs(qt[y] - g["qtilde"][str(y)]) < 1e-12


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("m,S", [(0, 20), (1, 20), (2, 12), (1, 50)])
def test_lemma4_sampled_proxy_above_fills(seed, m, S):
    r = np.random.default_rng(seed)
    V = 50
    t = odt.DraftTreeBuilder(V, 1, 1, 6, m, "all", S, 3)
    z = r.normal(0, 2, V)
    t.expand(1, [z], [float(r.random())])
    keep = odt.support_of(z, S)
    q = np.exp(z[keep] - z[keep].max())
    q /= q.sum()
    prox = [t.score[c] for c in range(1, len(t.score))]      # root score 1: score = proxy
    smp = [t.sampled[c] for c in range(1, len(t.score))]
    y = smp.index(True)
    assert prox[y] >= q[m] - 1e-15
    assert all(prox[y] >= prox[i] - 1e-15 for i in range(y + 1, len(prox)))


@pytest.mark.parametrize("seed", range(4))
def test_lemma5_scores_fall_and_prune_is_ancestor_closed(seed):
    V = 300
    t, (parent, token, sampled, cids, rows) = odt.build(
        V, 5, 4, 4, 1, "all", 32, 30,
        lambda c: gen.bf16_bits_to_f32(gen.draft_logits_row(seed, 0, c, V)).astype(np.float64),
        lambda d, r: gen.draft_uniform(seed, 0, d, r))
    for c in range(1, len(t.score)):
        assert t.score[c] <= t.score[t.parent[c]] + 1e-15
    assert (parent[1:] < np.arange(1, len(parent))).all()


def _first_token_distribution(p, z, K, m, R, S):
    """Exact law of the first emitted token: Y enumerated with probability q~(Y) (the builder's
    inverse CDF at the middle of Y's step), verification enumerated coin by coin."""
    V = p.size
    keep = odt.support_of(z, S)
    qT = np.exp(z[keep] - z[keep].max())
    qT /= qT.sum()
    tail = qT.copy()
    tail[:m] = 0.0
    tail /= tail.sum()
    ids = np.argsort(keep)
    cum = np.cumsum(tail[ids])
    dist = np.zeros(V)
    for j in range(len(ids)):
        w = tail[ids][j]
        if w <= 0:
            continue
        u = (cum[j] - w / 2)
        t = odt.DraftTreeBuilder(V, 1, 1, K, m, "all", S, R)
        t.expand(1, [z], [u])
        parent, token, sampled, cids, rows = t.prune()
        qtil = np.zeros(V)
        if rows[0] is not None:
            qtil[rows[0][0]] = rows[0][1]

        def run(ch):
            status, path, bonus = ov.rheo_verify_sequence(
                parent, token, sampled, lambda v: p if v == 0 else np.full(V, 1 / V),
                lambda v: qtil if (v == 0 and rows[0] is not None) else None, ch)
            return int(token[path[1]]) if len(path) > 1 else int(bonus)

        for tok, pr in enumerate_outcomes(run):
            dist[tok] += w * pr
    return dist


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("K,m,R,S", [(3, 1, 3, 6), (3, 0, 2, 6), (4, 2, 3, 6), (3, 1, 2, 4), (4, 1, 4, 5)])
def test_theorem1_one_layer_lossless(seed, K, m, R, S):
    r = np.random.default_rng(300 + seed)
    V = 6
    p = r.dirichlet(np.full(V, 0.8))
    z = r.normal(0, 1.5, V)
    dist = _first_token_distribution(p, z, K, m, R, S)
    np.testing.assert_allclose(dist, p, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_same_trees_as_the_input_generator(seed):
    V, D, K, slots, m, R = 400, 4, 3, 4, 1, 20
    logits = {}

    def z_of(c):
        if c not in logits:
            logits[c] = gen.bf16_bits_to_f32(gen.draft_logits_row(seed, 0, c, V)).astype(np.float64)
        return logits[c]

    t, (parent, token, sampled, cids, rows) = odt.build(V, D, K, slots, m, "all", V, R, z_of,
                                                        lambda d, r: gen.draft_uniform(seed, 0, d, r))
    # the generator's builder on the same distributions, with its sampled tokens forced to the
    # oracle's (its own sampler is a different stream)
    ys = {t.parent[c]: t.token[c] for c in range(1, len(t.token)) if t.sampled[c]}

    def probs(path, cid):
        q = np.exp(z_of(cid) - z_of(cid).max())
        q /= q.sum()
        return q, q

    calls = []

    def sample_tail(path, qt):
        return ys[calls[-1]]

    def probs_tracking(path, cid):
        calls.append(cid)
        return probs(path, cid)

    gp, gt, gs, gdraft, _, gcids = gen.build_rheo_tree(R, D, K, slots, m, lambda d, r: True, probs_tracking,
                                                      sample_tail)
    np.testing.assert_array_equal(gp, parent)
    np.testing.assert_array_equal(gt[1:], token[1:])
    np.testing.assert_array_equal(gs, sampled)
    np.testing.assert_array_equal(np.array(gcids), cids)
