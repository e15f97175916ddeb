"""Pins for the oracle's PreSTO log-acceptance and prefetched-subtree walk.

* Equation 6 (prefix cancelled) equals the unsimplified MH ratio of Equation 7,
  computed here from full-sequence sums over t = 1..T of both states
  (PreSTO Appendix B.1).
* y = x gives log A = 0; alpha = 1 with q_tau = p0 gives log A = 0; the
  unclamped log ratio is antisymmetric in (x, y) (Equation 1).
* Example 2 / Figure 8(b) (golden file): the BFS prefetching tree.
* Example 5 (golden file): path v0 -> v1 -> v4, trajectory x -> y -> y.
* Proposition 1: a plain sequential PowerMH chain, run here with the same
  per-decision proposals and uniforms, visits exactly the same states.
"""

import json
import os

import numpy as np
import pytest

import oracle
from workloads import gen

HERE = os.path.dirname(os.path.abspath(__file__))


class _FixedCuts:
    def __init__(self, cuts):
        self.cuts = list(cuts)

    def integers(self, lo, hi):
        c = self.cuts.pop(0)
        assert lo <= c < hi
        return c


def _inputs(T, pf, cuts, rng, alpha=4.0, u=None, max_transitions=100):
    pf_parent, pf_acc, pf_req, pf_cut = pf
    cuts = np.asarray(cuts, np.int32)
    lens = T - cuts
    off = np.zeros(len(cuts) + 1, np.int32)
    off[1:] = np.cumsum(lens)
    M = len(pf_parent)
    return gen.PrestoInputs(
        T=T, alpha=alpha,
        root_lp0=-rng.exponential(size=T), root_lq=-rng.exponential(size=T),
        cut=cuts, suffix_off=off,
        lp0=-rng.exponential(size=int(off[-1])), lq=-rng.exponential(size=int(off[-1])),
        pf_parent=np.asarray(pf_parent, np.int32), pf_is_accept=np.asarray(pf_acc, np.uint8),
        pf_request=np.asarray(pf_req, np.int32), pf_cut=np.asarray(pf_cut, np.int32),
        u=np.asarray(u if u is not None else rng.random(M), np.float64),
        max_transitions=max_transitions)


def _mh_log_ratio_eq7(x, y, c, alpha):
    """log [pi(y) q(x|y,c)] - log [pi(x) q(y|x,c)] with pi ∝ p0^alpha over the whole
    response (t = 1..T) and the suffix proposal probabilities at cut c."""
    lp0_x, lq_x = x
    lp0_y, lq_y = y
    target = alpha * (lp0_y.sum() - lp0_x.sum())
    proposal = lq_x[c:].sum() - lq_y[c:].sum()
    return target + proposal


@pytest.mark.parametrize("seed", [10086, 1, 2])
def test_equation6_equals_equation7(seed):
    rng = np.random.default_rng(seed)
    T = 40
    pf_parent, pf_acc, pf_req, pf_cut, cuts = gen.bfs_prefetch_tree(T, 12, np.random.default_rng(seed))
    pr = _inputs(T, (pf_parent, pf_acc, pf_req, pf_cut), cuts, rng)
    states = oracle.presto_states(pr)
    logA = oracle.presto_log_accept(pr, states)
    for v in range(1, len(pf_parent)):
        i = int(pf_req[v])
        if pf_acc[v] and i >= 0:
            x = states[int(pf_parent[v])]
            y = states[v]
            # the proposal keeps x's tokens up to the cut
            np.testing.assert_array_equal(y[0][: cuts[i]], x[0][: cuts[i]])
            ref = min(0.0, _mh_log_ratio_eq7(x, y, int(cuts[i]), pr.alpha))
            assert abs(logA[i] - ref) < 1e-9


def test_identical_proposal_and_symmetric_cases():
    rng = np.random.default_rng(0)
    T, c = 30, 11
    pf = ([-1, 0, 0], [0, 1, 0], [-1, 0, -1], [T, c, T])
    pr = _inputs(T, pf, [c], rng)
    # y == x: suffix equal to the state's own tokens -> log A = 0
    pr.lp0 = pr.root_lp0[c:].copy(); pr.lq = pr.root_lq[c:].copy()
    assert oracle.presto_log_accept(pr)[0] == 0.0
    # alpha = 1 and q_tau == p0 -> the ratio is exactly 1
    pr2 = _inputs(T, pf, [c], rng, alpha=1.0)
    pr2.root_lq = pr2.root_lp0.copy(); pr2.lq = pr2.lp0.copy()
    assert abs(oracle.presto_log_accept(pr2)[0]) < 1e-12
    # antisymmetry of the unclamped ratio: swap which sequence is the state
    pr3 = _inputs(T, pf, [c], rng)
    st = oracle.presto_states(pr3)
    x, y = st[0], st[1]
    fwd = _mh_log_ratio_eq7(x, y, c, pr3.alpha)
    swapped = gen.PrestoInputs(**{**pr3.__dict__})
    swapped.root_lp0, swapped.root_lq = y
    swapped.lp0, swapped.lq = x[0][c:].copy(), x[1][c:].copy()
    back = oracle.presto_log_accept(swapped)[0]
    assert abs(min(0.0, -fwd) - back) < 1e-9


def test_example2_bfs_tree_golden():
    g = json.load(open(os.path.join(HERE, "golden", "presto_examples.json")))["example2"]
    pf_parent, pf_acc, pf_req, pf_cut, cuts = gen.bfs_prefetch_tree(g["T"], 2, _FixedCuts(g["sampled_cuts"]))
    assert pf_parent.tolist() == g["pf_parent"]
    assert pf_acc.tolist() == g["pf_is_accept"]
    assert pf_req.tolist() == g["pf_request"]
    assert pf_cut.tolist() == g["pf_cut"]
    assert cuts.tolist() == g["request_cuts"]


def test_example5_walk_golden():
    g = json.load(open(os.path.join(HERE, "golden", "presto_examples.json")))
    e2, e5 = g["example2"], g["example5"]
    rng = np.random.default_rng(5)
    pf = (e2["pf_parent"], e2["pf_is_accept"], e2["pf_request"], e2["pf_cut"])
    pr = _inputs(e2["T"], pf, e2["request_cuts"], rng)
    st = oracle.presto_states(pr)
    a_yx = np.exp(min(0.0, _mh_log_ratio_eq7(st[0], st[1], e2["request_cuts"][0], pr.alpha)))
    a_zy = np.exp(min(0.0, _mh_log_ratio_eq7(st[1], st[3], e2["request_cuts"][1], pr.alpha)))
    if a_zy >= 1.0:                 # make the second proposal rejectable
        pr.lp0 = pr.lp0.copy(); pr.lp0[e2["T"] - e2["request_cuts"][0]:] -= 50.0
        st = oracle.presto_states(pr)
        a_zy = np.exp(min(0.0, _mh_log_ratio_eq7(st[1], st[3], e2["request_cuts"][1], pr.alpha)))
    u = np.zeros(5)
    u[0] = 0.5 * a_yx              # u <= A(y, x)
    u[1] = 0.5 * (1.0 + a_zy)      # u' > A(z, y)
    logA = oracle.presto_log_accept(pr, st)
    path, k, _ = oracle.presto_walk(pr, logA, u)
    assert path == e5["path"] and k == e5["transitions"]
    names = {0: "x", 1: "y", 3: "z"}
    traj = []
    for v in path:                  # a rejection child carries its parent's state
        while v not in names:
            v = e2["pf_parent"][v]
        traj.append(names[v])
    assert traj == e5["trajectory_states"]


def _coupling(seed, n_pf, T, u_pattern=None):
    rng = np.random.default_rng(seed)
    pf_parent, pf_acc, pf_req, pf_cut, cuts = gen.bfs_prefetch_tree(T, n_pf, rng)
    pr = _inputs(T, (pf_parent, pf_acc, pf_req, pf_cut), cuts, rng, max_transitions=int(rng.integers(2, 9)))
    if u_pattern is not None:                       # forced decisions: 0 accepts, ~1 rejects
        pr.u = np.array([u_pattern[v % len(u_pattern)] for v in range(len(pf_parent))], np.float64)
        pr.max_transitions = 100
    res = oracle.presto_workload(pr)
    # sequential PowerMH: one proposal per step, drawn at the decision's own cut
    M = len(pf_parent)
    acc = {int(pf_parent[v]): v for v in range(1, M) if pf_acc[v]}
    rej = {int(pf_parent[v]): v for v in range(1, M) if not pf_acc[v]}
    lp0, lq = np.asarray(pr.root_lp0, float), np.asarray(pr.root_lq, float)
    node, k, visited = 0, 0, [0]
    while k < pr.max_transitions and node in acc and int(pf_req[acc[node]]) >= 0:
        i = int(pf_req[acc[node]])
        c = int(cuts[i])
        a, b = int(pr.suffix_off[i]), int(pr.suffix_off[i + 1])
        y_lp0 = np.concatenate([lp0[:c], pr.lp0[a:b]])
        y_lq = np.concatenate([lq[:c], pr.lq[a:b]])
        A = min(1.0, np.exp(_mh_log_ratio_eq7((lp0, lq), (y_lp0, y_lq), c, pr.alpha)))
        if pr.u[node] <= A:
            lp0, lq = y_lp0, y_lq
            node = acc[node]
        else:
            node = rej[node]
        k += 1
        visited.append(node)
    assert res["path"] == visited and res["k_delta"] == k
    st = oracle.presto_states(pr)
    np.testing.assert_allclose(st[res["path"][-1]][0], lp0, rtol=0, atol=0)
    np.testing.assert_allclose(st[res["path"][-1]][1], lq, rtol=0, atol=0)


@pytest.mark.parametrize("seed", [10086, 1, 2, 3, 4])
@pytest.mark.parametrize("n_pf,T", [(6, 12), (20, 30), (32, 64)])
def test_proposition1_coupling_with_sequential_mh(seed, n_pf, T):
    _coupling(seed, n_pf, T)


def test_proposition1_coupling_forced_decisions():
    """Decision patterns that mix acceptances and rejections at every depth, so the walk
    evaluates proposals from states reached through rejection children of accepted nodes."""
    for seed in range(6):
        for pattern in ([0.0, 1 - 1e-7], [0.0, 0.0, 1 - 1e-7], [1 - 1e-7, 0.0], [0.0, 1 - 1e-7, 1 - 1e-7]):
            _coupling(seed, 32, 64, pattern)
