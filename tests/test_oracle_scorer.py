"""Pins for the oracle's per-token scorer and greedy verification.

* log p0 and log q_tau against torch's float64 log_softmax (a different implementation),
  q_tau = p0 at tau = 1, and the tempered ratio log q_tau(i) - log q_tau(j) = (l_i - l_j)/tau;
* the entropy against torch.distributions.Categorical's, and closed forms: log V for equal
  logits, 0 for a single finite logit, the binary entropy for two finite logits;
* the argmax against numpy's first maximum, ties resolved to the smallest id;
* greedy verification (Progressive Tree Drafting, Section 3.2) is the T -> 0 limit of the
  stochastic walk: with p = softmax(l / T) at T = 1e-4 (p one-hot on the argmax up to
  exp(-gap / T)) and uniforms away from 0 and 1, the stochastic walk takes the same path
  and draws the same final token.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.scorer as osc
import oracle.verify as ov
from workloads import gen


def _rows(seed, n, V, std=3.0):
    return np.random.default_rng(seed).normal(0.0, std, (n, V))


@pytest.mark.parametrize("tau", [0.25, 0.5, 1.0, 2.0])
def test_log_probs_match_torch(tau):
    L = _rows(1, 6, 300)
    toks = np.random.default_rng(2).integers(0, 300, 6)
    for l, t in zip(L, toks):
        lp0, lq, H, am = osc.token_scores(l, int(t), tau)
        tl = torch.tensor(l, dtype=torch.float64)
        assert abs(lp0 - float(torch.log_softmax(tl, 0)[t])) < 1e-12
        assert abs(lq - float(torch.log_softmax(tl / tau, 0)[t])) < 1e-12
        if tau == 1.0:
            assert abs(lq - lp0) < 1e-12
        j = (int(t) + 7) % 300
        lqj = osc.token_scores(l, j, tau)[1]
        assert abs((lq - lqj) - (l[t] - l[j]) / tau) < 1e-10


def test_entropy_matches_torch_and_closed_forms():
    for l in _rows(3, 5, 500):
        H = osc.token_scores(l, 0, 1.0)[2]
        ref = float(torch.distributions.Categorical(logits=torch.tensor(l, dtype=torch.float64)).entropy())
        assert abs(H - ref) < 1e-11
    assert abs(osc.token_scores(np.zeros(64), 3, 1.0)[2] - np.log(64)) < 1e-12
    one = np.full(50, -np.inf)
    one[17] = 2.5
    assert osc.token_scores(one, 17, 1.0)[2] == 0.0
    two = np.full(50, -np.inf)
    two[3], two[40] = 1.3, -0.4
    p = 1.0 / (1.0 + np.exp(-(1.3 + 0.4)))
    assert abs(osc.token_scores(two, 3, 1.0)[2] - (-p * np.log(p) - (1 - p) * np.log(1 - p))) < 1e-12


def test_argmax_first_of_ties():
    l = _rows(4, 1, 1000)[0]
    assert osc.argmax_token(l) == int(np.argmax(l))
    l2 = np.zeros(10)
    l2[[3, 7]] = 5.0
    assert osc.argmax_token(l2) == 3


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("tree", ["random", "binary", "star"])
def test_greedy_is_the_zero_temperature_limit(seed, tree):
    w = gen.tree_batch(seed, B=3, prefix_len=[1, 2, 3], tree=tree, n_nodes=[15, 9, 21], Hq=1, Hkv=1, D=8,
                       dtype="f32", V=40, temperature=1.0, max_depth=4)
    # make some children carry their parent's argmax, so paths go deeper than one step
    rng = np.random.default_rng(seed)
    for b in range(w.B):
        s, e = int(w.node_offsets[b]), int(w.node_offsets[b + 1])
        for v in range(e - s):
            kids = [c for c in range(s + 1, e) if int(w.parent[c]) == v]
            if kids and rng.random() < 0.7:
                a = osc.argmax_token(np.asarray(w.logits[s + v], np.float64))
                c = kids[int(rng.integers(0, len(kids)))]
                for k in kids:
                    if k != c and int(w.token[k]) == a:
                        w.token[k] = int(w.token[c])
                w.token[c] = a
    w.uniforms = np.clip(w.uniforms, 0.01, 0.99).astype(np.float32)
    w.temperature = np.zeros(w.B, np.float32)
    greedy = oracle.verify_workload(w)
    w.temperature = np.full(w.B, 1e-4, np.float32)
    cold = oracle.verify_workload(w)
    for g, c in zip(greedy, cold):
        assert g["path"] == c["path"] and g["bonus"] == c["bonus"]
        np.testing.assert_array_equal(g["status"], c["status"])
