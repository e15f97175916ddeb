"""Pins for the oracle's temperature softmax and per-node terminal statistics.

The target distribution at a node is p = softmax(l / T) (RheoSampling, Section
5.4: the temperature enters only sampling and verification).  These checks rest
on mathematics the oracle does not share with itself:

* torch's own float64 softmax of l / T (a different implementation);
* the ratio p_i / p_j = exp((l_i - l_j) / T) for every pair, which fixes both
  the direction of the temperature (divide, not multiply) and its value;
* invariance under (l, T) -> (c l, c T), and the limits T -> infinity (uniform)
  and T -> 0 (all mass on the largest logit);
* for the terminal statistics M, S, Z: M is the largest tempered logit,
  exp(l / T - M) / S is a distribution equal to torch's softmax, and Z equals
  the other side of RheoSampling's residual identity (Appendix C, Equation 10),
  sum (q~ - p)+ = 1 - sum min(p, q~), computed from torch's p;
* the terminal draw lies in the step of torch's cumulative residual (with the
  deterministic children's tokens removed) that contains u.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.verify as ov

TEMPS = [0.35, 0.7, 1.0, 1.9]


def _logits(seed, V, std=3.0):
    return np.random.default_rng(seed).normal(0.0, std, V)


def _torch_p(l, T):
    return torch.softmax(torch.tensor(l, dtype=torch.float64) / T, dim=0).numpy()


def pin_softmax_matches_torch():
    for seed, T in enumerate(TEMPS):
        l = _logits(seed, 97)
        p = ov.target_probs(l, T)
        np.testing.assert_allclose(p, _torch_p(l, T), rtol=1e-12, atol=1e-15)
        assert abs(p.sum() - 1.0) < 1e-12


def pin_softmax_pair_ratios():
    for seed, T in enumerate(TEMPS):
        l = _logits(10 + seed, 40, std=1.5)
        p = ov.target_probs(l, T)
        i, j = np.meshgrid(np.arange(40), np.arange(40), indexing="ij")
        np.testing.assert_allclose(p[i] / p[j], np.exp((l[i] - l[j]) / T), rtol=1e-10)


def pin_softmax_scale_invariance_and_limits():
    l = _logits(3, 64)
    for c in (0.5, 3.0, 11.0):
        np.testing.assert_allclose(ov.target_probs(c * l, c * 0.8), ov.target_probs(l, 0.8),
                                   rtol=1e-11, atol=1e-16)
    np.testing.assert_allclose(ov.target_probs(l, 1e12), np.full(64, 1 / 64), rtol=1e-9)
    cold = ov.target_probs(l, 1e-3)
    assert int(np.argmax(cold)) == int(np.argmax(l)) and cold.max() > 1 - 1e-12


def _qtilde(seed, V, support=None):
    r = np.random.default_rng(seed)
    q = r.gamma(0.6, size=V) + 1e-4
    if support is not None:
        keep = r.choice(V, size=support, replace=False)
        mask = np.zeros(V, bool)
        mask[keep] = True
        q = np.where(mask, q, 0.0)
    return q / q.sum()


def pin_terminal_stats_normaliser():
    for seed, T in enumerate(TEMPS):
        l = _logits(20 + seed, 300)
        M, S, Z, tok, _ = ov.node_terminal_stats(l, T, None, [], 0.37)
        assert abs(M - l.max() / T) < 1e-12 * max(1.0, abs(M))
        p = np.exp(l / T - M) / S
        np.testing.assert_allclose(p, _torch_p(l, T), rtol=1e-11, atol=1e-15)
        assert Z == 0.0


def pin_terminal_stats_residual_mass():
    for seed, T in enumerate(TEMPS):
        l = _logits(30 + seed, 300)
        for support in (None, 17):
            qt = _qtilde(40 + seed, 300, support)
            M, S, Z, tok, _ = ov.node_terminal_stats(l, T, qt, [], 0.5)
            p = _torch_p(l, T)
            other_side = np.maximum(qt - p, 0.0).sum()
            assert abs(Z - other_side) < 1e-12
            assert abs(Z - (1.0 - np.minimum(p, qt).sum())) < 1e-12


def pin_terminal_draw_in_torch_cdf_step():
    V = 200
    for seed, T in enumerate(TEMPS):
        l = _logits(50 + seed, V)
        qt = _qtilde(60 + seed, V, 31 if seed % 2 else None)
        det = [int(t) for t in np.argsort(-l)[:3]]
        p = torch.softmax(torch.tensor(l, dtype=torch.float64) / T, dim=0)
        for use_q in (False, True):
            w = torch.clamp(p - torch.tensor(qt), min=0.0) if use_q else p.clone()
            w[det] = 0.0
            F = torch.cumsum(w, 0) / w.sum()
            for u in np.linspace(0.001, 0.999, 23):
                _, _, _, tok, _ = ov.node_terminal_stats(l, T, qt if use_q else None, det, u)
                lo = float(F[tok - 1]) if tok > 0 else 0.0
                assert float(w[tok]) > 0.0 and lo - 1e-12 <= u < float(F[tok]) + 1e-12, (tok, u)


def pin_walk_uses_tempered_target():
    """One deterministic child: it is accepted iff u <= p(child) with p = softmax(l / T)."""
    from workloads import gen

    V = 50
    for seed, T in enumerate(TEMPS):
        w = gen.tree_batch(70 + seed, B=1, prefix_len=[1], tree="star", n_nodes=[2], Hq=1, Hkv=1,
                           D=8, dtype="f32", V=V, temperature=T)
        w.sampled[:] = 0
        w.draft_row[:] = -1
        p = _torch_p(np.asarray(w.logits[0], np.float64), T)
        for u in (0.01, 0.2, 0.6):
            w.uniforms[1, 0] = u
            res = oracle.verify_workload(w)[0]
            assert (len(res["path"]) > 1) == (u <= p[int(w.token[1])])


PINS = [pin_softmax_matches_torch, pin_softmax_pair_ratios, pin_softmax_scale_invariance_and_limits,
        pin_terminal_stats_normaliser, pin_terminal_stats_residual_mass,
        pin_terminal_draw_in_torch_cdf_step, pin_walk_uses_tempered_target]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
