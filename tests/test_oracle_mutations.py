"""Mutation run over the oracle: each plausible mistake, planted in a copy of one oracle
module, must make at least one pin fail.

A mutation replaces one snippet of an oracle module's source; the mutated module's
functions then stand in for the originals everywhere (the oracle package, its other
modules and the test modules that imported them) while the pins run, and are restored
afterwards.  The unmutated oracle passes every pin (checked first).  The mistakes
cover the temperature (ignored, multiplied, applied to one statistic only), the
accept ratio, the residual and its normaliser, the sequential rejection's zeroing
and renormalisation, the inverse-CDF side, the terminal statistics, the visibility
sets, the attention scale and key set, PreSTO's log-acceptance, state inheritance
and walk, the per-token scorer and greedy verification, the prefetching tree (the
cut generator, Condition 1, deferral, Equations 10, 11 and 14) and the draft-tree
builder (the sampled token's proxy, the tail off the leads).
"""

import contextlib
import inspect
import sys
import types

import pytest

import oracle
import oracle.attention
import oracle.draft_tree
import oracle.prefetch
import oracle.presto
import oracle.scorer
import oracle.tree
import oracle.verify

import test_oracle_draft_tree as tdt
import test_oracle_prefetch as tpf
import test_oracle_presto as tp
import test_oracle_scorer as tsc
import test_oracle_softmax_pins as ts
import test_oracle_tree_attention as ta
import test_oracle_verify as tv


def _mutated_module(mod, old, new, occurrence):
    src = inspect.getsource(mod)
    at = -1
    for _ in range(occurrence + 1):
        at = src.find(old, at + 1)
        assert at >= 0, f"snippet not found in {mod.__name__}: {old!r} (occurrence {occurrence})"
    m = types.ModuleType(mod.__name__)
    m.__package__ = mod.__package__
    m.__file__ = mod.__file__
    exec(compile(src[:at] + new + src[at + len(old):], mod.__file__, "exec"), m.__dict__)
    return m


@contextlib.contextmanager
def planted(mod, old, new, occurrence=0):
    m = _mutated_module(mod, old, new, occurrence)
    swaps = {}
    for name, obj in vars(mod).items():
        if getattr(obj, "__module__", None) == mod.__name__ and hasattr(m, name):
            swaps[id(obj)] = (obj, getattr(m, name))
    undo = []
    for mname, module in list(sys.modules.items()):
        if module is None or not (mname == "oracle" or mname.startswith("oracle.") or mname.startswith("test_")):
            continue
        for attr, val in list(vars(module).items()):
            if id(val) in swaps and swaps[id(val)][0] is val:
                undo.append((module, attr, val))
                setattr(module, attr, swaps[id(val)][1])
    try:
        yield
    finally:
        for module, attr, val in undo:
            setattr(module, attr, val)


PINS = [
    ("softmax vs torch", ts.pin_softmax_matches_torch),
    ("softmax pair ratios", ts.pin_softmax_pair_ratios),
    ("softmax scale invariance", ts.pin_softmax_scale_invariance_and_limits),
    ("terminal normaliser", ts.pin_terminal_stats_normaliser),
    ("terminal residual mass", ts.pin_terminal_stats_residual_mass),
    ("terminal draw", ts.pin_terminal_draw_in_torch_cdf_step),
    ("walk uses tempered p", ts.pin_walk_uses_tempered_target),
    ("one-layer lossless", lambda: tv.test_one_layer_lossless(0, 3, 1, 3)),
    ("one-layer lossless m=0", lambda: tv.test_one_layer_lossless(1, 4, 0, 4)),
    ("theorem 3", lambda: tv.test_acceptance_matches_theorem3(0, 3, 1)),
    ("sequential rejection", tv.test_sequential_rejection_selects_with_target_probability),
    ("two-layer lossless", lambda: tv.test_two_layer_lossless_with_global_pruning(0, 5)),
    ("q~ = p accepts", tv.test_qtilde_equal_to_p_always_accepts_sampled_child),
    ("speculative sampling", tv.test_chain_of_sampled_children_is_speculative_sampling),
    ("one-hot target", tv.test_one_hot_target_selects_that_child),
    ("inverse cdf", tv.test_inverse_cdf_small_cases),
    ("terminal = walk end", tv.test_terminal_stats_agree_with_walk_end),
    ("transitive closure", lambda: ta.test_visibility_is_transitive_closure(1)),
    ("chain = causal", lambda: ta.test_chain_equals_causal_attention(10086, "f32")),
    ("node = its path", lambda: ta.test_each_node_equals_attention_over_its_path(2, "random")),
    ("single key", ta.test_single_key_returns_its_value),
    ("eq 6 = eq 7", lambda: tp.test_equation6_equals_equation7(1)),
    ("symmetric cases", tp.test_identical_proposal_and_symmetric_cases),
    ("example 5", tp.test_example5_walk_golden),
    ("proposition 1", lambda: tp.test_proposition1_coupling_with_sequential_mh(1, 20, 30)),
    ("proposition 1, forced decisions", tp.test_proposition1_coupling_forced_decisions),
    ("truncated draft lossless", lambda: tv.test_one_layer_lossless_with_truncated_draft(0, 3, 1, 3, 3)),
    ("scorer vs torch", lambda: tsc.test_log_probs_match_torch(0.25)),
    ("scorer entropy", tsc.test_entropy_matches_torch_and_closed_forms),
    ("argmax first of ties", tsc.test_argmax_first_of_ties),
    ("greedy = T -> 0 limit", lambda: tsc.test_greedy_is_the_zero_temperature_limit(0, "random")),
    ("splitmix64 outputs", tpf.test_splitmix64_known_outputs),
    ("example 2 BFS", tpf.test_example2_bfs_golden),
    ("BFS deferral", tpf.test_bfs_deferral),
    ("lemma 1 = lemma 2 = traversal", lambda: tpf.test_lemma1_equals_lemma2_equals_traversal(0, "bfs", 0.01)),
    ("equation 10", tpf.test_equation10_rounding),
    ("equation 14 = lemma 3 midpoint", tpf.test_equation14_is_lemma3_midpoint),
    ("proposition 2", lambda: tpf.test_proposition2_dp_is_brute_force_optimum(0, 3, 5)),
    ("rheo table 1", tdt.test_table1_golden),
    ("lemma 4", lambda: tdt.test_lemma4_sampled_proxy_above_fills(0, 1, 20)),
    ("lemma 5", lambda: tdt.test_lemma5_scores_fall_and_prune_is_ancestor_closed(0)),
    ("draft tree lossless", lambda: tdt.test_theorem1_one_layer_lossless(0, 3, 1, 3, 6)),
]

V, A, T, P = oracle.verify, oracle.attention, oracle.tree, oracle.presto
S, PF, DT = oracle.scorer, oracle.prefetch, oracle.draft_tree
TEMP_LINE = "z = np.asarray(logits_row, dtype=np.float64) / float(temperature)"

MUTATIONS = {
    # temperature
    "T ignored in target_probs": (V, TEMP_LINE, "z = np.asarray(logits_row, dtype=np.float64)", 0),
    "l * T in target_probs": (V, TEMP_LINE, "z = np.asarray(logits_row, dtype=np.float64) * float(temperature)", 0),
    "T ignored in terminal stats": (V, TEMP_LINE, "z = np.asarray(logits_row, dtype=np.float64)", 1),
    "l * T in terminal stats": (V, TEMP_LINE, "z = np.asarray(logits_row, dtype=np.float64) * float(temperature)", 1),
    "T squared in target_probs": (V, TEMP_LINE, "z = np.asarray(logits_row, dtype=np.float64) / float(temperature) ** 2", 0),
    # verification walk
    "accept ratio inverted": (V, "min(1.0, p[ts] / qt[ts])", "min(1.0, qt[ts] / p[ts])", 0),
    "residual sign": (V, "r = _normalise(np.maximum(0.0, p - qt))", "r = _normalise(np.maximum(0.0, qt - p))", 0),
    "residual not clamped": (V, "r = _normalise(np.maximum(0.0, p - qt))", "r = _normalise(np.abs(p - qt))", 0),
    "rejected token kept": (V, "r[int(token[c])] = 0.0", "pass", 0),
    "no renormalisation after rejection": (V, "                r = _normalise(r)\n", "", 0),
    "inverse cdf left side": (V, 'side="right"', 'side="left"', 0),
    # terminal statistics
    "Z from the wrong side": (V, "resid = np.maximum(0.0, p - np.asarray(qtilde, dtype=np.float64))",
                              "resid = np.maximum(0.0, np.asarray(qtilde, dtype=np.float64) - p)", 0),
    "Z without clamp": (V, "Z = float(resid.sum())", "Z = float((p - np.asarray(qtilde)).sum())", 0),
    "Z sign": (V, "Z = float(resid.sum())", "Z = -float(resid.sum())", 0),
    "deterministic tokens kept in final draw": (V, "        r[int(t)] = 0.0", "        pass", 0),
    "M not the maximum": (V, "M = float(z.max())", "M = float(z.mean())", 0),
    # visibility and attention
    "self key dropped": (T, "path = [v]", "path = [v] if v == 0 else []", 0),
    "only the parent kept": (T, "            p = int(parent_local[p])\n", "            p = -1\n", 0),
    "depth off by one": (T, "depth[v] = len(path) - 1", "depth[v] = len(path)", 0),
    "scale dropped": (A, "s = scale * (q_rows @ K.T)", "s = q_rows @ K.T", 0),
    "wrong KV head": (A, "Kp, Vp = prefix_rows(w, b, g)", "Kp, Vp = prefix_rows(w, b, 0)", 0),
    "lse without the maximum": (A, "lse = m[:, 0] + np.log(den[:, 0])", "lse = np.log(den[:, 0])", 0),
    # PreSTO
    "log A proposal terms swapped": (P, "log_q_x - log_q_y", "log_q_y - log_q_x", 0),
    "log A sums from the cut token": (P, "log_q_x = x[1][c:].sum()", "log_q_x = x[1][c - 1:].sum()", 0),
    "log A not clamped": (P, "logA[i] = min(0.0, ", "logA[i] = (", 0),
    "rejection child takes the root state": (P, "states[v] = states[par]", "states[v] = states[0]", 0),
    "walk direction inverted": (P, "go = uu <= A", "go = uu > A", 0),
    # per-token scorer and greedy verification
    "scorer: tau ignored": (S, "z = l / float(tau)", "z = l", 0),
    "scorer: entropy sign": (S, "H = float(-np.sum(p[nz] * np.log(p[nz])))", "H = float(np.sum(p[nz] * np.log(p[nz])))", 0),
    "scorer: last of equal maxima": (S, "int(np.flatnonzero(l == l.max())[0])", "int(np.flatnonzero(l == l.max())[-1])", 0),
    "scorer: log p0 with the tempered normaliser": (S, "lp0 = float(l[token]) - _lse(l)", "lp0 = float(l[token]) - _lse(l / float(tau))", 0),
    "greedy: sampled child always accepted": (V, "hit = int(token[c]) == a", "hit = bool(sampled[c]) or int(token[c]) == a", 0),
    # prefetching tree
    "splitmix64 finaliser shift": (PF, "return z ^ (z >> 31)", "return z ^ (z >> 30)", 0),
    "condition 1 inverted": (PF, "if cut[a] <= cut[v]:", "if cut[a] >= cut[v]:", 0),
    "deferred request's sibling dropped": (PF, "queue.append(r)", "pass", 0),
    "equation 14 sign": (PF, "return 0.5 * (1.0 + P[ACCEPT] - P[REJECT])", "return 0.5 * (1.0 - P[ACCEPT] + P[REJECT])", 0),
    "equation 10 never rounds down": (PF, "if A <= eps:", "if A < 0.0:", 0),
    "rejection child's reaching weight": (PF, "R[v] = R[p] * (h if is_accept[v] else 1.0 - h)", "R[v] = R[p] * (h if is_accept[v] else h)", 0),
    # draft-tree builder
    "sampled token's proxy = its own q": (DT, "proxy = min(float(q[m - 1]), zres) if m > 0 else float(q[0]) + self.eps",
                                          "proxy = float(q[list(keep).index(y)])", 0),
    "leads left in the sampling tail": (DT, "tail[:m] = 0.0", "pass", 0),
}


def _failing_pins():
    failed = []
    for name, pin in PINS:
        try:
            pin()
        except Exception:  # an assertion, or an error the mistake provokes
            failed.append(name)
            break
    return failed


def test_unmutated_oracle_passes_every_pin():
    for name, pin in PINS:
        pin()


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_mutation_fails_a_pin(mutation):
    mod, old, new, occ = MUTATIONS[mutation]
    with planted(mod, old, new, occ):
        failed = _failing_pins()
    assert failed, f"no pin fails when '{mutation}' is planted"
