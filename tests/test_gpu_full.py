"""GPU parity at the five workloads' full sizes, seeds 10086, 1 and 2.

The main mode is the benchmark's launch configuration: one tav_tree_attn_verify call
on one stream (tree preparation, attention, merge, vocabulary workers and walk); the
split mode (tav_tree_prep, tav_tree_attention and tav_tree_verify / tav_presto_accept
on two streams with their own workspaces) runs at seed 10086.

The oracle computes sampled outputs one by one: the attention of a few nodes per
sequence (every sequence of the batched-verify workload, first and last row blocks of
the long-context one, requests of every length in the PreSTO batch), the verification
walk of every sequence decision by decision, and the vocabulary statistics of sampled
nodes.  Same tolerances as the small cases.
"""

import sys

import numpy as np
import pytest

from workloads import gen
import gpu_util as gu

pytestmark = pytest.mark.gpu

SEEDS = [10086, 1, 2]
_cache = {}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _workload(name, seed):
    key = (name, seed)
    if key not in _cache:
        _cache.clear()                 # one full-size workload in host memory at a time
        _cache[key] = gen.make(name, seed)
    return _cache[key]


def _sample_nodes(w, per_seq, seed):
    rng = np.random.default_rng(seed)
    out = []
    for b in range(w.B):
        nodes = list(w.seq_nodes(b))
        pick = {nodes[0], nodes[-1]}
        pick.update(int(x) for x in rng.choice(nodes, size=min(per_seq, len(nodes)), replace=False))
        out.extend(sorted(pick))
    return out


PER_SEQ = {"c2": 60, "c3": 4, "c5": 5}
TREE_CASES = [(n, s, False) for n in ("c2", "c3", "c5") for s in SEEDS] + \
             [(n, 10086, True) for n in ("c2", "c3", "c5")]


@pytest.mark.parametrize("name,seed,split", TREE_CASES)
def test_full_size_tree_configs(name, seed, split):
    _say("full", name, "seed", seed, "split calls" if split else "one call")
    w = _workload(name, seed)
    got = gu.run(w, split_calls=split, max_path=64)
    assert got["status"] == 0, got["status"]
    gu.check_tree_prep(w, got)
    nodes = _sample_nodes(w, PER_SEQ[name], seed)
    err = gu.check_attention(w, got, nodes)
    _say(name, "attention max abs err", err, "over", len(nodes), "nodes")
    flagged = gu.check_verify(w, got)
    _say(name, "walks ok; near-tie flags", flagged)
    gu.check_node_stats(w, got, _sample_nodes(w, 2, seed + 1))


@pytest.mark.parametrize("seed,split", [(s, False) for s in SEEDS] + [(10086, True)])
def test_full_size_presto(seed, split):
    _say("full c4 seed", seed, "split calls" if split else "one call")
    w = _workload("c4", seed)
    got = gu.run(w, split_calls=split)
    assert got["status"] == 0, got["status"]
    gu.check_presto(w, got)
    lens = np.diff(w.node_offsets)
    order = np.argsort(lens)
    picks = []
    for b in [int(order[0]), int(order[len(order) // 2]), int(order[-1])]:
        s, e = int(w.node_offsets[b]), int(w.node_offsets[b + 1])
        picks += sorted({s, (s + e) // 2, e - 1})
    err = gu.check_attention(w, got, picks)
    _say("c4 attention max abs err", err, "over", len(picks), "query tokens")


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_full_size_sparse_draft(name):
    """The batched-verify and long-context workloads with sparse top-128 draft rows."""
    _say("full sparse", name)
    _cache.clear()
    w = gen.make(name, 10086, draft_support=128)
    got = gu.run(w, max_path=64)
    assert got["status"] == 0, got["status"]
    flagged = gu.check_verify(w, got)
    _say(name, "sparse walks ok; near-tie flags", flagged)
    gu.check_node_stats(w, got, _sample_nodes(w, 3, 7))
    gu.check_attention(w, got, _sample_nodes(w, 1, 8))
