"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (tav_tree_attention and tav_tree_verify on two streams).

The oracle computes sampled outputs one by one: the attention of a few nodes
per sequence (every sequence of c3, first and last row blocks of c5, requests
of every length in c4), the verification walk of every sequence, and the
vocabulary statistics of sampled nodes.  Same tolerances as the small cases.
"""

import sys

import numpy as np
import pytest

from workloads import gen
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _sample_nodes(w, per_seq, seed):
    rng = np.random.default_rng(seed)
    out = []
    for b in range(w.B):
        nodes = list(w.seq_nodes(b))
        pick = {nodes[0], nodes[-1]}
        pick.update(int(x) for x in rng.choice(nodes, size=min(per_seq, len(nodes)), replace=False))
        out.extend(sorted(pick))
    return out


@pytest.mark.parametrize("name,per_seq", [("c2", 60), ("c3", 4), ("c5", 5)])
def test_full_size_tree_configs(name, per_seq):
    _say("full", name)
    w = gen.make(name, 10086)
    got = gu.run(w, split_calls=True, max_path=64)
    assert got["status"] == 0, got["status"]
    gu.check_tree_prep(w, got)
    nodes = _sample_nodes(w, per_seq, 1)
    err = gu.check_attention(w, got, nodes)
    _say(name, "attention max abs err", err, "over", len(nodes), "nodes")
    flagged = gu.check_verify(w, got)
    _say(name, "walks ok; near-tie flags", flagged)
    gu.check_node_stats(w, got, _sample_nodes(w, 2, 2))


def test_full_size_presto():
    _say("full c4")
    w = gen.make("c4", 10086)
    got = gu.run(w, split_calls=True)
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
