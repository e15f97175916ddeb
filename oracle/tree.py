"""Tree visibility sets, depths and positions.

Progressive Tree Drafting, Section 3.1 ("Tree Construction"): every node v has a
unique parent P(v); the set of nodes v may attend to is pi(v) = {v} U pi(P(v)),
and v's positional index is determined by |pi(v)|.  With a cached prefix of L
rows in front of the tree, the node's position is L + |pi(v)| - 1 = L + depth(v)
(0-based).
"""

from __future__ import annotations

import numpy as np


class TreeError(ValueError):
    pass


def _seq_prep(parent_local: np.ndarray, prefix_len: int):
    n = len(parent_local)
    if n == 0:
        raise TreeError("empty sequence")
    if int(parent_local[0]) != -1:
        raise TreeError("node 0 must be the root (parent -1)")
    for v in range(1, n):
        p = int(parent_local[v])
        if not (0 <= p < v):
            raise TreeError(f"node {v}: parent {p} is not an earlier node")
    # pi(v) = {v} U pi(P(v)), built by following parent pointers to the root
    anc = []
    depth = np.zeros(n, dtype=np.int64)
    for v in range(n):
        path = [v]
        p = int(parent_local[v])
        while p != -1:
            path.append(p)
            p = int(parent_local[p])
        path.reverse()                       # root ... v
        anc.append(path)
        depth[v] = len(path) - 1             # |pi(v)| - 1
    pos = prefix_len + depth
    is_chain = all(int(parent_local[v]) == v - 1 for v in range(1, n))
    return depth, pos, anc, is_chain


def tree_prep(parent: np.ndarray, node_offsets: np.ndarray, prefix_len: np.ndarray, seqs=None):
    """Per-node depth and position and the visibility set of every node.

    Returns a dict with ``depth`` [N], ``pos`` [N], ``anc`` (list, per node, of
    the sequence-local ids of pi(v) from the root down to v) and ``is_chain``
    [B] (True when every node's parent is the node just before it, i.e. the
    tree is a path and the mask is ordinary causal attention).  With ``seqs``
    only those sequences are prepared (the others' entries stay empty).
    """
    B = len(node_offsets) - 1
    N = int(node_offsets[-1])
    depth = np.zeros(N, dtype=np.int64)
    pos = np.zeros(N, dtype=np.int64)
    anc = [None] * N
    is_chain = np.zeros(B, dtype=bool)
    for b in (range(B) if seqs is None else seqs):
        s, e = int(node_offsets[b]), int(node_offsets[b + 1])
        d, p, a, ch = _seq_prep(np.asarray(parent[s:e]), int(prefix_len[b]))
        depth[s:e] = d
        pos[s:e] = p
        anc[s:e] = a
        is_chain[b] = ch
    return {"depth": depth, "pos": pos, "anc": anc, "is_chain": is_chain}


def ancestor_words(anc_local, nwords: int = 4) -> np.ndarray:
    """Bit j of the result is set iff sequence-local node j is in pi(v)."""
    words = np.zeros(nwords, dtype=np.uint64)
    for j in anc_local:
        words[j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return words
