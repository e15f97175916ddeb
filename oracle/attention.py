"""Tree-masked attention over a paged prefix plus the node's own ancestors.

Progressive Tree Drafting, Section 3.1 ("Tree Construction") and Section 3.2
("Candidate Verification"): each node attends only to pi(v) (itself and its
ancestors) in front of the shared context; RheoSampling (Section 2.1) and PreSTO
(Section 3.2, "Batched proposal sampling"; Appendix B.3, Example 4) score such
trees / suffix batches in one forward pass that reuses the cached prefix KV.

The pages give no attention formula, so this is the standard scaled dot-product
attention, evaluated exactly in float64:

  keys/values of node v, KV head g = floor(h / G):
     prefix rows r = 0 .. L_b - 1 (row r lives in physical block
       block_table[b][r // block_size], slot r % block_size; the key cache is
       stored [block, head, slot, d] and the value cache [block, head, d, slot]),
     then the nodes of pi(v) from the root down to v;
  s_j = scale * <q_v,h , k_j>,  w_j = exp(s_j - max s),
  out = sum_j w_j v_j / sum_j w_j,  lse = max s + log sum_j w_j.
"""

from __future__ import annotations

import numpy as np

from .tree import tree_prep


def _f64(arr, dtype):
    if dtype == "bf16":
        a = np.ascontiguousarray(arr, dtype=np.uint16).astype(np.uint32) << 16
        return a.view(np.float32).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def prefix_rows(w, b: int, g: int):
    """Keys and values of prefix rows 0..L_b-1 of KV head g, gathered through the block table."""
    L = int(w.prefix_len[b])
    bs = w.block_size
    nblk = (L + bs - 1) // bs
    blocks = np.asarray(w.block_table[b, :nblk], dtype=np.int64)
    if nblk and (blocks.min() < 0 or blocks.max() >= w.k_cache.shape[0]):
        raise ValueError("block table entry out of range")
    K = _f64(w.k_cache[blocks, g], w.dtype).reshape(-1, w.D)[:L]
    V = _f64(w.v_cache[blocks, g], w.dtype).transpose(0, 2, 1).reshape(-1, w.D)[:L]
    return K, V


def node_attention(q_rows, K, V, scale):
    """Exact attention of the query rows q_rows [G, D] over keys K and values V [n, D]."""
    s = scale * (q_rows @ K.T)                    # [G, n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    out = (e @ V) / den
    lse = m[:, 0] + np.log(den[:, 0])
    return out, lse


def tree_attention(w, nodes=None, prep=None):
    """Attention output [len(nodes), Hq, D] and log-sum-exp [len(nodes), Hq] (float64)."""
    if nodes is None:
        nodes = range(w.N)
    nodes = [int(v) for v in nodes]
    seq_of = np.searchsorted(np.asarray(w.node_offsets), np.arange(w.N), side="right") - 1
    if prep is None:
        prep = tree_prep(w.parent, w.node_offsets, w.prefix_len, sorted({int(seq_of[v]) for v in nodes}))
    G = w.G
    out = np.zeros((len(nodes), w.Hq, w.D), dtype=np.float64)
    lse = np.zeros((len(nodes), w.Hq), dtype=np.float64)
    by_seq = {}
    for i, v in enumerate(nodes):
        by_seq.setdefault(int(seq_of[v]), []).append((i, v))
    for b, items in by_seq.items():
        off = int(w.node_offsets[b])
        for g in range(w.Hkv):
            Kp, Vp = prefix_rows(w, b, g)
            for i, v in items:
                anc = off + np.asarray(prep["anc"][v], dtype=np.int64)
                K = np.concatenate([Kp, _f64(w.k_node[anc, g], w.dtype)], axis=0)
                V = np.concatenate([Vp, _f64(w.v_node[anc, g], w.dtype)], axis=0)
                qg = _f64(w.q[v, g * G:(g + 1) * G], w.dtype)
                o, l = node_attention(qg, K, V, w.sm_scale)
                out[i, g * G:(g + 1) * G] = o
                lse[i, g * G:(g + 1) * G] = l
    return out, lse
