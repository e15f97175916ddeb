"""Pins for the oracle's visibility sets and tree-masked attention.

Each check rests on something other than the oracle's own formula:
  * visibility sets against the transitive closure of the parent relation
    (computed by boolean matrix powers) -- Progressive Tree Drafting, Section 3.1;
  * a path-shaped tree against ordinary causal attention over prefix + path,
    computed by torch's scaled_dot_product_attention in float64;
  * every node against attention over its own materialised path sequence, the
    path found here by walking parent pointers;
  * one-key cases, node relabelling and paged-vs-contiguous layouts.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import prefix_rows
from oracle.tree import TreeError
from workloads import gen


def _closure(parent):
    n = len(parent)
    A = np.zeros((n, n), dtype=bool)            # A[v, p] = p is the parent of v
    for v in range(1, n):
        A[v, parent[v]] = True
    R = np.eye(n, dtype=bool)
    P = np.eye(n, dtype=bool)
    for _ in range(n):
        P = (P.astype(np.int64) @ A.astype(np.int64)) > 0
        R |= P
    return R                                     # R[v, j] = j is v or an ancestor of v


@pytest.mark.parametrize("seed", [10086, 1, 2])
def test_visibility_is_transitive_closure(seed):
    rng = np.random.default_rng(seed)
    for n in [1, 2, 7, 40, 130]:
        parent = gen.random_depth_parents(n, 9, rng)
        prep = oracle.tree_prep(parent, np.array([0, n]), np.array([5]))
        R = _closure(parent)
        for v in range(n):
            assert sorted(prep["anc"][v]) == list(np.nonzero(R[v])[0])
            assert prep["depth"][v] == R[v].sum() - 1
            assert prep["pos"][v] == 5 + R[v].sum() - 1
            words = oracle.ancestor_words(prep["anc"][v], 4)
            bits = [j for j in range(256) if (int(words[j // 64]) >> (j % 64)) & 1]
            assert bits == list(np.nonzero(R[v])[0])


def test_chain_detection_and_lower_triangular_mask():
    parent = gen.chain_parents(9)
    prep = oracle.tree_prep(parent, np.array([0, 9]), np.array([0]))
    assert prep["is_chain"][0]
    for v in range(9):
        assert prep["anc"][v] == list(range(v + 1))
    tree = gen.complete_binary_parents(7)
    assert not oracle.tree_prep(tree, np.array([0, 7]), np.array([0]))["is_chain"][0]


@pytest.mark.parametrize("bad", [[0, 0], [-1, 1], [-1, 2, 0], [-1, -1]])
def test_invalid_parent_arrays_rejected(bad):
    with pytest.raises(TreeError):
        oracle.tree_prep(np.array(bad, np.int32), np.array([0, len(bad)]), np.array([0]))


def _small(seed, tree, dtype, n_nodes=(1, 9, 20), prefix=(0, 37, 70), Hq=4, Hkv=2, D=16,
           shuffle=True):
    return gen.tree_batch(seed, B=len(n_nodes), prefix_len=list(prefix), tree=tree,
                          n_nodes=list(n_nodes), Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                          shuffle_blocks=shuffle)


def _sdpa(q, K, V, mask, scale):
    """torch scaled_dot_product_attention in float64 on the CPU."""
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        attn_mask=torch.from_numpy(mask)[None], scale=scale)
    return o[0].numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seed", [10086, 1])
def test_chain_equals_causal_attention(seed, dtype):
    w = _small(seed, "chain", dtype, n_nodes=(13, 5), prefix=(21, 0))
    out, lse = oracle.tree_attention(w)
    for b in range(w.B):
        s, e = int(w.node_offsets[b]), int(w.node_offsets[b + 1])
        n, L = e - s, int(w.prefix_len[b])
        for g in range(w.Hkv):
            Kp, Vp = prefix_rows(w, b, g)
            K = np.concatenate([Kp, gen.as_f64(w.k_node[s:e, g], dtype)])
            V = np.concatenate([Vp, gen.as_f64(w.v_node[s:e, g], dtype)])
            # query i (chain position i) sees the whole prefix and chain positions <= i
            mask = np.arange(L + n)[None, :] <= (L + np.arange(n))[:, None]
            for h in range(g * w.G, (g + 1) * w.G):
                q = gen.as_f64(w.q[s:e, h], dtype)
                ref = _sdpa(q, K, V, mask, w.sm_scale)
                np.testing.assert_allclose(out[s:e, h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tree", ["random", "binary"])
@pytest.mark.parametrize("seed", [10086, 2])
def test_each_node_equals_attention_over_its_path(seed, tree):
    w = _small(seed, tree, "bf16")
    out, lse = oracle.tree_attention(w)
    for b in range(w.B):
        s, e = int(w.node_offsets[b]), int(w.node_offsets[b + 1])
        L = int(w.prefix_len[b])
        for v in range(s, e):
            path = []                            # follow parent pointers to the root
            x = v - s
            while x != -1:
                path.append(s + x)
                x = int(w.parent[s + x])
            path = path[::-1]
            for g in range(w.Hkv):
                # the prefix rows, read block by block in logical order
                rows_k, rows_v = [], []
                for r in range(L):
                    blk = int(w.block_table[b, r // w.block_size])
                    rows_k.append(gen.as_f64(w.k_cache[blk, g, r % w.block_size], "bf16"))
                    rows_v.append(gen.as_f64(w.v_cache[blk, g, :, r % w.block_size], "bf16"))
                K = np.array(rows_k + [gen.as_f64(w.k_node[p, g], "bf16") for p in path])
                V = np.array(rows_v + [gen.as_f64(w.v_node[p, g], "bf16") for p in path])
                for h in range(g * w.G, (g + 1) * w.G):
                    q = gen.as_f64(w.q[v, h], "bf16")
                    s_ = w.sm_scale * K @ q
                    m = s_.max()
                    p_ = np.exp(s_ - m)
                    ref = p_ @ V / p_.sum()
                    np.testing.assert_allclose(out[v, h], ref, rtol=1e-12, atol=1e-12)
                    assert abs(lse[v, h] - (m + math.log(p_.sum()))) < 1e-12


def test_single_key_returns_its_value():
    w = _small(3, "random", "f32", n_nodes=(1, 1), prefix=(0, 0))
    out, lse = oracle.tree_attention(w)
    for v in range(w.N):
        for h in range(w.Hq):
            np.testing.assert_array_equal(out[v, h], w.v_node[v, h // w.G].astype(np.float64))
            s_ = w.sm_scale * float(np.dot(w.q[v, h].astype(np.float64),
                                          w.k_node[v, h // w.G].astype(np.float64)))
            assert abs(lse[v, h] - s_) < 1e-12


def test_relabelling_permutes_outputs():
    w = _small(7, "random", "f32", n_nodes=(25,), prefix=(19,))
    out, _ = oracle.tree_attention(w)
    n = w.N
    rng = np.random.default_rng(0)
    # a random topological relabelling: new order keeps parents before children
    order = [0]
    remaining = set(range(1, n))
    while remaining:
        ready = sorted(v for v in remaining if int(w.parent[v]) in order)
        pick = ready[int(rng.integers(0, len(ready)))]
        order.append(pick)
        remaining.remove(pick)
    new_of = {old: i for i, old in enumerate(order)}
    w2 = gen.Workload(**{**w.__dict__})
    w2.parent = np.array([-1] + [new_of[int(w.parent[o])] for o in order[1:]], np.int32)
    w2.q = w.q[order]; w2.k_node = w.k_node[order]; w2.v_node = w.v_node[order]
    out2, _ = oracle.tree_attention(w2)
    np.testing.assert_allclose(out2, out[order], rtol=1e-13, atol=1e-13)


def test_paged_shuffled_equals_contiguous():
    a = _small(11, "random", "bf16", shuffle=False)
    b = _small(11, "random", "bf16", shuffle=True)
    # same logical rows: rebuild b's physical cache from a's contiguous one
    kb = np.zeros_like(a.k_cache); vb = np.zeros_like(a.v_cache)
    for s in range(a.B):
        nblk = (int(a.prefix_len[s]) + a.block_size - 1) // a.block_size
        for j in range(nblk):
            kb[b.block_table[s, j]] = a.k_cache[a.block_table[s, j]]
            vb[b.block_table[s, j]] = a.v_cache[a.block_table[s, j]]
    b.k_cache, b.v_cache = kb, vb
    oa, la = oracle.tree_attention(a)
    ob, lb = oracle.tree_attention(b)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)
