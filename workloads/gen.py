"""Seeded generators for the five workload shapes and for small test cases.

Every array gets its own seeded stream keyed by the seed and the array's name
(numpy's counter-based Philox for small arrays, torch's seeded CPU generator for
the bulk normal arrays), so adding an array never shifts another one.

Shapes follow the pages' workloads:
  * Qwen3-8B-like attention heads (32 query / 8 KV heads, head_dim 128),
  * draft trees of tens of nodes and depth 6-10 (RheoSampling's tree size 60 /
    depth 8 default, PTD's width 4 / depth 6),
  * vocabulary 151936,
  * PreSTO states of T tokens with a prefetch batch of N_pf suffix requests
    collected by breadth-first search under Condition 1.
"""

from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np
import torch

CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")

CONFIG_DESCRIPTIONS = {
    "c1": "tiny fp32: 1 seq, prefix 128, complete binary tree of 15 nodes, 4/1 heads, d=64, V=1000, T=1",
    "c2": "Qwen3-8B-shaped layer bf16: 1 seq, prefix 2048, 60-node top-8 expansion tree depth<=6, 32/8 heads, d=128, V=151936, T=0.7",
    "c3": "batched verify bf16: 16 seqs, prefix U[1024,8192], shuffled paged KV (block 16), 64-node random trees depth<=8, 32/8 heads, d=128, V=151936, T=1",
    "c4": "PreSTO prefetch bf16: shared state T=4096, 32 BFS/Condition-1 suffix requests, 32/8 heads, d=128, alpha=4, tau=1/4",
    "c5": "long context bf16: 4 seqs, prefix 32768 shuffled paged KV, 128-node top-8 expansion trees depth<=10, 32/8 heads, d=128, V=151936, T=1",
}


DRAFT_PEAK_DEFAULT = (4.0, 7.0)

# ----------------------------------------------------------------------------
# random streams and bf16 storage helpers
# ----------------------------------------------------------------------------

def _key(seed: int, *names) -> list:
    key = [int(seed) & 0xFFFFFFFF]
    for n in names:
        key.append(zlib.crc32(str(n).encode()) & 0xFFFFFFFF)
    return key


def _rng(seed: int, *names) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence(_key(seed, *names))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored array (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def _normal(key: list, shape, std=1.0) -> np.ndarray:
    """Bulk N(0, std^2) float32 array from its own seeded stream."""
    g = torch.Generator().manual_seed(int(np.random.SeedSequence(key).generate_state(1, np.uint64)[0] >> 1))
    out = torch.randn(tuple(int(s) for s in shape), generator=g, dtype=torch.float32).numpy()
    if std != 1.0:
        out *= np.float32(std)
    return out


def _top_tokens(q: np.ndarray, k: int) -> np.ndarray:
    """The k most probable token ids, by descending probability then ascending id."""
    k = min(k, q.size)
    if k < q.size:
        part = np.argpartition(-q, k - 1)[:k]
        kth = q[part].min()
        cand = np.nonzero(q >= kth)[0]           # keeps every token tied with the k-th
    else:
        cand = np.arange(q.size)
    order = np.lexsort((cand, -q[cand]))
    return cand[order][:k]


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def _draft_softmax(z: np.ndarray) -> np.ndarray:
    """Softmax of a draft model's logits (input construction only)."""
    z = z.astype(np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def _truncate(z: np.ndarray, k: Optional[int]):
    """A draft row's logits kept at its k largest entries (ties: lower token id first), the
    others set to -inf before the softmax (RheoSampling's sparse draft, Section 3.2); returns the
    truncated logits and the kept token ids in ascending order (all ids when k is None)."""
    if k is None or k >= z.size:
        return z, np.arange(z.size)
    keep = np.sort(_top_tokens(z, k))
    out = np.full(z.size, -np.inf)
    out[keep] = z[keep]
    return out, keep


# ----------------------------------------------------------------------------
# containers
# ----------------------------------------------------------------------------

@dataclass
class PrestoInputs:
    """One PreSTO prefetch round (Section 3.2 and Appendix B of the PreSTO page).

    Per-token arrays are indexed by position t = 1..T; entry t-1 holds token t.
    """
    T: int
    alpha: float
    root_lp0: np.ndarray          # [T] f32, log p0(x_t | x_{0:t-1}) of the current state
    root_lq: np.ndarray           # [T] f32, log q_tau(x_t | x_{0:t-1})
    cut: np.ndarray               # [R] i32, cut index c_i in {0..T-1}
    suffix_off: np.ndarray        # [R+1] i32, CSR offsets into lp0/lq (request i owns T - c_i tokens)
    lp0: np.ndarray               # [sum S] f32, suffix tokens t = c_i+1..T of request i
    lq: np.ndarray                # [sum S] f32
    pf_parent: np.ndarray         # [M] i32, prefetching-tree parent (-1 root), parent < self
    pf_is_accept: np.ndarray      # [M] u8, 1 for an acceptance (left) child
    pf_request: np.ndarray        # [M] i32, request id of an acceptance child in this batch, -1 otherwise
    pf_cut: np.ndarray            # [M] i32, cut index carried by each tree node (root: T)
    u: np.ndarray                 # [M] f32, MH uniform used for the decision taken at each node
    max_transitions: int


@dataclass
class Workload:
    name: str
    dtype: str                    # "f32" or "bf16" for q/k/v/logits storage
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    sm_scale: float
    node_offsets: np.ndarray      # [B+1] i32
    parent: np.ndarray            # [N] i32, sequence-local, -1 for the root (node 0 of each sequence)
    prefix_len: np.ndarray        # [B] i32
    q: np.ndarray                 # [N, Hq, D]
    k_node: np.ndarray            # [N, Hkv, D]
    v_node: np.ndarray            # [N, Hkv, D]
    k_cache: np.ndarray           # [num_blocks, Hkv, block_size, D]
    v_cache: np.ndarray           # [num_blocks, Hkv, D, block_size] (d-major within a block)
    block_table: np.ndarray       # [B, max_blocks] i32 (-1 where unused)
    V: int = 0
    logits: Optional[np.ndarray] = None       # [N, V]
    temperature: Optional[np.ndarray] = None  # [B] f32
    draft: Optional[np.ndarray] = None        # [R, V] f32 (dense draft rows), or None when sparse
    draft_row: Optional[np.ndarray] = None    # [N] i32, -1 if the node has no sampled child
    draft_k: int = 0                          # sparse draft rows: support size K (0 = dense)
    draft_idx: Optional[np.ndarray] = None    # [R, K] i32, support token ids, ascending
    draft_val: Optional[np.ndarray] = None    # [R, K] f32, q~ at those tokens
    token: Optional[np.ndarray] = None        # [N] i32
    sampled: Optional[np.ndarray] = None      # [N] u8
    uniforms: Optional[np.ndarray] = None     # [N, 2] f32
    presto: Optional[PrestoInputs] = None
    info: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return int(self.node_offsets[-1])

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def seq_nodes(self, b: int) -> range:
        return range(int(self.node_offsets[b]), int(self.node_offsets[b + 1]))


# ----------------------------------------------------------------------------
# tree shapes
# ----------------------------------------------------------------------------

def complete_binary_parents(n: int) -> np.ndarray:
    return np.array([-1] + [(i - 1) // 2 for i in range(1, n)], dtype=np.int32)


def chain_parents(n: int) -> np.ndarray:
    return np.arange(-1, n - 1, dtype=np.int32)


def star_parents(n: int) -> np.ndarray:
    """The root and n - 1 children of the root."""
    return np.array([-1] + [0] * (n - 1), dtype=np.int32)


def random_depth_parents(n: int, max_depth: int, rng) -> np.ndarray:
    """Node i picks a depth d uniform in 1..min(max_depth, deepest so far + 1) and a
    parent uniform among the nodes already at depth d-1."""
    parents = [-1]
    by_depth = {0: [0]}
    deepest = 0
    for i in range(1, n):
        d = int(rng.integers(1, min(max_depth, deepest + 1) + 1))
        cands = by_depth[d - 1]
        p = cands[int(rng.integers(0, len(cands)))]
        parents.append(p)
        by_depth.setdefault(d, []).append(i)
        deepest = max(deepest, d)
    return np.array(parents, dtype=np.int32)


@dataclass
class _Cand:
    cid: int
    parent: int
    depth: int
    token: int
    proxy: float
    score: float
    sampled: bool = False
    slot: int = 0


def build_rheo_tree(R: int, depth: int, expand_k: int, slots_k: int, m: int,
                    hybrid_rule: Callable[[int, int], bool],
                    draft_probs: Callable[[List[int], int], tuple],
                    sample_tail: Callable[[List[int], np.ndarray], int],
                    eps: float = 1e-6, proxy_override: Optional[float] = None):
    """EAGLE-style expand-then-rerank draft tree with RheoSampling's hybrid pool
    (RheoSampling, Section 2.1 and 3.2; Appendix C.1 for proxies and tie-breaks).

    * Each depth expands the ``expand_k`` frontier nodes with the highest path
      score (ties: earlier creation first).
    * A plain parent gets its ``slots_k`` highest-probability draft tokens.
    * A hybrid parent (``hybrid_rule(depth, rank)``) gets its top-m lead tokens,
      one token Y drawn from the renormalised tail q~, and fill tokens (the
      highest remaining ones).  Y carries the proxy min{q(x_m), z} with
      z = 1 - sum of the lead masses (q(x_1) + eps when m = 0); verification
      uses the true q~.
    * Global pruning keeps the R best nodes by path score, then shallower
      first, then left-to-right (creation order).

    ``proxy_override`` replaces the sampled token's proxy by a fixed value (the
    ad-hoc proxy of RheoSampling Table 1, used only to show why it is wrong).

    ``draft_probs(path_tokens, cid)`` returns (q_untempered, q_tempered) over
    the vocabulary for the node reached by ``path_tokens``;
    ``sample_tail(path_tokens, qtilde)`` returns the sampled token.

    Returns (parent, token, sampled, draft_of_parent, path_tokens_per_node, cids)
    with nodes renumbered so that parent < child; node 0 is the root.
    """
    root = _Cand(cid=0, parent=-1, depth=0, token=-1, proxy=1.0, score=1.0)
    cands = [root]
    paths = {0: []}
    drafts = {}
    frontier = [root]
    for d in range(1, depth + 1):
        order = sorted(frontier, key=lambda c: (-c.score, c.cid))[:expand_k]
        new = []
        for rank, par in enumerate(order):
            q, q_t = draft_probs(paths[par.cid], par.cid)
            by_q = _top_tokens(q, slots_k + 1)               # descending q, ties by token id
            if hybrid_rule(d, rank):
                lead = [int(t) for t in by_q[:m]]
                z = 1.0 - float(sum(q[t] for t in lead))
                qtilde = q_t.copy()
                qtilde[lead] = 0.0
                qtilde /= qtilde.sum()
                y = int(sample_tail(paths[par.cid], qtilde))
                proxy_y = min(float(q[lead[-1]]), z) if m > 0 else float(q[by_q[0]]) + eps
                if proxy_override is not None:
                    proxy_y = float(proxy_override)
                fill = [int(t) for t in by_q if int(t) not in lead and int(t) != y][: slots_k - m - 1]
                slots = [(t, float(q[t]), False) for t in lead] + [(y, proxy_y, True)] + \
                        [(t, float(q[t]), False) for t in fill]
                drafts[par.cid] = qtilde
            else:
                slots = [(int(t), float(q[t]), False) for t in by_q[:slots_k]]
            for si, (tok, proxy, smp) in enumerate(slots):
                c = _Cand(cid=len(cands), parent=par.cid, depth=d, token=tok, proxy=proxy,
                          score=par.score * proxy, sampled=smp, slot=si)
                cands.append(c)
                paths[c.cid] = paths[par.cid] + [tok]
                new.append(c)
        frontier = new
    kept = sorted(cands[1:], key=lambda c: (-c.score, c.depth, c.cid))[:R]
    kept_ids = {c.cid for c in kept} | {0}
    for c in kept:
        assert c.parent in kept_ids, "global pruning must keep the tree ancestor-closed"
    nodes = [root] + sorted(kept, key=lambda c: (c.depth, c.cid))
    new_id = {c.cid: i for i, c in enumerate(nodes)}
    parent = np.array([-1] + [new_id[c.parent] for c in nodes[1:]], dtype=np.int32)
    token = np.array([-1] + [c.token for c in nodes[1:]], dtype=np.int64)
    sampled = np.array([0] + [1 if c.sampled else 0 for c in nodes[1:]], dtype=np.uint8)
    draft_of = {}
    for c in nodes[1:]:
        if c.sampled:
            draft_of[new_id[c.parent]] = drafts[c.parent]
    return parent, token, sampled, draft_of, [paths[c.cid] for c in nodes], [c.cid for c in nodes]


# ----------------------------------------------------------------------------
# paged prefix KV
# ----------------------------------------------------------------------------

def _paged_prefix(seed, prefix_len, Hkv, D, bs, dtype, shuffle=True, shared=False):
    B = len(prefix_len)
    nblk = [(int(L) + bs - 1) // bs for L in prefix_len]
    if shared:
        total = max(nblk) if nblk else 0
    else:
        total = int(sum(nblk))
    perm = _rng(seed, "block_perm").permutation(total) if shuffle else np.arange(total)
    max_blocks = max(1, max(nblk) if nblk else 1)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        if shared:
            table[b, : nblk[b]] = perm[: nblk[b]]
        else:
            table[b, : nblk[b]] = perm[off: off + nblk[b]]
            off += nblk[b]
    nb = max(total, 1)
    k_cache = _store(_normal(_key(seed, "k_cache"), (nb, Hkv, bs, D)), dtype)
    v_cache = _store(_normal(_key(seed, "v_cache"), (nb, Hkv, D, bs)), dtype)
    return k_cache, v_cache, table


# ----------------------------------------------------------------------------
# tree batches (configurations c1, c2, c3, c5 and small test cases)
# ----------------------------------------------------------------------------

def tree_batch(seed: int, *, B: int, prefix_len, tree: str, n_nodes, Hq: int, Hkv: int, D: int,
               dtype: str, V: int = 0, temperature: float = 1.0, logit_std: float = 3.0,
               draft_noise: float = 0.5, max_depth: int = 8, expand_k: int = 8,
               hybrid: str = "level", shuffle_blocks: bool = True, block_size: int = 16,
               draft_peak=None, draft_support: Optional[int] = None,
               name: str = "custom") -> Workload:
    """A batch of B independent sequences, each a prefix in paged KV plus one
    token tree whose node 0 is the root (the last committed token).

    tree: "binary" (complete binary, children 2i+1 sampled / 2i+2 deterministic),
          "random" (random-depth tree, first child of each node sampled),
          "chain"  (a path; no verification decoration beyond the same rule),
          "star"   (n - 1 children of the root),
          "eagle"  (top-k expand-then-rerank with the Rheo hybrid pool).
    """
    prefix_len = np.asarray(prefix_len, dtype=np.int32).reshape(-1)
    if prefix_len.size == 1 and B > 1:
        prefix_len = np.full(B, int(prefix_len[0]), dtype=np.int32)
    n_nodes = np.asarray(n_nodes, dtype=np.int64).reshape(-1)
    if n_nodes.size == 1 and B > 1:
        n_nodes = np.full(B, int(n_nodes[0]))

    parents, tokens, sampled_l, draft_rows_l, logits_l, supports_l = [], [], [], [], [], []
    have_verify = V > 0
    for b in range(B):
        n = int(n_nodes[b])
        if tree == "eagle":
            par, tok, smp, dr, lg, sup = _eagle_seq(seed, b, n, V, temperature, logit_std, draft_noise,
                                                    max_depth, expand_k, hybrid, dtype, draft_peak,
                                                    draft_support)
        else:
            if tree == "binary":
                par = complete_binary_parents(n)
            elif tree == "chain":
                par = chain_parents(n)
            elif tree == "star":
                par = star_parents(n)
            elif tree == "random":
                par = random_depth_parents(n, max_depth, _rng(seed, "tree", b))
            else:
                raise ValueError(tree)
            if have_verify:
                tok, smp, dr, lg, sup = _decorate_first_child_sampled(seed, b, par, V, temperature,
                                                                      logit_std, draft_noise, dtype,
                                                                      draft_support)
            else:
                tok = np.zeros(n, np.int64); smp = np.zeros(n, np.uint8); dr = {}; lg = None; sup = {}
        parents.append(par); tokens.append(tok); sampled_l.append(smp)
        draft_rows_l.append(dr); logits_l.append(lg); supports_l.append(sup)

    node_offsets = np.zeros(B + 1, dtype=np.int32)
    node_offsets[1:] = np.cumsum([len(p) for p in parents])
    N = int(node_offsets[-1])
    parent = np.concatenate(parents).astype(np.int32)

    q = _store(_normal(_key(seed, "q"), (N, Hq, D)), dtype)
    k_node = _store(_normal(_key(seed, "k_node"), (N, Hkv, D)), dtype)
    v_node = _store(_normal(_key(seed, "v_node"), (N, Hkv, D)), dtype)
    k_cache, v_cache, table = _paged_prefix(seed, prefix_len, Hkv, D, block_size, dtype,
                                            shuffle=shuffle_blocks)
    w = Workload(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size,
                 sm_scale=1.0 / math.sqrt(D), node_offsets=node_offsets, parent=parent,
                 prefix_len=prefix_len, q=q, k_node=k_node, v_node=v_node, k_cache=k_cache,
                 v_cache=v_cache, block_table=table)
    if have_verify:
        w.V = V
        w.logits = np.concatenate(logits_l, axis=0)
        w.temperature = np.full(B, temperature, dtype=np.float32)
        w.token = np.concatenate(tokens).astype(np.int32)
        w.sampled = np.concatenate(sampled_l).astype(np.uint8)
        draft_row = np.full(N, -1, dtype=np.int32)
        rows, idx = [], []
        for b in range(B):
            for v_local in sorted(draft_rows_l[b]):
                draft_row[node_offsets[b] + v_local] = len(rows)
                rows.append(draft_rows_l[b][v_local])
                idx.append(supports_l[b][v_local])
        w.draft_row = draft_row
        if draft_support is None:
            w.draft = (np.stack(rows).astype(np.float32) if rows else np.zeros((0, V), np.float32))
        else:                      # sparse rows: the support ids (ascending) and q~ there
            K = int(draft_support)
            w.draft_k = K
            w.draft_idx = (np.stack(idx).astype(np.int32) if idx else np.zeros((0, K), np.int32))
            w.draft_val = (np.stack([r[i] for r, i in zip(rows, idx)]).astype(np.float32) if rows
                           else np.zeros((0, K), np.float32))
        w.uniforms = _rng(seed, "uniforms").random((N, 2), dtype=np.float32)
    return w


def _node_logits(seed, b, key, V, std, dtype):
    raw = _normal(_key(seed, "logits", b, key), (V,), std)
    stored = _store(raw, dtype)
    return stored, (bf16_bits_to_f32(stored) if dtype == "bf16" else stored)


def _decorate_first_child_sampled(seed, b, parent, V, T, std, noise, dtype, support=None):
    """Per internal node v: draft q_v = softmax((l_v + N(0, noise)) / T) (with ``support``,
    the logits truncated to their ``support`` largest entries first).  The lowest-id child is
    the sampled one (token ~ q_v, draft row = q_v); the other children take the highest
    remaining draft tokens in child-id order (the m = 0 hybrid pool).  The root's own token
    is arbitrary."""
    n = len(parent)
    stored, vals = [], []
    for v in range(n):
        s, f = _node_logits(seed, b, v, V, std, dtype)
        stored.append(s); vals.append(f)
    token = np.zeros(n, dtype=np.int64)
    token[0] = int(_rng(seed, "root_token", b).integers(0, V))
    sampled = np.zeros(n, dtype=np.uint8)
    drafts, supports = {}, {}
    children = [[] for _ in range(n)]
    for c in range(1, n):
        children[parent[c]].append(c)
    for v in range(n):
        if not children[v]:
            continue
        r = _rng(seed, "draft", b, v)
        zt, supports[v] = _truncate((vals[v].astype(np.float64) + noise * r.standard_normal(V)) / T, support)
        qv = _draft_softmax(zt)
        q32 = qv.astype(np.float32)
        y = int(r.choice(V, p=qv))
        while q32[y] <= 0.0:              # the stored draft must give the sampled token mass
            y = int(r.choice(V, p=qv))
        kids = sorted(children[v])
        token[kids[0]] = y
        sampled[kids[0]] = 1
        drafts[v] = q32
        by_q = _top_tokens(qv, len(kids) + 1)
        rest = [int(t) for t in by_q[: len(kids) + 1] if int(t) != y][: len(kids) - 1]
        for c, t in zip(kids[1:], rest):
            token[c] = t
    return token, sampled, drafts, np.stack(stored), supports


def _eagle_seq(seed, b, n_nodes, V, T, std, noise, depth, expand_k, hybrid, dtype, peak=None,
               support=None):
    cache = {}
    support_of = {}

    def logits_of(cid):
        if cid not in cache:
            cache[cid] = _node_logits(seed, b, ("cand", cid), V, std, dtype)
        return cache[cid]

    def draft_probs(path, cid):
        _, f = logits_of(cid)
        r = _rng(seed, "draft_noise", b, cid)
        z = f.astype(np.float64) + noise * r.standard_normal(V)
        if peak is not None:
            # a drafter's confident next token: its largest logit raised by U(peak) (the tree's
            # depth then comes from the budget, as with a trained drafter, not from flat rows)
            z[int(np.argmax(z))] += r.uniform(peak[0], peak[1])
        z, support_of[cid] = _truncate(z, support)
        return _draft_softmax(z), _draft_softmax(z / T)

    tail_rng = _rng(seed, "tail", b)

    def sample_tail(path, qtilde):
        q32 = qtilde.astype(np.float32)
        while True:
            y = int(tail_rng.choice(qtilde.size, p=qtilde))
            if q32[y] > 0.0:
                return y

    if hybrid == "level":
        rule = lambda d, rank: rank == 0          # one sampled slot per depth
    elif hybrid == "all":
        rule = lambda d, rank: True               # every expanded parent samples
    else:
        rule = lambda d, rank: False
    parent, token, sampled, draft_of, _paths, cids = build_rheo_tree(
        n_nodes - 1, depth, expand_k, 8, 1, rule, draft_probs, sample_tail)
    token = token.copy()
    token[0] = int(_rng(seed, "root_token", b).integers(0, V))
    logits = np.stack([logits_of(c)[0] for c in cids])
    drafts = {v: q.astype(np.float32) for v, q in draft_of.items()}
    return parent, token, sampled, drafts, logits, {v: support_of[cids[v]] for v in draft_of}


# ----------------------------------------------------------------------------
# PreSTO prefetch batch (configuration c4 and small test cases)
# ----------------------------------------------------------------------------

def bfs_prefetch_tree(T: int, n_pf: int, rng, max_nodes: int = 1 << 20):
    """Breadth-first collection of feasible suffix requests (PreSTO Section 3.2,
    Condition 1, Example 2).  The root carries cut T.  Expanding a node creates
    an acceptance child with a fresh cut c' ~ Unif{0..T-1}, kept in the batch
    (and queued) iff c' <= the node's cut, otherwise deferred; and a rejection
    child that inherits the node's cut and is always queued.  Stops at n_pf
    requests or an empty queue."""
    pf_parent = [-1]; pf_acc = [0]; pf_req = [-1]; pf_cut = [T]
    req_cut = []
    queue = [0]
    while queue and len(req_cut) < n_pf and len(pf_parent) < max_nodes:
        v = queue.pop(0)
        c_new = int(rng.integers(0, T))
        a = len(pf_parent)
        pf_parent.append(v); pf_acc.append(1); pf_cut.append(c_new)
        if c_new <= pf_cut[v]:
            pf_req.append(len(req_cut)); req_cut.append(c_new); queue.append(a)
        else:
            pf_req.append(-1)
        r = len(pf_parent)
        pf_parent.append(v); pf_acc.append(0); pf_req.append(-1); pf_cut.append(pf_cut[v])
        queue.append(r)
    return (np.array(pf_parent, np.int32), np.array(pf_acc, np.uint8), np.array(pf_req, np.int32),
            np.array(pf_cut, np.int32), np.array(req_cut, np.int32))


def presto_batch(seed: int, *, T: int, n_pf: int, Hq: int, Hkv: int, D: int, dtype: str = "bf16",
                 alpha: float = 4.0, max_transitions: int = 100, block_size: int = 16,
                 with_attention: bool = True, name: str = "custom") -> Workload:
    """One PreSTO prefetch round.  Request i keeps the shared prefix x_{0:c_i}
    (prefix rows 0..c_i of the cached state; row 0 stands for the prompt) and
    scores its own suffix of T - c_i tokens causally.  Every request's block
    table points at the same physical prefix blocks."""
    pf_parent, pf_acc, pf_req, pf_cut, cut = bfs_prefetch_tree(T, n_pf, _rng(seed, "bfs"))
    R = len(cut)
    lens = (T - cut).astype(np.int64)
    suffix_off = np.zeros(R + 1, dtype=np.int32)
    suffix_off[1:] = np.cumsum(lens)
    lp_rng = _rng(seed, "logprobs")
    pr = PrestoInputs(
        T=T, alpha=float(alpha),
        root_lp0=(-lp_rng.exponential(size=T)).astype(np.float32),
        root_lq=(-lp_rng.exponential(size=T)).astype(np.float32),
        cut=cut, suffix_off=suffix_off,
        lp0=(-lp_rng.exponential(size=int(suffix_off[-1]))).astype(np.float32),
        lq=(-lp_rng.exponential(size=int(suffix_off[-1]))).astype(np.float32),
        pf_parent=pf_parent, pf_is_accept=pf_acc, pf_request=pf_req, pf_cut=pf_cut,
        u=_rng(seed, "mh_uniforms").random(len(pf_parent), dtype=np.float32),
        max_transitions=int(max_transitions))
    if not with_attention:
        w = Workload(name=name, dtype=dtype, B=0, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size,
                     sm_scale=1.0 / math.sqrt(D), node_offsets=np.zeros(1, np.int32),
                     parent=np.zeros(0, np.int32), prefix_len=np.zeros(0, np.int32),
                     q=np.zeros((0, Hq, D)), k_node=np.zeros((0, Hkv, D)),
                     v_node=np.zeros((0, Hkv, D)), k_cache=np.zeros((1, Hkv, block_size, D)),
                     v_cache=np.zeros((1, Hkv, D, block_size)),
                     block_table=np.full((0, 1), -1, np.int32), presto=pr)
        return w
    B = R
    node_offsets = suffix_off.copy()
    N = int(node_offsets[-1])
    parent = np.concatenate([chain_parents(int(n)) for n in lens]).astype(np.int32)
    prefix_len = (cut + 1).astype(np.int32)
    q = _store(_normal(_key(seed, "q"), (N, Hq, D)), dtype)
    k_node = _store(_normal(_key(seed, "k_node"), (N, Hkv, D)), dtype)
    v_node = _store(_normal(_key(seed, "v_node"), (N, Hkv, D)), dtype)
    # the cached state has rows 0..T-1; every request maps the same blocks
    full = np.full(B, T, dtype=np.int32)
    k_cache, v_cache, table = _paged_prefix(seed, full, Hkv, D, block_size, dtype,
                                            shuffle=True, shared=True)
    return Workload(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size,
                    sm_scale=1.0 / math.sqrt(D), node_offsets=node_offsets, parent=parent,
                    prefix_len=prefix_len, q=q, k_node=k_node, v_node=v_node, k_cache=k_cache,
                    v_cache=v_cache, block_table=table, presto=pr)


def draft_logits_row(seed: int, b: int, cid: int, V: int, std: float = 3.0, peak=DRAFT_PEAK_DEFAULT):
    """A drafter's bf16 logits at candidate `cid` of tree `b`: N(0, std^2) with the largest entry
    raised by U(peak) (a confident next token, as in the expansion trees above); bf16 bits."""
    z = _normal(_key(seed, "draft_logits", b, cid), (V,), std)
    if peak is not None:
        r = _rng(seed, "draft_peak", b, cid)
        z[int(np.argmax(z))] += np.float32(r.uniform(peak[0], peak[1]))
    return f32_to_bf16_bits(z)


def draft_uniform(seed: int, b: int, d: int, rank: int) -> float:
    """The uniform of the parent of rank `rank` at depth d of tree b (float32 value)."""
    return float(np.float32(_rng(seed, "draft_uniform", b, d, rank).random()))


def device_logits(seed: int, rows: int, V: int, std: float = 3.0, device="cuda"):
    """[rows, V] bfloat16 logits ~ N(0, std^2) drawn on the device by torch's seeded generator
    (for batches too large to draw on the host; sampled rows copied back serve the checks)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence(_key(seed, "device_logits")).generate_state(1, np.uint64)[0] >> 1))
    out = torch.randn((int(rows), int(V)), generator=g, device=device, dtype=torch.float32)
    return out.mul_(std).to(torch.bfloat16)


# ----------------------------------------------------------------------------
# the five workload shapes
# ----------------------------------------------------------------------------

# Raise of each draft row's largest logit in the top-8 expansion trees of the one-tree and
# long-context workloads (see _eagle_seq): flat N(0, 3^2) rows over 151936 tokens give a top-1
# draft probability of a few percent, and the global prune then keeps only 3-4 levels.
DRAFT_PEAK = (4.0, 7.0)


def make(name: str, seed: int = 10086, draft_support: Optional[int] = None) -> Workload:
    """One of the five workloads; with draft_support (the tree workloads with verification),
    its draft rows are sparse: the draft logits truncated to their top draft_support entries
    before the softmax (RheoSampling Section 3.2), stored as (ids, values)."""
    sp = {} if draft_support is None else {"draft_support": int(draft_support)}
    if draft_support is not None and name not in ("c2", "c3", "c5"):
        raise ValueError("sparse draft rows apply to the tree workloads c2, c3 and c5")
    if name == "c1":
        w = tree_batch(seed, B=1, prefix_len=128, tree="binary", n_nodes=15, Hq=4, Hkv=1, D=64,
                       dtype="f32", V=1000, temperature=1.0, logit_std=2.0, draft_noise=0.5,
                       shuffle_blocks=False, name="c1")
    elif name == "c2":
        w = tree_batch(seed, B=1, prefix_len=2048, tree="eagle", n_nodes=60, Hq=32, Hkv=8, D=128,
                       dtype="bf16", V=151936, temperature=0.7, logit_std=3.0, max_depth=6,
                       expand_k=8, hybrid="level", draft_peak=DRAFT_PEAK, name="c2", **sp)
    elif name == "c3":
        L = _rng(seed, "prefix_lens").integers(1024, 8193, size=16).astype(np.int32)
        w = tree_batch(seed, B=16, prefix_len=L, tree="random", n_nodes=64, Hq=32, Hkv=8, D=128,
                       dtype="bf16", V=151936, temperature=1.0, logit_std=3.0, max_depth=8,
                       name="c3", **sp)
    elif name == "c4":
        w = presto_batch(seed, T=4096, n_pf=32, Hq=32, Hkv=8, D=128, dtype="bf16", alpha=4.0,
                         name="c4")
    elif name == "c5":
        w = tree_batch(seed, B=4, prefix_len=32768, tree="eagle", n_nodes=128, Hq=32, Hkv=8,
                       D=128, dtype="bf16", V=151936, temperature=1.0, logit_std=3.0,
                       max_depth=10, expand_k=8, hybrid="all", draft_peak=DRAFT_PEAK, name="c5", **sp)
    else:
        raise ValueError(name)
    w.info["description"] = CONFIG_DESCRIPTIONS[name] + (
        f", sparse draft rows (top-{draft_support} support)" if draft_support is not None else "")
    w.info["seed"] = seed
    return w
