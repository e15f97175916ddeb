"""Draft-tree construction: expand-then-rerank with RheoSampling's hybrid pool and global
pruning (test infrastructure only).

RheoSampling, Section 2.1 (EAGLE's dynamic tree): at each depth the drafter runs on K selected
parents; each parent gets a candidate pool of K slots; a candidate's path score is the product
of the proxy probabilities along its root path; the K candidates of the depth with the highest
scores are the next depth's parents; after D depths the tree is pruned to a budget of R nodes by
score.  Section 3.2 and Appendix C.1: a hybrid pool takes the top-m lead tokens x_1..x_m (proxy
q(x_i)), one token Y drawn from the tail q~ = q / z off the leads (z = 1 - sum q(x_i)) with proxy
min{q(x_m), z} (q(x_1) + eps when m = 0), then the highest remaining tokens as fills (proxy q); the
draft logits are truncated to their top-128 entries before the softmax (the sparse draft).
Global pruning keeps the R nodes with the highest path scores, ties broken by depth (shallower
first) then left-to-right order; the pruned tree is ancestor-closed (Lemma 5).

Readings where the pages leave a step open:
* a candidate's id is its creation order (the root 0; at each depth the parents in rank order,
  each parent's slots in pool order); "left-to-right" = ascending id; frontier ties go to the
  smaller id as well;
* proxies and path scores use the drafter's distribution q = softmax(z) over the support; the
  sampled token is drawn from the tail of softmax(z / T) over the support (temperature only in
  sampling and verification, RheoSampling Section 5.4), which is also the draft row verification
  uses; with T = 1 the two coincide;
* the draw of Y is the inverse CDF in token-id order with the parent's uniform: the smallest
  token t with sum_{s <= t} q~(s) > u;
* the support of a row is its S largest draft logits, ties at the S-th value to the smaller ids;
* per depth d the parents are the top min(K, candidates of depth d-1) candidates of depth d-1
  (depth 1: the root); a pool has min(K_slots, S) slots;
* nodes of the pruned tree are numbered by (depth, id), the root first.
Decisions that floating-point rounding could flip (different scores within 1e-9 relative at a
cut, a uniform within 1e-9 of a CDF step) are recorded as near-ties; equal scores at a cut go by
the tie rule (the next parents: smaller id; the prune: shallower, then smaller id).
"""

from __future__ import annotations

import numpy as np

TIE = 1e-9


def support_of(z: np.ndarray, S: int) -> np.ndarray:
    """Token ids of the S largest logits (ties to the smaller id), in that order."""
    order = np.lexsort((np.arange(z.size), -z))
    return order[:S]


class DraftTreeBuilder:
    def __init__(self, V, depth, expand_k, slots, lead_m, hybrid, support, budget, temperature=1.0, eps=1e-6,
                 proxy_override=None):
        assert 0 <= lead_m < slots <= support <= V
        self.proxy_override = proxy_override     # a fixed proxy for Y (only to show why it is wrong)
        self.V, self.D, self.K, self.slots, self.m = V, depth, expand_k, slots, lead_m
        self.hybrid, self.S, self.R, self.T, self.eps = hybrid, support, budget, float(temperature), eps
        # candidates: id -> (parent id, depth, token, score, sampled)
        self.parent, self.depth, self.token, self.score, self.sampled = [-1], [0], [-1], [1.0], [False]
        self.rows = {}                 # parent id -> (support ids ascending, q~ at them)
        self.frontier = [0]
        self.ties = []

    def is_hybrid(self, rank):
        return self.hybrid == "all" or (self.hybrid == "first" and rank == 0)

    def _pool(self, pid, rank, z, u):
        keep = support_of(z, self.S)                      # by logit, descending
        zk = z[keep]
        q = np.exp(zk - zk.max())
        q /= q.sum()
        qT = np.exp((zk - zk.max()) / self.T)
        qT /= qT.sum()
        n = self.slots
        if not self.is_hybrid(rank):
            return [(int(keep[i]), float(q[i]), False) for i in range(n)]
        m = self.m
        zres = 1.0 - float(q[:m].sum())
        tail = qT.copy()
        tail[:m] = 0.0
        tail /= tail.sum()
        ids = np.argsort(keep)                            # token-id order
        cum = np.cumsum(tail[ids])
        j = int(np.searchsorted(cum, u, side="right"))
        if j >= len(ids):
            j = int(np.nonzero(tail[ids] > 0)[0][-1])
        if abs(cum[j] - u) < TIE or (j > 0 and abs(cum[j - 1] - u) < TIE):
            self.ties.append(("sample", pid))
        y = int(keep[ids[j]])
        proxy = min(float(q[m - 1]), zres) if m > 0 else float(q[0]) + self.eps
        if self.proxy_override is not None:
            proxy = float(self.proxy_override)
        fills = [i for i in range(len(keep)) if i >= m and int(keep[i]) != y][: n - m - 1]
        slots = [(int(keep[i]), float(q[i]), False) for i in range(m)] + [(y, proxy, True)] + \
                [(int(keep[i]), float(q[i]), False) for i in fills]
        self.rows[pid] = (keep[ids].astype(np.int64), tail[ids].copy())
        return slots

    def expand(self, d, logits_rows, uniforms):
        """Depth d: pools of the current parents (logits_rows[j] = the drafter's logits at
        parent rank j, uniforms[j] its uniform); returns the next parents (candidate ids)."""
        new = []
        for rank, pid in enumerate(self.frontier):
            z = np.asarray(logits_rows[rank], np.float64)
            for tok, proxy, smp in self._pool(pid, rank, z, float(uniforms[rank])):
                self.parent.append(pid)
                self.depth.append(d)
                self.token.append(tok)
                self.score.append(self.score[pid] * proxy)
                self.sampled.append(smp)
                new.append(len(self.parent) - 1)
        order = sorted(new, key=lambda c: (-self.score[c], c))
        k = min(self.K, len(order))
        self._cut_tie(order, k)
        self.frontier = order[:k]
        return list(self.frontier)

    def _cut_tie(self, order, k):
        """Records a near-tie at a cut: two scores that differ, but by at most TIE relative.  Equal
        scores are not recorded: the stated tie rule decides them."""
        if 0 < k < len(order):
            a, b = self.score[order[k - 1]], self.score[order[k]]
            if a != b and abs(a - b) <= TIE * max(abs(a), abs(b)):
                self.ties.append(("cut", order[k - 1], order[k]))

    def prune(self):
        """Global top-R by (score desc, depth asc, id asc); nodes renumbered by (depth, id).
        Returns parent, token, sampled, the candidate id of each node, and per node the draft row
        (support ids ascending, q~) of its sampled child's pool, or None."""
        cands = list(range(1, len(self.parent)))
        order = sorted(cands, key=lambda c: (-self.score[c], self.depth[c], c))
        R = min(self.R, len(order))
        self._cut_tie(order, R)
        kept = set(order[:R])
        for c in kept:
            assert self.parent[c] == 0 or self.parent[c] in kept, "pruned tree must be ancestor-closed"
        nodes = [0] + sorted(kept, key=lambda c: (self.depth[c], c))
        new_id = {c: i for i, c in enumerate(nodes)}
        parent = np.array([-1] + [new_id[self.parent[c]] for c in nodes[1:]], np.int32)
        token = np.array([-1] + [self.token[c] for c in nodes[1:]], np.int64)
        sampled = np.array([0] + [1 if self.sampled[c] else 0 for c in nodes[1:]], np.uint8)
        rows = [None] * len(nodes)
        for c in nodes[1:]:
            if self.sampled[c]:
                rows[new_id[self.parent[c]]] = self.rows[self.parent[c]]
        return parent, token, sampled, np.array(nodes, np.int64), rows


def build(V, depth, expand_k, slots, lead_m, hybrid, support, budget, logits_of, uniform_of,
          temperature=1.0, eps=1e-6):
    """The whole construction with the drafter's logits at candidate c given by logits_of(c) and
    the uniform of the parent at (depth, rank) by uniform_of(d, rank)."""
    t = DraftTreeBuilder(V, depth, expand_k, slots, lead_m, hybrid, support, budget, temperature, eps)
    for d in range(1, depth + 1):
        rows = [logits_of(c) for c in t.frontier]
        t.expand(d, rows, [uniform_of(d, r) for r in range(len(t.frontier))])
    return t, t.prune()
