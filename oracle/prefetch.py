"""Which suffix requests PreSTO prefetches in one batch (test infrastructure only).

PreSTO, Section 3.2 step (1) and Appendix C:

* the prefetching tree: node v holds an MH state with cut index c_v (the root: the current
  state, cut T); expanding v creates an acceptance child v+ with a new cut c+ drawn uniformly
  from {0..T-1} -- its suffix-resampling request -- and a rejection child v- that keeps v's state
  and cut;
* Condition 1: the request at v+ can go into the current batch iff c+ <= c_v;
* the BFS rule: traverse from the root in breadth-first order; a feasible acceptance child is
  added to the batch and enqueued, an infeasible one is deferred (not enqueued); the rejection
  child is always enqueued; stop at N_pf requests or an empty queue;
* the predictive rule (Appendix C.1-C.4): candidate nodes I_max are the expandable nodes
  (depth < K' and Condition 1 at their acceptance child) whose strict ancestors are all
  expandable; predicted branch probabilities h^(v+) = (1 + P^(accept) - P^(reject)) / 2
  (Equation 14) from a three-class logistic regression on the cut fraction c+/T; reaching
  weights R^(v0) = 1, R^(v+-) = R^(v) h^(v+-) (Equation 11); the selection maximises
  sum_{v in I} R^(v) over ancestor-closed I within I_max, |I| <= N_pf (Equation 17), computed by
  the dynamic program of Equation 19;
* after scoring: epsilon-rounded branch probabilities h(v+) from A(v+, v) (Equation 10), the
  reaching weights (Equation 11) and the expected number of completed transitions
  F = sum_{v in I} R(v) (Lemma 1, Equation 12), equal to the recursion of Equation 13.

Reading where the pages leave it open: a node of the (infinite) binary prefetching tree is named
by its heap index (root 1, acceptance child 2h, rejection child 2h + 1); the cut of the acceptance
child with heap index h is drawn by the caller's cut_of(h) -- for parity runs, SplitMix64
(splitmix64 below) keyed by (seed, h): c = floor(U T) with U the top 53 bits over 2^53.  Output
nodes are listed in ascending heap index (parent before child); requests in the order of their
acceptance nodes.
"""

from __future__ import annotations

import math
from functools import lru_cache

import numpy as np

MASK64 = (1 << 64) - 1
REJECT, ACCEPT, UNCERTAIN = 0, 1, 2


def splitmix64(x: int) -> int:
    """SplitMix64 output for state x (Steele, Lea and Flood, 2014): add the golden-ratio
    increment, then the variant-13 finaliser."""
    z = (x + 0x9E3779B97F4A7C15) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def splitmix_cut(seed: int, heap: int, T: int) -> int:
    """Cut of the acceptance child with heap index `heap`: floor(U * T), U = top 53 bits / 2^53 of
    splitmix64(seed + heap * golden) -- integer arithmetic, no rounding."""
    z = splitmix64((seed + heap * 0x9E3779B97F4A7C15) & MASK64)
    return ((z >> 11) * T) >> 53


def _depth(h: int) -> int:
    return h.bit_length() - 1


def _tree_arrays(nodes, cut, requests):
    """Output arrays of a prefetching tree given as a set of heap indices (parents included)."""
    order = sorted(nodes)
    pos = {h: i for i, h in enumerate(order)}
    M = len(order)
    parent = np.full(M, -1, np.int32)
    is_acc = np.zeros(M, np.uint8)
    request = np.full(M, -1, np.int32)
    cuts = np.zeros(M, np.int32)
    req_cut = []
    for i, h in enumerate(order):
        cuts[i] = cut[h]
        if h > 1:
            parent[i] = pos[h // 2]
            is_acc[i] = 1 if h % 2 == 0 else 0
            if h in requests:
                request[i] = len(req_cut)
                req_cut.append(cut[h])
    return {"parent": parent, "is_accept": is_acc, "request": request, "cut": cuts,
            "request_cut": np.array(req_cut, np.int32), "heap": np.array(order, np.int64)}


def bfs_tree(T: int, budget: int, depth_cap: int, cut_of):
    """The BFS rule of PreSTO Section 3.2 (1), with the depth cap K' of Appendix C.1."""
    cut = {1: T}
    nodes = {1}
    requests = set()
    queue = [1]
    while queue and len(requests) < budget:
        v = queue.pop(0)
        if _depth(v) >= depth_cap:
            continue
        a, r = 2 * v, 2 * v + 1
        cut[a] = int(cut_of(a))
        cut[r] = cut[v]
        nodes.update((a, r))
        if cut[a] <= cut[v]:                     # Condition 1: in this batch
            requests.add(a)
            queue.append(a)
        queue.append(r)                          # a deferred request's sibling is still enqueued
    return _tree_arrays(nodes, cut, requests)


def class_probs(class_w, frac: float):
    """Three-class logistic regression on the cut fraction: softmax over the classes (certain
    reject, certain accept, uncertain) of bias + slope * frac."""
    z = np.array([class_w[2 * k] + class_w[2 * k + 1] * frac for k in range(3)], np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def predicted_h(class_w, cut_plus: int, T: int) -> float:
    """h^(v+) of Equation 14: (1 + P^(certain accept) - P^(certain reject)) / 2."""
    P = class_probs(class_w, cut_plus / T)
    return 0.5 * (1.0 + P[ACCEPT] - P[REJECT])


class _Candidates:
    """The candidate set I_max over heap indices, with cuts, predicted branch probabilities and
    predicted reaching weights, explored lazily."""

    def __init__(self, T, depth_cap, cut_of, class_w):
        self.T, self.K, self.cut_of, self.w = T, depth_cap, cut_of, class_w
        self._cut = {1: T}

    def cut(self, h):
        if h not in self._cut:
            self._cut[h] = self.cut(h // 2) if h % 2 else int(self.cut_of(h))
        return self._cut[h]

    def expandable(self, h):
        return _depth(h) < self.K and self.cut(2 * h) <= self.cut(h)

    def candidate(self, h):
        while h >= 1:
            if not self.expandable(h):
                return False
            h //= 2
        return True

    def h_plus(self, h):
        return predicted_h(self.w, self.cut(2 * h), self.T)

    def reach(self, h):
        r = 1.0
        while h > 1:
            hp = self.h_plus(h // 2)
            r *= hp if h % 2 == 0 else 1.0 - hp
            h //= 2
        return r


def dp_value(T, budget, depth_cap, cut_of, class_w):
    """V(v0, N_pf) of Equation 19 and one optimal selection (a set of heap indices), by the
    recursion over the acceptance and rejection subtrees with the budget split m."""
    C = _Candidates(T, depth_cap, cut_of, class_w)

    @lru_cache(maxsize=None)
    def V(h, b):
        if b == 0 or not C.candidate(h):
            return 0.0, ()
        hp = C.h_plus(h)
        best, sel = -1.0, ()
        for m in range(b):
            va, sa = V(2 * h, m)
            vr, sr = V(2 * h + 1, b - 1 - m)
            val = 1.0 + hp * va + (1.0 - hp) * vr
            if val > best + 1e-15:
                best, sel = val, (h,) + sa + sr
        return best, sel

    val, sel = V(1, budget)
    return val, set(sel), C


def predictive_tree(T, budget, depth_cap, cut_of, class_w):
    """The predictive rule: the DP's selection I, then the prefetched subtree (the root and both
    children of every node of I); the request of v+ for every v in I.  Returns the tree arrays
    and the predicted transition count F^ (Equation 17)."""
    val, sel, C = dp_value(T, budget, depth_cap, cut_of, class_w)
    nodes = {1}
    cut = {1: T}
    requests = set()
    for h in sel:
        for c in (2 * h, 2 * h + 1):
            nodes.add(c)
            cut[c] = C.cut(c)
        cut[h] = C.cut(h)
        requests.add(2 * h)
    out = _tree_arrays(nodes, cut, requests)
    out["predicted_transitions"] = val
    out["selection"] = sel
    return out


def rounded_h(A: float, eps: float) -> float:
    """h(v+; eps) of Equation 10."""
    if A <= eps:
        return 0.0
    if A >= 1.0 - eps:
        return 1.0
    return A


def reaching_weights(parent, is_accept, request, log_accept, eps):
    """R(v; eps) of Equation 11 for every node of a scored prefetching tree (parent < child), and
    the expected number of completed transitions F = sum over expanded nodes of R (Equation 12).
    A node is expanded when its acceptance child carries a request of this batch; the walk stops
    at any other node (a leaf, or a deferred request)."""
    M = len(parent)
    acc = {}
    for v in range(1, M):
        if is_accept[v]:
            acc[int(parent[v])] = v
    R = np.zeros(M, np.float64)
    R[0] = 1.0
    expanded = np.zeros(M, bool)
    for v in range(1, M):
        p = int(parent[v])
        a = acc.get(p)
        if a is None or int(request[a]) < 0:
            continue                              # p was not expanded: v is not reachable
        h = rounded_h(math.exp(float(log_accept[int(request[a])])), eps)
        R[v] = R[p] * (h if is_accept[v] else 1.0 - h)
    for v in range(M):
        a = acc.get(v)
        expanded[v] = a is not None and int(request[a]) >= 0
    return R, float(np.sum(R[expanded])), expanded


def transitions_recursive(parent, is_accept, request, log_accept, eps, v=0):
    """F(v; eps) by Equation 13: 1 + h(v+) F(v+) + h(v-) F(v-) at an expanded node, else 0."""
    kids = [c for c in range(len(parent)) if int(parent[c]) == v]
    a = next((c for c in kids if is_accept[c]), None)
    r = next((c for c in kids if not is_accept[c]), None)
    if a is None or int(request[a]) < 0:
        return 0.0
    h = rounded_h(math.exp(float(log_accept[int(request[a])])), eps)
    fa = transitions_recursive(parent, is_accept, request, log_accept, eps, a)
    fr = transitions_recursive(parent, is_accept, request, log_accept, eps, r) if r is not None else 0.0
    return 1.0 + h * fa + (1.0 - h) * fr


def predicted_transitions(parent, is_accept, request, cut, class_w, T):
    """F^ of a prefetching tree: the sum of predicted reaching weights (Equation 11 with h^ of
    Equation 14 from the acceptance child's cut) over the nodes whose acceptance child carries a
    request of this batch and that the walk can reach (every ancestor likewise)."""
    M = len(parent)
    acc = {int(parent[v]): v for v in range(1, M) if is_accept[v]}
    R = np.zeros(M, np.float64)
    R[0] = 1.0
    reach = np.zeros(M, bool)
    reach[0] = True
    total = 0.0
    for v in range(M):
        if v > 0:
            p = int(parent[v])
            a = acc.get(p)
            if reach[p] and a is not None and int(request[a]) >= 0:
                hp = predicted_h(class_w, int(cut[a]), T)
                R[v] = R[p] * (hp if is_accept[v] else 1.0 - hp)
                reach[v] = True
        a = acc.get(v)
        if reach[v] and a is not None and int(request[a]) >= 0:
            total += R[v]
    return total
