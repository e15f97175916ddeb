"""Temperature softmax and layer-by-layer tree verification.

RheoSampling, Section 3.3, Algorithm 1 (RheoVerification), applied at every
layer of the pruned tree from the root down (Theorem 1 / Appendix C.3 apply it
"layer-by-layer"):

  * with a sampled candidate u_s (s != -1): draw eta and accept u_s iff
    eta <= min(1, p(u_s) / q~(u_s)), using the true sampling distribution q~;
    on rejection drop u_s and set r = norm(max(0, p - q~));
  * without one (s = -1): r = p;
  * then test the remaining candidates one at a time: accept u_i iff
    eta <= r(u_i); otherwise set r(u_i) = 0 and renormalise r;
  * if every candidate is rejected, draw the output token from the final r.

With no sampled candidates this is the sequential rejection of Progressive Tree
Drafting (Section 3.2, Appendix E Algorithm 2, Appendix F); with one sampled
child per node it is standard speculative sampling (RheoSampling Section 2.2).
The accepted path from the root plus the final token is X' (Progressive Tree
Drafting, Section 3.2).

Readings taken where the pages leave a step open:
  * p = softmax(l / T) with the node's target logits l (RheoSampling Section 5.4:
    temperature only enters sampling and verification); the draft row supplied
    for a node is the distribution its sampled child was drawn from;
  * candidate order: the sampled child first (stochastic-first), then the other
    children by ascending node id (Algorithm 1 allows any order);
  * the test is eta <= threshold (PreSTO Example 5 and RheoSampling Algorithm 1
    use <=; the PTD appendix writes <); decisions within 1e-5 of the
    threshold are flagged as near-ties;
  * uniforms: u[c][0] drives the test of candidate c, u[v][1] the final draw at
    v; a draw from weights w picks the smallest j with
    sum_{i<=j} w_i > u * sum_i w_i (token-id order).
"""

from __future__ import annotations

import numpy as np

UNVISITED, ACCEPTED, REJECTED = 0, 1, 2
TIE = 1e-5


def target_probs(logits_row, temperature: float) -> np.ndarray:
    """p = softmax(l / T) in float64."""
    z = np.asarray(logits_row, dtype=np.float64) / float(temperature)
    e = np.exp(z - z.max())
    return e / e.sum()


def inverse_cdf(weights: np.ndarray, u: float):
    """Smallest j with sum_{i<=j} w_i > u * sum_i w_i; also returns the normalised CDF."""
    w = np.asarray(weights, dtype=np.float64)
    cum = np.cumsum(w)
    total = cum[-1]
    if not total > 0.0:
        raise ValueError("cannot sample from a distribution with no mass")
    F = cum / total
    j = int(np.searchsorted(cum, u * total, side="right"))
    if j >= w.size:                       # u * total rounded onto the total
        j = int(np.nonzero(w > 0)[0][-1])
    return j, F


class UniformChooser:
    """Takes every decision with the supplied uniforms and records it.

    Each record is (kind, node, outcome, flagged, extra); ``flagged`` marks a
    near-tie (|u - threshold| < 1e-5, or u within 1e-5 of the CDF step on either
    side of the drawn token).  For a draw, ``extra`` holds (F(j-1), F(j)) of the
    normalised CDF so another implementation's token can be checked against it.
    """

    def __init__(self, uniforms: np.ndarray, tie: float = TIE):
        self.u = np.asarray(uniforms)
        self.tie = tie
        self.decisions = []

    def test(self, node: int, threshold: float) -> bool:
        u = float(self.u[node][0])
        out = u <= threshold
        self.decisions.append(("test", node, out, abs(u - threshold) < self.tie, threshold))
        return out

    def sample(self, node: int, weights: np.ndarray) -> int:
        u = float(self.u[node][1])
        j, F = inverse_cdf(weights, u)
        lo = float(F[j - 1]) if j > 0 else 0.0
        hi = float(F[j])
        flagged = abs(hi - u) < self.tie or (j > 0 and abs(lo - u) < self.tie)
        self.decisions.append(("sample", node, j, flagged, (lo, hi, F)))
        return j


def _normalise(r: np.ndarray) -> np.ndarray:
    s = r.sum()
    if not s > 0.0:
        raise ValueError("residual distribution has no mass left")
    return r / s


def rheo_verify_sequence(parent, token, sampled, p_of, qtilde_of, chooser):
    """Verify one tree.  Node 0 is the root (the last committed token).

    parent/token/sampled are sequence-local arrays; p_of(v) returns the target
    distribution at node v; qtilde_of(v) returns the distribution v's sampled
    child was drawn from (None if v has none).  Returns (status, path, token)
    where status[v] is ACCEPTED / REJECTED / UNVISITED, path lists the accepted
    nodes from the root, and token is the final draw at the last path node.
    """
    n = len(parent)
    children = [[] for _ in range(n)]
    for c in range(1, n):
        children[int(parent[c])].append(c)
    status = np.zeros(n, dtype=np.uint8)
    status[0] = ACCEPTED
    path = [0]
    v = 0
    while True:
        cands = list(children[v])                 # ascending node id
        samp = [c for c in cands if sampled[c]]
        if len(samp) > 1:
            raise ValueError(f"node {v} has more than one sampled child")
        toks = [int(token[c]) for c in cands]
        if len(set(toks)) != len(toks):
            raise ValueError(f"children of node {v} repeat a token")
        nxt = None
        if samp:
            s = samp[0]
            p = p_of(v)
            qt = qtilde_of(v)
            if qt is None:
                raise ValueError(f"node {v} has a sampled child but no draft distribution")
            ts = int(token[s])
            if not qt[ts] > 0.0:
                raise ValueError(f"sampled token of node {s} has no draft mass")
            if chooser.test(s, min(1.0, p[ts] / qt[ts])):
                nxt = s
            else:
                status[s] = REJECTED
                cands.remove(s)
                r = _normalise(np.maximum(0.0, p - qt))
        else:
            r = p_of(v)
        if nxt is None:
            for c in cands:
                if chooser.test(c, float(r[int(token[c])])):
                    nxt = c
                    break
                status[c] = REJECTED
                r = r.copy()
                r[int(token[c])] = 0.0
                r = _normalise(r)
        if nxt is not None:
            status[nxt] = ACCEPTED
            path.append(nxt)
            v = nxt
            continue
        return status, path, chooser.sample(v, r)


def greedy_verify_sequence(parent, token, sampled, logits_of, decisions=None):
    """Greedy verification (T = 0) of one tree, Progressive Tree Drafting Section 3.2: the
    verification token of node n is its highest-probability prediction (the argmax of its
    logits, smallest id among equal maxima); the edge to a child is eligible when the child's
    token is that verification token; X' follows eligible edges from the root and ends with the
    verification token of the last node.  The children are looked at in the stochastic walk's
    order (sampled child first, then ascending id): each one passed over before the eligible
    one is marked rejected.  Returns (status, path, token) like rheo_verify_sequence."""
    from .scorer import argmax_token

    n = len(parent)
    children = [[] for _ in range(n)]
    for c in range(1, n):
        children[int(parent[c])].append(c)
    status = np.zeros(n, dtype=np.uint8)
    status[0] = ACCEPTED
    path = [0]
    v = 0
    while True:
        toks = [int(token[c]) for c in children[v]]
        if len(set(toks)) != len(toks):
            raise ValueError(f"children of node {v} repeat a token")
        a = argmax_token(logits_of(v))
        order = [c for c in children[v] if sampled[c]] + [c for c in children[v] if not sampled[c]]
        nxt = None
        for c in order:
            hit = int(token[c]) == a
            if decisions is not None:
                decisions.append(("test", c, hit, False, None))
            if hit:
                nxt = c
                break
            status[c] = REJECTED
        if nxt is None:
            if decisions is not None:
                decisions.append(("sample", v, a, False, None))
            return status, path, a
        status[nxt] = ACCEPTED
        path.append(nxt)
        v = nxt


def node_terminal_stats(logits_row, temperature, qtilde, det_tokens, u1):
    """Vocabulary statistics of one node, as the walk would use them if it ended there.

    M = max l/T, S = sum exp(l/T - M) (so p = exp(l/T - M) / S),
    Z = sum (p - q~)+ (0 without a draft), and the token drawn with u1 from the
    final residual: (p - q~)+ (or p) with the tokens of the node's deterministic
    children zeroed.  Returns (M, S, Z, token, (F(j-1), F(j))).
    """
    z = np.asarray(logits_row, dtype=np.float64) / float(temperature)
    M = float(z.max())
    e = np.exp(z - M)
    S = float(e.sum())
    p = e / S
    if qtilde is not None:
        resid = np.maximum(0.0, p - np.asarray(qtilde, dtype=np.float64))
        Z = float(resid.sum())
        r = resid
    else:
        Z = 0.0
        r = p.copy()
    for t in det_tokens:
        r[int(t)] = 0.0
    if not r.sum() > 0.0:
        return M, S, Z, -1, (0.0, 0.0)
    j, F = inverse_cdf(r, float(u1))
    return M, S, Z, j, (float(F[j - 1]) if j > 0 else 0.0, float(F[j]))


def verify_workload(w, seqs=None):
    """Run the verification walk of every (or the given) sequence of a workload.

    Returns a list, per sequence, of dicts with node_status (sequence-local),
    path (sequence-local ids), bonus token and the chooser's decision records.  A sequence
    with temperature 0 is verified greedily (greedy_verify_sequence).
    """
    if seqs is None:
        seqs = range(w.B)
    results = []
    for b in seqs:
        s, e = int(w.node_offsets[b]), int(w.node_offsets[b + 1])
        T = float(w.temperature[b])
        cache = {}

        def p_of(v, s=s, T=T, cache=cache):
            if v not in cache:
                cache[v] = target_probs(_logits_f64(w, s + v), T)
            return cache[v]

        def qtilde_of(v, s=s):
            r = int(w.draft_row[s + v])
            return None if r < 0 else dense_draft_row(w, r)

        if T == 0.0:                          # greedy decoding
            dec = []
            status, path, bonus = greedy_verify_sequence(w.parent[s:e], w.token[s:e], w.sampled[s:e],
                                                         lambda v, s=s: _logits_f64(w, s + v), dec)
            results.append({"status": status, "path": path, "bonus": bonus, "decisions": dec})
            continue
        ch = UniformChooser(w.uniforms[s:e])
        status, path, bonus = rheo_verify_sequence(w.parent[s:e], w.token[s:e], w.sampled[s:e],
                                                   p_of, qtilde_of, ch)
        results.append({"status": status, "path": path, "bonus": bonus,
                        "decisions": ch.decisions})
    return results


def dense_draft_row(w, r):
    """Draft row r over the whole vocabulary in float64.  A sparse row (RheoSampling Section
    3.2: the draft's logits truncated to their top entries before the softmax) is its support
    values placed at their token ids, zero everywhere else -- the distribution the sampled
    token was drawn from, so the verification rule applies to it unchanged."""
    if getattr(w, "draft_k", 0):
        q = np.zeros(w.V, dtype=np.float64)
        idx = np.asarray(w.draft_idx[r], dtype=np.int64)
        if len(set(idx.tolist())) != idx.size or idx.min() < 0 or idx.max() >= w.V:
            raise ValueError("sparse draft row: support ids must be distinct tokens of the vocabulary")
        q[idx] = np.asarray(w.draft_val[r], dtype=np.float64)
        return q
    return np.asarray(w.draft[r], dtype=np.float64)


def _logits_f64(w, v):
    row = w.logits[v]
    if w.dtype == "bf16":
        return (np.asarray(row, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(row, dtype=np.float64)
