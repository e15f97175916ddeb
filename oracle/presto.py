"""PreSTO log-acceptance and the MH walk over the prefetched subtree.

PreSTO, Section 3.2:
  * each acceptance (left) child carries a suffix-resampling request with cut c;
    its proposal keeps the state's prefix up to c and replaces tokens c+1..T
    (Equation 5); a rejection (right) child keeps its parent's state;
  * Equation 6 (Example 3; derived in Appendix B.1 from Equations 7-9):
      log A(y, x) = min{0, log q_tau(x_{c+1:T}|x_{0:c}) - log q_tau(y_{c+1:T}|x_{0:c})
                           + alpha (log p0(y_{c+1:T}|x_{0:c}) - log p0(x_{c+1:T}|x_{0:c}))},
    each sequence-level term being the sum of per-token log-probabilities over
    t = c+1..T;
  * step (3) / Appendix B.3 Example 5: from the subtree root, at node v draw u
    and go to the acceptance child iff u <= A(v+, v), else to the rejection
    child; a leaf, or an acceptance child whose request was deferred, ends the
    walk for this batch (Section 3.2 (1)), as does the cap on transitions
    (Section 3.2, MHTransition runs at most K - k transitions).

State arrays are materialised explicitly: the state of every node is the full
per-token array pair (log p0, log q_tau) at t = 1..T.
"""

from __future__ import annotations

import numpy as np

TIE = 1e-5


def presto_states(pr):
    """(lp0[T], lq[T]) of every prefetching-tree node; None where the state is not
    available in this batch (a deferred request and, formally, its subtree)."""
    M = len(pr.pf_parent)
    states = [None] * M
    states[0] = (np.asarray(pr.root_lp0, np.float64), np.asarray(pr.root_lq, np.float64))
    for v in range(1, M):
        par = int(pr.pf_parent[v])
        if not (0 <= par < v):
            raise ValueError("prefetch tree parent must be an earlier node")
        if states[par] is None:
            continue
        if pr.pf_is_accept[v]:
            i = int(pr.pf_request[v])
            if i < 0:
                continue                              # deferred request
            c = int(pr.cut[i])
            a, b = int(pr.suffix_off[i]), int(pr.suffix_off[i + 1])
            if b - a != pr.T - c:
                raise ValueError("request suffix must cover tokens c+1..T")
            lp0 = states[par][0].copy()
            lq = states[par][1].copy()
            lp0[c:] = np.asarray(pr.lp0[a:b], np.float64)     # tokens t = c+1..T
            lq[c:] = np.asarray(pr.lq[a:b], np.float64)
            states[v] = (lp0, lq)
        else:
            states[v] = states[par]
    return states


def presto_log_accept(pr, states=None):
    """log A of every request in the batch (Equation 6), float64, indexed by request id."""
    if states is None:
        states = presto_states(pr)
    R = len(pr.cut)
    logA = np.full(R, np.nan)
    for v in range(1, len(pr.pf_parent)):
        i = int(pr.pf_request[v])
        if not pr.pf_is_accept[v] or i < 0:
            continue
        x = states[int(pr.pf_parent[v])]
        y = states[v]
        c = int(pr.cut[i])
        log_q_x = x[1][c:].sum()
        log_q_y = y[1][c:].sum()
        log_p_x = x[0][c:].sum()
        log_p_y = y[0][c:].sum()
        logA[i] = min(0.0, log_q_x - log_q_y + pr.alpha * (log_p_y - log_p_x))
    return logA


def presto_walk(pr, logA, u=None, tie=TIE):
    """MH transitions over the prefetched subtree.

    Returns (path of tree nodes from the root, number of completed transitions,
    decision records (node, accepted?, flagged near-tie)).
    """
    if u is None:
        u = pr.u
    M = len(pr.pf_parent)
    acc_child = [-1] * M
    rej_child = [-1] * M
    for v in range(1, M):
        p = int(pr.pf_parent[v])
        if pr.pf_is_accept[v]:
            acc_child[p] = v
        else:
            rej_child[p] = v
    v, k, path, dec = 0, 0, [0], []
    while k < pr.max_transitions:
        a, r = acc_child[v], rej_child[v]
        if a < 0 or r < 0:
            break                                   # leaf of the prefetched subtree
        i = int(pr.pf_request[a])
        if i < 0:
            break                                   # proposal deferred to a later batch
        A = float(np.exp(logA[i]))
        uu = float(u[v])
        go = uu <= A
        dec.append((v, go, abs(uu - A) < tie))
        v = a if go else r
        k += 1
        path.append(v)
    return path, k, dec


def presto_workload(pr):
    states = presto_states(pr)
    logA = presto_log_accept(pr, states)
    path, k, dec = presto_walk(pr, logA)
    return {"logA": logA, "path": path, "k_delta": k, "decisions": dec}
