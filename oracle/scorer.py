"""Per-token scores of sampled tokens from the unprocessed logits (test infrastructure only).

PreSTO, Appendix D.3 (the patched sampler): for each sampled token x_t the forward pass
returns (i) log q_tau(x_t | x_{0:t-1}), the proposal log-probability from the processed
logits -- here temperature tau, q_tau = softmax(l / tau); (ii) the base-model
log-probability log p0(x_t | x_{0:t-1}) from the unprocessed copy, p0 = softmax(l); and
(iii) the full-vocabulary entropy of p0 in natural log, H_t = -sum_u p0(u) log p0(u).
These are the per-token inputs of the log-acceptance (PreSTO Section 3.2, Example 3).

Progressive Tree Drafting, Section 3.2: under greedy decoding the verification token of a
node is the model's highest-probability prediction, i.e. the argmax of the logits (the
reading here: the smallest token id among equal maxima).
"""

from __future__ import annotations

import numpy as np


def _lse(z: np.ndarray) -> float:
    m = float(np.max(z))
    if m == -np.inf:
        return -np.inf
    return m + float(np.log(np.sum(np.exp(z - m))))


def argmax_token(logits_row) -> int:
    """Smallest token id with the largest logit."""
    l = np.asarray(logits_row, dtype=np.float64)
    return int(np.flatnonzero(l == l.max())[0])


def token_scores(logits_row, token: int, tau: float):
    """(log p0(token), log q_tau(token), H(p0), argmax) of one row, in float64."""
    l = np.asarray(logits_row, dtype=np.float64)
    lp0 = float(l[token]) - _lse(l)
    z = l / float(tau)
    lq = float(z[token]) - _lse(z)
    p = np.exp(l - _lse(l))
    nz = p > 0.0
    H = float(-np.sum(p[nz] * np.log(p[nz])))
    return lp0, lq, H, argmax_token(l)


def score_rows(logits, tokens, tau: float, dtype: str = "f32"):
    """token_scores of every row of a [N, V] array (bf16 bits or float32)."""
    rows = np.asarray(logits)
    if dtype == "bf16":
        rows = (np.ascontiguousarray(rows, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    out = np.zeros((rows.shape[0], 3), np.float64)
    am = np.zeros(rows.shape[0], np.int64)
    for i in range(rows.shape[0]):
        a, b, c, d = token_scores(rows[i], int(tokens[i]), tau)
        out[i] = (a, b, c)
        am[i] = d
    return out, am
