"""Exact enumeration of every random outcome of a decision procedure.

A procedure takes a "chooser" and calls chooser.test(node, threshold) (true with
probability threshold for a uniform u <= threshold) and chooser.sample(node,
weights) (index j with probability w_j / sum w).  ``enumerate_outcomes`` replays
the procedure once per branch, so every result comes with its exact probability
(no Monte Carlo).
"""

import numpy as np


class Fork(Exception):
    def __init__(self, options):
        super().__init__("fork")
        self.options = options


class ForkChooser:
    def __init__(self, forced):
        self.forced = forced
        self.i = 0

    def _next(self, options):
        if self.i < len(self.forced):
            out = self.forced[self.i]
            self.i += 1
            return out
        raise Fork(options)

    def test(self, node, threshold):
        t = min(1.0, max(0.0, float(threshold)))
        return self._next([(True, t), (False, 1.0 - t)])

    def sample(self, node, weights):
        w = np.asarray(weights, dtype=np.float64)
        w = w / w.sum()
        return self._next([(int(j), float(w[j])) for j in np.nonzero(w > 0)[0]])


def enumerate_outcomes(run):
    """run(chooser) -> result; returns [(result, probability)] over all branches."""
    out = []
    stack = [([], 1.0)]
    while stack:
        forced, prob = stack.pop()
        ch = ForkChooser(forced)
        try:
            res = run(ch)
        except Fork as f:
            for o, pr in f.options:
                if pr > 0.0:
                    stack.append((forced + [o], prob * pr))
            continue
        out.append((res, prob))
    return out
