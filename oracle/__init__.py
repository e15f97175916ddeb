"""Reference oracle for the tree-masked scoring pass (test infrastructure only).

Plain, slow, float64 CPU definitions of what the scoring pass computes, written
from the pages:

* tree visibility, depths and positions (Progressive Tree Drafting, Section 3.1,
  "Tree Construction": a node sees exactly itself and its ancestors, and its
  position follows from the size of that set);
* tree-masked attention over a paged prefix plus the node's ancestors (the same
  section; RheoSampling and PreSTO score trees / suffix batches with the target
  model in one forward pass);
* temperature softmax and RheoVerification / sequential rejection
  (RheoSampling, Section 3.3 Algorithm 1 and Section 5.4; Progressive Tree
  Drafting, Section 3.2 and Appendix E);
* PreSTO's log-acceptance and the MH walk over the prefetched subtree (PreSTO,
  Section 3.2 Example 3 / Equation 6, Appendix B.1 Equations 7-9, Appendix B.3
  Example 5);
* per-token scores of sampled tokens (log p0, log q_tau, entropy of p0; PreSTO
  Appendix D.3) and greedy verification (Progressive Tree Drafting, Section 3.2);
* the prefetching tree of a PreSTO batch (BFS and predictive rules, rounded and
  predicted reaching weights; PreSTO Section 3.2 step (1), Appendix C).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything here.  The HIP library never does, and this
package imports nothing from it.
"""

from .tree import tree_prep, ancestor_words  # noqa: F401
from .attention import tree_attention, node_attention  # noqa: F401
from .verify import (  # noqa: F401
    ACCEPTED, REJECTED, UNVISITED, UniformChooser, target_probs, rheo_verify_sequence,
    verify_workload, inverse_cdf, node_terminal_stats, dense_draft_row, greedy_verify_sequence,
)
from .presto import presto_states, presto_log_accept, presto_walk, presto_workload  # noqa: F401
from .scorer import token_scores, score_rows, argmax_token  # noqa: F401
from . import prefetch  # noqa: F401
