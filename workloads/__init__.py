"""Seeded synthetic inputs for the tree-masked scoring pass.

This package only *creates inputs*: token trees, paged KV caches, node
queries/keys/values, target logits, draft distributions, uniforms and the
PreSTO per-token log-probability arrays.  It computes none of what the scoring
pass computes (no attention, no temperature softmax of target logits, no
residuals, no accept/reject decisions, no log-acceptance), so the oracle and the
HIP path can both draw their inputs from here without sharing any of the
method's arithmetic.  Random numbers the method itself consumes (the
verification uniforms and the MH uniforms) are generated here and passed in.
"""

from .gen import (  # noqa: F401
    Workload,
    PrestoInputs,
    make,
    tree_batch,
    presto_batch,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    as_f64,
    CONFIG_NAMES,
    CONFIG_DESCRIPTIONS,
)
