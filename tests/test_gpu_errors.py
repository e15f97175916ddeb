"""Device-detected errors, sentinel outputs, -inf logits and run-to-run determinism.

Each error case corrupts one input of the middle sequence of a three-sequence batch and
checks (a) the status bit, (b) the sentinel outputs of that sequence (attention rows
zero with lse -inf for errors of its tree or prefix; path_len 0, path -1, bonus -1 and
node_status 0 for any error), and (c) that the other two sequences still match the
oracle.  Every corrupted value is one the kernels check before they use it (parents are
only compared; block ids are clamped to block 0 before any copy; child tokens are
range-checked before the logits / draft reads; logits, temperatures and draft masses
only enter arithmetic), so each kernel still runs in bounds and exits normally.
"""

import sys

import numpy as np
import pytest

import oracle
from workloads import gen
import gpu_util as gu

pytestmark = pytest.mark.gpu

BAD = 1            # the corrupted sequence
GOOD = [0, 2]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _batch(seed=5, V=4096, T=1.0, tree="random", n=(20, 24, 18), L=(300, 517, 64)):
    return gen.tree_batch(seed, B=3, prefix_len=list(L), tree=tree, n_nodes=list(n), Hq=32, Hkv=8,
                          D=128, dtype="bf16", V=V, temperature=T, max_depth=5)


def _children(w, b, v_local):
    s, e = int(w.node_offsets[b]), int(w.node_offsets[b + 1])
    return [c for c in range(s + 1, e) if int(w.parent[c]) == v_local]


def _check_good(w, got):
    nodes = [v for b in GOOD for v in w.seq_nodes(b)]
    gu.check_attention(w, got, nodes)
    gu.check_verify(w, got, GOOD)


def _check_verify_sentinel(w, got, b=BAD):
    s, e = int(w.node_offsets[b]), int(w.node_offsets[b + 1])
    assert int(got["path_len"][b]) == 0
    assert int(got["bonus"][b]) == -1
    assert (got["path"][b] == -1).all()
    assert (got["node_status"][s:e] == 0).all()


def _check_attn_sentinel(w, got, b=BAD):
    s, e = int(w.node_offsets[b]), int(w.node_offsets[b + 1])
    assert (got["out"][s:e] == 0).all()
    assert np.isneginf(got["lse"][s:e]).all()


def _run(w, bit, attn_sentinel, max_path=64):
    import tree_masked_verification_attn_amd as tav

    got = gu.run(w, max_path=max_path)
    names = tav.device_status_names(got["status"])
    _say("status", names)
    assert got["status"] & bit, names
    _check_verify_sentinel(w, got)
    if attn_sentinel:
        _check_attn_sentinel(w, got)
    return got


def test_bad_parent():
    import tree_masked_verification_attn_amd as tav

    w = _batch()
    s = int(w.node_offsets[BAD])
    w.parent[s + 5] = 7                          # a later node
    got = _run(w, 1 << 0, True)                  # TAV_DEV_BAD_PARENT
    _check_good(w, got)


def test_block_id_out_of_range():
    w = _batch()
    w.block_table[BAD, 3] = w.k_cache.shape[0] + 11
    got = _run(w, 1 << 2, True)                  # TAV_DEV_BAD_BLOCK
    _check_good(w, got)


def test_negative_block_id():
    w = _batch()
    w.block_table[BAD, 0] = -1
    got = _run(w, 1 << 2, True)
    _check_good(w, got)


def test_child_token_out_of_range():
    w = _batch()
    c = _children(w, BAD, 0)[-1]
    w.token[c] = w.V + 3
    got = _run(w, 1 << 3, False)                 # TAV_DEV_BAD_TOKEN
    _check_good(w, got)
    gu.check_attention(w, got, list(w.seq_nodes(BAD)))   # attention of that sequence is unaffected


def test_duplicate_sibling_tokens():
    w = _batch(tree="star", n=(9, 12, 7))
    kids = _children(w, BAD, 0)
    w.token[kids[2]] = w.token[kids[1]]
    got = _run(w, 1 << 4, False)                 # TAV_DEV_DUP_SIBLING_TOKEN
    _check_good(w, got)


def test_two_sampled_children():
    w = _batch(tree="star", n=(9, 12, 7))
    kids = _children(w, BAD, 0)
    w.sampled[kids[1]] = 1
    got = _run(w, 1 << 5, False)                 # TAV_DEV_MULTI_SAMPLED
    _check_good(w, got)


def test_sampled_child_without_draft_row():
    w = _batch()
    s = int(w.node_offsets[BAD])
    w.draft_row[s] = -1                          # the root has a sampled child
    got = _run(w, 1 << 6, False)                 # TAV_DEV_NO_DRAFT
    _check_good(w, got)


def test_sampled_token_without_draft_mass():
    w = _batch()
    s = int(w.node_offsets[BAD])
    ks = [c for c in _children(w, BAD, 0) if w.sampled[c]][0]
    w.draft = w.draft.copy()
    w.draft[int(w.draft_row[s]), int(w.token[ks])] = 0.0
    got = _run(w, 1 << 7, False)                 # TAV_DEV_ZERO_DRAFT_MASS
    _check_good(w, got)


@pytest.mark.parametrize("bad_value", [np.nan, np.inf])
def test_nonfinite_logits(bad_value):
    w = _batch()
    s = int(w.node_offsets[BAD])
    bits = gen.f32_to_bf16_bits(np.array([bad_value], np.float32))[0]
    w.logits[s + 2, 1234] = bits
    got = _run(w, 1 << 8, False)                 # TAV_DEV_NONFINITE_LOGITS
    _check_good(w, got)


@pytest.mark.parametrize("bad_t", [-1.0, np.nan, np.inf])
def test_bad_temperature(bad_t):
    w = _batch()
    w.temperature = w.temperature.copy()
    w.temperature[BAD] = bad_t
    got = _run(w, 1 << 14, False)                # TAV_DEV_BAD_TEMPERATURE
    _check_good(w, got)


def test_path_overflow():
    w = gen.tree_batch(8, B=3, prefix_len=[40, 50, 60], tree="chain", n_nodes=[6, 12, 5], Hq=8, Hkv=2,
                       D=128, dtype="bf16", V=1024, temperature=1.0)
    w.uniforms[:, 0] = 0.0                       # every first-tested candidate is accepted
    got = _run(w, 1 << 10, False, max_path=8)    # TAV_DEV_PATH_OVERFLOW on the 12-node chain only
    _check_good(w, got)


def test_negative_infinite_logits_are_zero_mass():
    """-inf logits are allowed (p = 0 there): a child whose token has -inf logit is rejected,
    and no final draw lands on a -inf token."""
    w = _batch(seed=9)
    ninf = gen.f32_to_bf16_bits(np.array([-np.inf], np.float32))[0]
    rng = np.random.default_rng(0)
    for v in range(w.N):
        w.logits[v, rng.choice(w.V, size=w.V // 3, replace=False)] = ninf
    for b in range(w.B):                         # one deterministic child per sequence hits -inf
        s = int(w.node_offsets[b])
        det = [c for c in _children(w, b, 0) if not w.sampled[c]]
        if det:
            w.logits[s, int(w.token[det[0]])] = ninf
    got = gu.run(w)
    assert got["status"] == 0, got["status"]
    gu.check_attention(w, got)
    gu.check_verify(w, got)
    gu.check_node_stats(w, got, range(w.N))
    for b in range(w.B):
        v = int(got["path"][b][int(got["path_len"][b]) - 1]) + int(w.node_offsets[b])
        assert gen.bf16_bits_to_f32(w.logits[v, int(got["bonus"][b])]) != -np.inf


def test_two_runs_bit_identical():
    """Two calls on the same inputs give bit-identical outputs, with several deterministic
    children of one node inside the same 512-token chunk of the vocabulary (their weights are
    taken out of that chunk in a fixed order)."""
    w = gen.tree_batch(12, B=3, prefix_len=[900, 3000, 77], tree="star", n_nodes=[40, 33, 9], Hq=32,
                       Hkv=8, D=128, dtype="bf16", V=151936, temperature=0.9)
    for b in range(w.B):
        det = [c for c in _children(w, b, 0) if not w.sampled[c]]
        samp_tok = [int(w.token[c]) for c in _children(w, b, 0) if w.sampled[c]]
        free = [t for t in range(1000, 1512) if t not in samp_tok]
        for i, c in enumerate(det):
            w.token[c] = free[3 * i % len(free)] if b != 2 else free[i]
    first = gu.run(w)
    second = gu.run(w)
    assert first["status"] == 0 and second["status"] == 0
    for key in ("out", "lse", "stats", "term", "node_status", "path", "path_len", "bonus", "mask"):
        a, b = np.asarray(first[key]), np.asarray(second[key])
        assert a.tobytes() == b.tobytes(), key
    gu.check_attention(w, first, [v for b in range(w.B) for v in list(w.seq_nodes(b))[:5]])
    gu.check_verify(w, first)
    gu.check_node_stats(w, first, [int(w.node_offsets[b]) for b in range(w.B)])


def test_many_children_packed_chunks():
    """255 children of one root (more than one wave's worth, most of them past the window of
    following nodes a node's children are gathered from) with the deterministic children's
    tokens packed into one 512-token chunk, and 99 children spread over a few chunks: matches
    the oracle and repeats bit for bit."""
    w = gen.tree_batch(21, B=2, prefix_len=[300, 41], tree="star", n_nodes=[256, 100], Hq=16, Hkv=4,
                       D=128, dtype="bf16", V=8192, temperature=0.8)
    for b in range(w.B):
        kids = _children(w, b, 0)
        det = [c for c in kids if not w.sampled[c]]
        samp_tok = {int(w.token[c]) for c in kids if w.sampled[c]}
        lo, hi = (1024, 1536) if b == 0 else (1000, 2200)
        free = [t for t in range(lo, hi) if t not in samp_tok]
        step = 1 if b == 0 else 7
        assert len(det) <= len(free)
        for i, c in enumerate(det):
            w.token[c] = free[(step * i) % len(free)]
        assert len({int(w.token[c]) for c in kids}) == len(kids)
    _say("many children packed chunks")
    first = gu.run(w)
    second = gu.run(w)
    assert first["status"] == 0 and second["status"] == 0, (first["status"], second["status"])
    for key in ("stats", "term", "node_status", "path", "path_len", "bonus"):
        a, b = np.asarray(first[key]), np.asarray(second[key])
        assert a.tobytes() == b.tobytes(), key
    gu.check_verify(w, first)
    gu.check_node_stats(w, first, [int(w.node_offsets[b]) for b in range(w.B)])
