"""GPU parity of the draft-tree construction (tav_draft_expand / tav_draft_prune) with the oracle.

Both sides build the same trees depth by depth: at each depth the drafter's logits are those of
the parents the GPU selected (a seeded function of the candidate id), and the oracle's own
selection must name the same parents; the pruned trees (parents, tokens, sampled flags, candidate
ids) must be identical and the sparse draft rows equal (ids exactly, q~ within 1e-6 relative).
Comparison of a tree stops at its first decision the oracle flags as a near-tie.  The trees then
go through the scoring pass's verification as they are.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.draft_tree as odt
from workloads import gen
import gpu_util as gu

pytestmark = pytest.mark.gpu


def build_both(seed, B, V, D, K, slots, m, hybrid, S, R, T, row_fn=None):
    import tree_masked_verification_attn_amd as tav

    row_fn = row_fn or gen.draft_logits_row
    hyb = {"all": tav.TAV_DRAFT_HYBRID_ALL, "first": tav.TAV_DRAFT_HYBRID_FIRST, "none": tav.TAV_DRAFT_HYBRID_NONE}
    prm = tav.draft_params(num_seqs=B, vocab=V, depth=D, expand_k=K, slots=slots, lead_m=m, hybrid=hyb[hybrid],
                           support=S, budget=R, temperature=T, eps=1e-6)
    ws = torch.zeros((tav.tav_draft_workspace_size(prm) + 7) // 8, dtype=torch.float64, device="cuda")
    front = torch.full((B, K), -5, dtype=torch.int32, device="cuda")
    ora = [odt.DraftTreeBuilder(V, D, K, slots, m, hybrid, S, R, T) for _ in range(B)]
    live = [True] * B                          # compared up to the first flagged near-tie
    gpu_front = [[0] for _ in range(B)]
    for d in range(1, D + 1):
        kd = len(gpu_front[0])
        rows = np.zeros((B, kd, V), np.uint16)
        uni = np.zeros((B, kd), np.float32)
        for b in range(B):
            for j, c in enumerate(gpu_front[b]):
                rows[b, j] = row_fn(seed, b, c, V)
                uni[b, j] = gen.draft_uniform(seed, b, d, j)
        lg = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).cuda()
        tav.tav_draft_expand(prm, d, lg, torch.from_numpy(uni).cuda(), front, ws)
        torch.cuda.synchronize()
        nxt = front.cpu().numpy()
        for b in range(B):
            if live[b]:
                ot = ora[b]
                ot.expand(d, [gen.bf16_bits_to_f32(rows[b, j]).astype(np.float64) for j in range(kd)], uni[b])
                if ot.ties:
                    live[b] = False
                elif d < D:                    # after the last depth no parents are named
                    assert list(ot.frontier) == [int(x) for x in nxt[b] if x >= 0], (b, d)
        gpu_front = [[int(x) for x in nxt[b] if x >= 0] for b in range(B)]
    n = R + 1
    out = {k: torch.full((B * n,), -9, dtype=torch.int32, device="cuda")
           for k in ("parent", "token", "cand_id", "draft_row")}
    out["sampled"] = torch.full((B * n,), 9, dtype=torch.uint8, device="cuda")
    out["draft_idx"] = torch.full((B * n, S), -9, dtype=torch.int32, device="cuda")
    out["draft_val"] = torch.full((B * n, S), -9.0, dtype=torch.float32, device="cuda")
    tav.tav_draft_prune(prm, out["parent"], out["token"], out["sampled"], out["cand_id"], out["draft_row"],
                        out["draft_idx"], out["draft_val"], ws)
    torch.cuda.synchronize()
    assert tav.tav_read_status(ws) == 0
    got = {k: v.cpu().numpy() for k, v in out.items()}
    compared = 0
    for b in range(B):
        if not live[b]:
            continue
        parent, token, sampled, cids, orows = ora[b].prune()
        if ora[b].ties:
            continue
        sl = slice(b * n, (b + 1) * n)
        np.testing.assert_array_equal(got["parent"][sl], parent)
        np.testing.assert_array_equal(got["token"][sl], token)
        np.testing.assert_array_equal(got["sampled"][sl], sampled)
        np.testing.assert_array_equal(got["cand_id"][sl], cids)
        for v in range(n):
            if orows[v] is None:
                assert got["draft_row"][b * n + v] == -1
            else:
                r = got["draft_row"][b * n + v]
                assert r == b * n + v
                np.testing.assert_array_equal(got["draft_idx"][r], orows[v][0])
                np.testing.assert_allclose(got["draft_val"][r], orows[v][1], rtol=1e-6, atol=1e-9)
        compared += 1
    return got, compared


CASES = {
    # name: (B, V, D, K, slots, m, hybrid, S, R, T)
    "c5_shape": (4, 151936, 10, 8, 8, 1, "all", 128, 127, 1.0),
    "c2_shape": (1, 151936, 6, 8, 8, 1, "first", 128, 59, 0.7),
    "small_m0": (3, 4096, 4, 4, 5, 0, "all", 32, 40, 1.3),
    "plain": (2, 2048, 3, 3, 4, 0, "none", 16, 20, 1.0),
}


@pytest.mark.parametrize("seed", [10086, 1, 2])
@pytest.mark.parametrize("case", sorted(CASES))
def test_draft_tree_parity(case, seed):
    got, compared = build_both(seed, *CASES[case])
    assert compared >= 1


def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def tied_row(seed, b, c, V, S=16, n_top=24):
    """n_top tokens at logit 2, the rest at -3: the support is the S smallest of those ids (ties at
    the threshold), q = 1/S exactly on it, so every proxy and path score is a power of two and
    scores tie exactly across parents and slots (the next parents and the prune go by the tie
    rule)."""
    rng = np.random.default_rng([seed, b, c, 17])
    z = np.full(V, -3.0, np.float32)
    z[rng.choice(V, n_top, replace=False)] = 2.0
    return _bf16_bits(z)


def one_stride_row(seed, b, c, V, S=128):
    """S distinct logits in [1, 3) on tokens 8192 k + (0..7) (one 8-token group every 8192 tokens),
    every other token at 0: the largest logits gather in few groups, far more than 4096 tokens
    share the next value, and the top S are still distinct."""
    rng = np.random.default_rng([seed, b, c, 29])
    ids = np.array([8192 * k + e for k in range(V // 8192 + 1) for e in range(8)])
    ids = ids[ids < V][:S]
    assert ids.size == S
    z = np.zeros(V, np.float32)
    z[ids] = 1.0 + rng.permutation(S) / 64.0
    return _bf16_bits(z)


def test_draft_tree_exact_ties():
    """Exact score ties everywhere (powers of two) and logits tied at the support's threshold: the
    frontier, the prune and the support all go by their tie rules on both sides."""
    got, compared = build_both(3, 2, 4096, 4, 4, 4, 1, "all", 16, 30, 1.0, row_fn=tied_row)
    assert compared == 2


def test_draft_tree_top_in_few_groups():
    """Rows whose largest logits sit in a few 8-token groups and whose remaining tokens all tie:
    the support is still the S largest (the select does not rely on the largest logits being
    spread over the row)."""
    got, compared = build_both(5, 1, 151936, 3, 2, 4, 1, "all", 128, 8, 1.0, row_fn=one_stride_row)
    assert compared == 1


def test_draft_tree_feeds_the_scoring_pass():
    """Trees built on the GPU, verified by the scoring pass with their sparse draft rows."""
    B, V, D, K, slots, m, hybrid, S, R, T = 2, 4096, 5, 4, 4, 1, "all", 64, 30, 1.0
    got, _ = build_both(7, B, V, D, K, slots, m, hybrid, S, R, T)
    n = R + 1
    w = gen.tree_batch(7, B=B, prefix_len=[100, 40], tree="star", n_nodes=[n, n], Hq=8, Hkv=2, D=128,
                       dtype="bf16", V=V, temperature=T)
    w.parent = got["parent"].astype(np.int32)
    w.token = np.maximum(got["token"], 0).astype(np.int32)
    w.sampled = got["sampled"].astype(np.uint8)
    w.draft_row = got["draft_row"].astype(np.int32)
    w.draft, w.draft_k = None, S
    w.draft_idx = got["draft_idx"].copy()
    w.draft_val = got["draft_val"].copy()
    unused = w.draft_row < 0
    w.draft_idx[unused] = np.arange(S)[None, :]          # rows nobody reads: any valid support
    w.draft_val[unused] = 0.0
    res = gu.run(w)
    assert res["status"] == 0, res["status"]
    gu.check_verify(w, res)
    gu.check_node_stats(w, res, range(w.N))
