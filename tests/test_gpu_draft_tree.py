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


def build_both(seed, B, V, D, K, slots, m, hybrid, S, R, T):
    import tree_masked_verification_attn_amd as tav

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
                rows[b, j] = gen.draft_logits_row(seed, b, c, V)
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
