"""GPU parity of the per-token scorer and of greedy (T = 0) verification.

Scorer (PreSTO Appendix D.3): log p0 and log q_tau of the sampled token, the entropy of p0 and
the argmax of each row against the oracle's float64 values; tolerance 1e-4 absolute plus 1e-5
relative for the float outputs (the kernel sums in float per thread and in float64 across
threads), the argmax exact.  The scores then feed PreSTO's log-acceptance: the log A of a
prefetch batch whose per-token log-probabilities come from logits through the scorer matches
the oracle's chain within 1e-3.  Greedy verification: the walk and every node's statistics
match the oracle's greedy walk exactly.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import device as wdev
from workloads import gen
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _scores(logits_np, tokens, tau, dtype):
    import tree_masked_verification_attn_amd as tav

    N = logits_np.shape[0]
    lg = wdev._store_tensor(logits_np, dtype, "cuda")
    tok = torch.from_numpy(np.asarray(tokens, np.int32)).cuda()
    out = [torch.full((N,), 7.0, device="cuda") for _ in range(3)]
    am = torch.full((N,), -9, dtype=torch.int32, device="cuda")
    ws = torch.zeros(64, dtype=torch.float64, device="cuda")
    tav.tav_token_scores(lg, tok, tau, ws, *out, am)
    torch.cuda.synchronize()
    return [o.cpu().numpy().astype(np.float64) for o in out], am.cpu().numpy(), tav.tav_read_status(ws)


@pytest.mark.parametrize("dtype,V,tau", [("bf16", 151936, 0.25), ("bf16", 4096, 1.0), ("bf16", 1000, 0.7),
                                         ("f32", 20004, 0.25), ("f32", 8, 2.0), ("bf16", 50000, 0.5),
                                         ("bf16", 3000, 1.0 / 3.0), ("f32", 5000, 0.125)])
def test_scores_match_oracle(dtype, V, tau):
    rng = np.random.default_rng(V)
    N = 37
    x = rng.normal(0.0, 3.0, (N, V)).astype(np.float32)
    x[3, rng.choice(V, V // 2, replace=False)] = -np.inf          # half the row at -inf
    x[5, :] = 1.25                                                 # all equal: argmax 0, entropy log V
    x[6, V // 2] = x[6].max() + 1.0
    x[6, V - 1] = x[6, V // 2]                                     # tie: the smaller id
    if V >= 16:
        x[7, [5, 6]] = x[7].max() + 2.0                            # tie inside one 16-byte unit
        x[8, [V - 2, 1]] = x[8].max() + 2.0                        # tie far apart (first wins)
    stored = gen.f32_to_bf16_bits(x) if dtype == "bf16" else x
    tokens = rng.integers(0, V, N)
    tokens[3] = int(np.flatnonzero(np.isfinite(x[3]))[0])
    (lp0, lq, H), am, status = _scores(stored, tokens, tau, dtype)
    assert status == 0
    ref, ref_am = oracle.score_rows(stored, tokens, tau, dtype)
    for got, col, name in ((lp0, 0, "log p0"), (lq, 1, "log q"), (H, 2, "entropy")):
        np.testing.assert_allclose(got, ref[:, col], rtol=1e-5, atol=1e-4, err_msg=name)
    np.testing.assert_array_equal(am, ref_am)


def test_scores_bad_token_and_nan_row():
    V = 4096
    rng = np.random.default_rng(1)
    x = rng.normal(0.0, 3.0, (4, V)).astype(np.float32)
    x[2, 77] = np.nan
    tokens = np.array([5, V + 3, 9, 11])
    (lp0, lq, H), am, status = _scores(gen.f32_to_bf16_bits(x), tokens, 0.25, "bf16")
    assert status & (1 << 3) and status & (1 << 8)
    assert np.isnan(lp0[1]) and np.isnan(lq[1]) and np.isnan(lp0[2]) and np.isnan(H[2])
    ref, _ = oracle.score_rows(gen.f32_to_bf16_bits(x[[0, 3]]), tokens[[0, 3]], 0.25, "bf16")
    np.testing.assert_allclose(lp0[[0, 3]], ref[:, 0], rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("seed", [10086, 1, 2])
def test_presto_log_accept_from_scored_logits(seed):
    """PreSTO's per-token log p0 / log q_tau of the state and of every suffix computed from logits
    by the scorer, then log A and the walk: against the oracle scorer + oracle log A."""
    import tree_masked_verification_attn_amd as tav

    T, V, tau = 64, 2048, 0.25
    w = gen.presto_batch(seed, T=T, n_pf=10, Hq=8, Hkv=2, D=128, dtype="bf16", alpha=4.0, max_transitions=6,
                         with_attention=False)
    pr = w.presto
    rng = np.random.default_rng(seed)
    rows = T + int(pr.suffix_off[-1])
    logits = gen.f32_to_bf16_bits(rng.normal(0.0, 3.0, (rows, V)).astype(np.float32))
    tokens = rng.integers(0, V, rows)
    ref, _ = oracle.score_rows(logits, tokens, tau, "bf16")
    # oracle chain: scores -> log A
    pr.root_lp0, pr.root_lq = ref[:T, 0].astype(np.float32), ref[:T, 1].astype(np.float32)
    pr.lp0, pr.lq = ref[T:, 0].astype(np.float32), ref[T:, 1].astype(np.float32)
    want = oracle.presto_workload(pr)
    # GPU chain: scorer -> the PreSTO arrays -> tav_presto_accept
    d = wdev.upload(w, "cuda")
    lp0 = torch.empty(rows, device="cuda")
    lq = torch.empty(rows, device="cuda")
    ws = torch.zeros(64, dtype=torch.float64, device="cuda")
    tav.tav_token_scores(wdev._store_tensor(logits, "bf16", "cuda"),
                         torch.from_numpy(tokens.astype(np.int32)).cuda(), tau, ws, lp0, lq)
    d.presto.root_lp0, d.presto.root_lq = lp0[:T], lq[:T]
    d.presto.lp0, d.presto.lq = lp0[T:], lq[T:]
    tav.tav_presto_accept(d.presto, d.workspace)
    torch.cuda.synchronize()
    assert tav.tav_read_status(ws) == 0 and tav.tav_read_status(d.workspace) == 0
    got = d.presto.log_accept.cpu().numpy().astype(np.float64)
    ok = ~np.isnan(want["logA"])
    np.testing.assert_allclose(got[ok], want["logA"][ok], rtol=1e-3, atol=1e-3)
    path = [int(x) for x in d.presto.pf_path.cpu().numpy()[: int(d.presto.pf_path_len.cpu().numpy()[0])]]
    for k, (node, go, flagged) in enumerate(want["decisions"]):
        if flagged:
            return
        assert path[k] == node
    assert path == want["path"]


GREEDY = {
    "random": ("random", [64, 30, 9], [700, 129, 0], 20008, {}),
    "eagle": ("eagle", [40, 22], [2048, 300], 151936, {"max_depth": 6, "hybrid": "all", "draft_peak": (4.0, 7.0)}),
    "star": ("star", [40, 14], [33, 16], 4096, {}),
}


@pytest.mark.parametrize("seed", [10086, 1, 2])
@pytest.mark.parametrize("case", sorted(GREEDY))
def test_greedy_verification(case, seed):
    tree, n, L, V, extra = GREEDY[case]
    w = gen.tree_batch(seed, B=len(n), prefix_len=L, tree=tree, n_nodes=n, Hq=32, Hkv=8, D=128, dtype="bf16",
                       V=V, temperature=1.0, **extra)
    # every sequence greedy except the last (a mixed batch), and children that carry their
    # parent's argmax, so that paths go deeper than the root
    rng = np.random.default_rng(seed)
    for b in range(w.B):
        s, e = int(w.node_offsets[b]), int(w.node_offsets[b + 1])
        for v in range(e - s):
            kids = [c for c in range(s + 1, e) if int(w.parent[c]) == v]
            if kids and rng.random() < 0.8:
                a = oracle.argmax_token(oracle.verify._logits_f64(w, s + v))
                c = kids[int(rng.integers(0, len(kids)))]
                for k in kids:
                    if k != c and int(w.token[k]) == a:
                        w.token[k] = int(w.token[c])
                w.token[c] = a
    w.temperature = w.temperature.copy()
    w.temperature[:-1] = 0.0
    got = gu.run(w)
    assert got["status"] == 0, got["status"]
    gu.check_verify(w, got)
    gu.check_node_stats(w, got, range(w.N))
    assert max(int(got["path_len"][b]) for b in range(w.B - 1)) > 1


def test_greedy_long_accepted_path():
    """Greedy chains whose every child carries its parent's argmax: the whole chain is accepted, so
    the walk follows 1100 steps (more than it stages in LDS, a path longer than it keeps in LDS) and
    its statuses cover more nodes than each thread holds in registers; a mixed batch with a short
    stochastic chain beside it."""
    w = gen.tree_batch(4, B=2, prefix_len=[10, 40], tree="chain", n_nodes=[1100, 30], Hq=4, Hkv=1, D=64,
                       dtype="bf16", V=256, temperature=1.0)
    s, e = int(w.node_offsets[0]), int(w.node_offsets[1])
    for c in range(s + 1, e):
        w.token[c] = oracle.argmax_token(oracle.verify._logits_f64(w, int(w.parent[c]) + s))
    w.sampled = w.sampled.copy()
    w.sampled[s:e] = 0
    w.temperature = w.temperature.copy()
    w.temperature[0] = 0.0
    got = gu.run(w, max_path=1200)
    assert got["status"] == 0, got["status"]
    assert int(got["path_len"][0]) == 1100
    gu.check_verify(w, got)
