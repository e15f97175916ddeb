"""GPU parity of libtav against the oracle on seeded inputs (small and mid-size cases).

Tolerances: attention out / lse within 2e-2 abs+rel in bf16 and 1e-5 in fp32;
tree prep, accept flags, paths and tokens bit-exact except at decisions the
oracle flags as near-ties (|u - threshold| < 1e-5, or u within 1e-5 of a CDF
step); PreSTO log A within 1e-3.
"""

import sys

import numpy as np
import pytest

from workloads import gen
import gpu_util as gu

pytestmark = pytest.mark.gpu

SEEDS = [10086, 1, 2]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("seed", SEEDS)
def test_c1_tiny_fp32(seed):
    _say("c1", seed)
    w = gen.make("c1", seed)
    got = gu.run(w)
    assert got["status"] == 0, got["status"]
    gu.check_tree_prep(w, got)
    gu.check_attention(w, got)
    gu.check_verify(w, got)
    gu.check_node_stats(w, got, range(w.N))


CASES = {
    # name: (tree, n_nodes, prefix_len, Hq, Hkv, D, V, T, extra)
    "random_ragged": ("random", [1, 3, 64, 65, 200], [0, 1, 63, 700, 129], 32, 8, 128, 4096, 1.0, {}),
    "binary_g8_d64": ("binary", [15, 31, 7], [16, 200, 3], 16, 2, 64, 2048, 0.7, {}),
    "random_g1": ("random", [40, 10], [77, 1000], 4, 4, 128, 1024, 1.3, {}),
    "eagle_hybrid": ("eagle", [30, 22], [2048, 300], 32, 8, 128, 8192, 0.7, {"max_depth": 5, "hybrid": "all"}),
    "random_g16": ("random", [16, 17], [64, 65], 16, 1, 128, 512, 1.0, {}),
    # 39 / 13 / 12 children of one node (beyond and at the children kept per node record);
    # V = 20008 spans two vocabulary slices, the second one ragged
    "star_two_slices": ("star", [40, 14, 13], [33, 0, 16], 8, 2, 64, 20008, 0.9, {}),
}


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("case", sorted(CASES))
def test_small_bf16_trees(case, seed):
    tree, n, L, Hq, Hkv, D, V, T, extra = CASES[case]
    _say("tree case", case, seed)
    w = gen.tree_batch(seed, B=len(n), prefix_len=L, tree=tree, n_nodes=n, Hq=Hq, Hkv=Hkv, D=D,
                       dtype="bf16", V=V, temperature=T, **extra)
    got = gu.run(w, two_streams=(seed == 1))
    assert got["status"] == 0, got["status"]
    gu.check_tree_prep(w, got)
    gu.check_attention(w, got)
    gu.check_verify(w, got)
    gu.check_node_stats(w, got, range(w.N))


@pytest.mark.parametrize("seed", SEEDS)
def test_chains_bf16(seed):
    _say("chains", seed)
    w = gen.tree_batch(seed, B=3, prefix_len=[5, 0, 130], tree="chain", n_nodes=[1, 100, 300],
                       Hq=32, Hkv=8, D=128, dtype="bf16", V=1024, temperature=1.0)
    got = gu.run(w, max_path=512)
    assert got["status"] == 0, got["status"]
    gu.check_tree_prep(w, got)
    gu.check_attention(w, got)
    gu.check_verify(w, got)


@pytest.mark.parametrize("seed", SEEDS)
def test_f32_multi_slice(seed):
    """fp32 logits over three vocabulary slices (8192 tokens each), the last one ragged."""
    _say("f32 multi-slice", seed)
    w = gen.tree_batch(seed, B=2, prefix_len=[50, 3], tree="random", n_nodes=[20, 9], Hq=4, Hkv=1,
                       D=64, dtype="f32", V=20004, temperature=1.1)
    got = gu.run(w)
    assert got["status"] == 0, got["status"]
    gu.check_attention(w, got)
    gu.check_verify(w, got)
    gu.check_node_stats(w, got, range(w.N))


@pytest.mark.parametrize("seed", SEEDS[:1])
def test_long_chain_walk(seed):
    """A 1100-node chain: the walk reads its per-node values from memory, not LDS."""
    _say("long chain", seed)
    w = gen.tree_batch(seed, B=2, prefix_len=[10, 40], tree="chain", n_nodes=[1100, 30], Hq=4, Hkv=1,
                       D=64, dtype="bf16", V=256, temperature=1.0)
    got = gu.run(w, max_path=1200)
    assert got["status"] == 0, got["status"]
    gu.check_attention(w, got)
    gu.check_verify(w, got)


@pytest.mark.parametrize("seed", SEEDS)
def test_split_kv_long_prefix(seed):
    _say("split", seed)
    w = gen.tree_batch(seed, B=2, prefix_len=[20000, 3000], tree="random", n_nodes=[48, 9],
                       Hq=8, Hkv=2, D=128, dtype="bf16")
    got = gu.run(w, with_verify=False)
    assert got["status"] == 0, got["status"]
    gu.check_attention(w, got)


@pytest.mark.parametrize("seed", SEEDS)
def test_sharp_softmax(seed):
    """Queries scaled by 24 (score std about 35 in log2 units): a row's running maximum keeps
    rising by more than the kernel's slack from tile to tile inside one segment, so the rescale
    path runs mid-segment, not only at a segment's first tile."""
    _say("sharp softmax", seed)
    w = gen.tree_batch(seed, B=2, prefix_len=[5000, 700], tree="random", n_nodes=[40, 12],
                       Hq=8, Hkv=2, D=128, dtype="bf16")
    w.q = gen.f32_to_bf16_bits(gen.bf16_bits_to_f32(w.q) * 24.0)
    got = gu.run(w, with_verify=False)
    assert got["status"] == 0, got["status"]
    gu.check_attention(w, got)


@pytest.mark.parametrize("seed", SEEDS)
def test_presto_small(seed):
    _say("presto", seed)
    w = gen.presto_batch(seed, T=96, n_pf=12, Hq=8, Hkv=2, D=128, dtype="bf16", alpha=4.0,
                         max_transitions=6)
    got = gu.run(w)
    assert got["status"] == 0, got["status"]
    gu.check_attention(w, got)
    gu.check_presto(w, got)


@pytest.mark.gpu
def test_attention_kernel_timing_events():
    """The timing hook records one event pair per bf16 attention call, around the kernel."""
    import tree_masked_verification_attn_amd as tav
    from workloads import device as wdev

    w = gen.tree_batch(5, B=2, prefix_len=[300, 70], tree="random", n_nodes=[20, 9], Hq=8, Hkv=2,
                       D=128, dtype="bf16")
    d = wdev.upload(w, "cuda", with_verify=False)
    tav.tav_kernel_timing(True)
    for _ in range(3):
        tav.tav_tree_attention(d.prob, d.tree, d.attn, d.workspace)
    ms, n = tav.tav_kernel_timing_read()
    tav.tav_kernel_timing(False)
    assert n == 3 and ms > 0.0


BLOCK_CASES = {
    # name: (block_size, dtype, D, Hkv): caches of 32 and 64 rows per block in bf16 (the packed node
    # blocks then take two heads, or one, per LDS round) and of 8 rows in fp32
    "bf16_bs32_d128": (32, "bf16", 128, 8),
    "bf16_bs64_d64": (64, "bf16", 64, 3),
    "bf16_bs64_d128": (64, "bf16", 128, 2),
    "f32_bs8_d64": (8, "f32", 64, 2),
}


@pytest.mark.parametrize("case", sorted(BLOCK_CASES))
def test_block_sizes(case):
    """Prefix copies, packed node blocks and their tiles at block sizes other than 16, with ragged
    prefixes and trees (a tree of one node, trees ending inside and on a block boundary)."""
    bs, dtype, D, Hkv = BLOCK_CASES[case]
    _say("block size case", case)
    w = gen.tree_batch(11, B=4, prefix_len=[0, 100, 777, 64], tree="random", n_nodes=[70, 1, 130, 64],
                       Hq=4 * Hkv, Hkv=Hkv, D=D, dtype=dtype, V=2048, temperature=1.0, block_size=bs)
    got = gu.run(w)
    assert got["status"] == 0, got["status"]
    gu.check_tree_prep(w, got)
    gu.check_attention(w, got)
    gu.check_verify(w, got)
    gu.check_node_stats(w, got, range(w.N))


@pytest.mark.parametrize("bs,n", [(32, [12000, 13000]), (64, [9000, 8000])])
def test_long_chains_packed_heads(bs, n):
    """Long chains at 32 and 64 rows per block: with thousands of (node block, KV head) pairs each
    packing block takes several heads (4 and 2 here), in two LDS rounds; sampled rows at the
    sequences' ends, block edges and middles."""
    _say("long chains, block size", bs)
    w = gen.tree_batch(4, B=2, prefix_len=[100, 37], tree="chain", n_nodes=n, Hq=32, Hkv=8, D=128,
                       dtype="bf16", V=256, temperature=1.0, block_size=bs)
    got = gu.run(w, max_path=max(n) + 1)
    assert got["status"] == 0, got["status"]
    picks = []
    for b in range(2):
        s, e = int(w.node_offsets[b]), int(w.node_offsets[b + 1])
        picks += [s, s + bs - 1, s + bs, (s + e) // 2, e - bs - 1, e - 1]
    # a chain's visibility sets by their definition (node i of a chain sees nodes 0..i), so that
    # the oracle does not list the sets of every node of the long chains
    anc = [None] * w.N
    for b in range(2):
        s = int(w.node_offsets[b])
        for v in picks[6 * b:6 * b + 6]:
            anc[v] = list(range(v - s + 1))
    gu.check_attention(w, got, sorted(set(picks)), prep={"anc": anc})
    gu.check_verify(w, got)


@pytest.mark.parametrize("B", [300, 2100])
def test_many_sequences(B):
    """More sequences than one block-wide scan of the preparation covers (300), and more than the
    work plan stages in LDS (2100): row-block offsets, node packing, chain flags and the walk of
    every sequence."""
    _say("many sequences", B)
    rng = np.random.default_rng(B)
    n = rng.integers(1, 20, size=B)
    L = rng.integers(0, 40, size=B)
    w = gen.tree_batch(3, B=B, prefix_len=L, tree="random", n_nodes=n, Hq=8, Hkv=2, D=64,
                       dtype="bf16", V=512, temperature=1.0)
    got = gu.run(w)
    assert got["status"] == 0, got["status"]
    gu.check_tree_prep(w, got)
    gu.check_attention(w, got, list(range(0, w.N, 7)) + [w.N - 1])
    gu.check_verify(w, got)
    gu.check_node_stats(w, got, range(0, w.N, 97))


SPARSE_CASES = {
    # name: (tree, n_nodes, prefix_len, V, T, K, extra)
    "random_k128": ("random", [64, 30, 9], [700, 129, 0], 20008, 1.0, 128, {}),
    "eagle_k128": ("eagle", [40, 22], [2048, 300], 8192, 0.7, 128,
                   {"max_depth": 6, "hybrid": "all", "draft_peak": (4.0, 7.0)}),
    "star_k24": ("star", [40, 14], [33, 16], 4096, 0.9, 24, {}),
    "random_k7_f32": ("random", [20, 9], [50, 3], 20004, 1.1, 7, {}),
}


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("case", sorted(SPARSE_CASES))
def test_sparse_draft_rows(case, seed):
    """Sparse top-K draft rows (RheoSampling Section 3.2): no second pass over the row; the walk
    and every node's M, S, Z and would-be final draw match the oracle on the scattered rows."""
    tree, n, L, V, T, K, extra = SPARSE_CASES[case]
    _say("sparse draft", case, seed)
    dtype = "f32" if case.endswith("f32") else "bf16"
    Hq, Hkv, D = (4, 1, 64) if dtype == "f32" else (32, 8, 128)
    w = gen.tree_batch(seed, B=len(n), prefix_len=L, tree=tree, n_nodes=n, Hq=Hq, Hkv=Hkv, D=D,
                       dtype=dtype, V=V, temperature=T, draft_support=K, **extra)
    assert w.draft_k == K and w.draft is None
    got = gu.run(w)
    assert got["status"] == 0, got["status"]
    gu.check_attention(w, got, [v for b in range(w.B) for v in list(w.seq_nodes(b))[:3]])
    gu.check_verify(w, got)
    gu.check_node_stats(w, got, range(w.N))


def test_sparse_draft_row_not_ascending():
    import tree_masked_verification_attn_amd as tav

    w = gen.tree_batch(4, B=3, prefix_len=[30, 40, 50], tree="random", n_nodes=[12, 15, 9], Hq=8, Hkv=2,
                       D=128, dtype="bf16", V=4096, temperature=1.0, draft_support=32)
    s = int(w.node_offsets[1])
    r = int(w.draft_row[s])
    w.draft_idx[r, 5], w.draft_idx[r, 6] = w.draft_idx[r, 6], w.draft_idx[r, 5]
    got = gu.run(w)
    assert got["status"] & (1 << 15), tav.device_status_names(got["status"])
    assert int(got["path_len"][1]) == 0 and int(got["bonus"][1]) == -1
    gu.check_verify(w, got, [0, 2])


@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("seed", SEEDS)
def test_presto_batch_from_prefetch_builder(rule, seed):
    """A prefetch batch whose tree comes from tav_prefetch_build (BFS or predictive rule): its
    arrays feed tav_presto_io directly; log A and the walk match the oracle."""
    import tree_masked_verification_attn_amd as tav

    T = 512
    t = tav.tav_prefetch_build(T, 24, 40, rule, seed, [1.0, -3.0, -1.0, 2.5, 0.0, 0.0])
    rng = np.random.default_rng(seed)
    cuts = t["request_cut"].astype(np.int32)
    off = np.zeros(len(cuts) + 1, np.int32)
    off[1:] = np.cumsum(T - cuts)
    pr = gen.PrestoInputs(
        T=T, alpha=4.0, root_lp0=(-rng.exponential(size=T)).astype(np.float32),
        root_lq=(-rng.exponential(size=T)).astype(np.float32), cut=cuts, suffix_off=off,
        lp0=(-rng.exponential(size=int(off[-1]))).astype(np.float32),
        lq=(-rng.exponential(size=int(off[-1]))).astype(np.float32),
        pf_parent=t["parent"], pf_is_accept=t["is_accept"], pf_request=t["request"], pf_cut=t["cut"],
        u=rng.random(len(t["parent"]), dtype=np.float32), max_transitions=30)
    w = gen.presto_batch(seed, T=8, n_pf=1, Hq=8, Hkv=2, D=128, with_attention=False)
    w.presto = pr
    from workloads import device as wdev

    d = wdev.upload(w, "cuda")
    tav.tav_presto_accept(d.presto, d.workspace)
    status = tav.tav_read_status(d.workspace)
    assert status == 0, status
    got = {"logA": d.presto.log_accept.cpu().numpy().astype(np.float64),
           "pf_path": d.presto.pf_path.cpu().numpy(),
           "pf_path_len": int(d.presto.pf_path_len.cpu().numpy()[0])}
    gu.check_presto(w, got)
