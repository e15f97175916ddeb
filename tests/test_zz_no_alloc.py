"""The allocation-free whole pass (tav_tree_attn_verify_noalloc) against tav_tree_attn_verify.

Both calls run the same kernels on the same inputs, one on a caller workspace and one on
the library's own device array, so every output must be bit-identical.  Two calls in a
row, the second with a smaller problem (the array keeps the first call's contents, which
the second must not read), and once more with the first problem.
"""

import numpy as np
import pytest
import torch

from workloads import device as wdev
from workloads import gen

pytestmark = pytest.mark.gpu

KEYS = ("out", "lse", "depth", "position", "mask", "is_chain")
VKEYS = ("node_status", "path", "path_len", "bonus_token", "node_stats", "node_term_token")


def _outputs(d):
    got = {k: getattr(d.attn, k, None) if k in ("out", "lse") else getattr(d.tree_out, k) for k in KEYS}
    if d.verify is not None:
        got.update({k: getattr(d.verify, k) for k in VKEYS})
    return {k: v.clone() for k, v in got.items()}


def _reset(d):
    d.attn.out.fill_(7.0)
    d.attn.lse.fill_(7.0)
    for t in (d.tree_out.depth, d.tree_out.position, d.tree_out.mask, d.tree_out.is_chain):
        t.fill_(5)
    if d.verify is not None:
        for k in VKEYS:
            getattr(d.verify, k).fill_(3)


def _compare(w):
    import tree_masked_verification_attn_amd as tav

    d = wdev.upload(w, "cuda")
    tav.tav_tree_attn_verify(d.prob, d.tree, d.attn, d.verify, None, d.tree_out, d.workspace)
    torch.cuda.synchronize()
    assert tav.tav_read_status(d.workspace) == 0
    ref = _outputs(d)
    _reset(d)
    status = torch.full((1,), 77, dtype=torch.int32, device="cuda")
    tav.tav_tree_attn_verify_noalloc(d.prob, d.tree, d.attn, d.verify, None, d.tree_out, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = _outputs(d)
    for k in ref:
        a = ref[k].contiguous().view(-1).view(torch.uint8).cpu()
        b = got[k].contiguous().view(-1).view(torch.uint8).cpu()
        assert torch.equal(a, b), k


def test_noalloc_matches_workspace_call_twice():
    big = gen.tree_batch(31, B=5, prefix_len=[4000, 1200, 77, 2500, 600], tree="random",
                         n_nodes=[64, 40, 9, 64, 30], Hq=32, Hkv=8, D=128, dtype="bf16", V=20008,
                         temperature=0.9)
    small = gen.tree_batch(32, B=2, prefix_len=[300, 45], tree="random", n_nodes=[20, 9], Hq=32,
                           Hkv=8, D=128, dtype="bf16", V=4096, temperature=1.1)
    _compare(big)
    _compare(small)
    _compare(big)


def test_noalloc_f32_and_chain():
    _compare(gen.make("c1", 10086))
    _compare(gen.tree_batch(4, B=2, prefix_len=[5, 130], tree="chain", n_nodes=[40, 100], Hq=8, Hkv=2,
                            D=128, dtype="bf16", V=1024, temperature=1.0))
