"""Helpers for the GPU parity tests: run libtav on a workload and compare with the oracle."""

import numpy as np
import torch

import oracle
from oracle.verify import node_terminal_stats
from workloads import device as wdev

TIE = 1e-5


def run(w, two_streams=False, max_path=64, with_verify=True, with_presto=True, split_calls=False):
    """Upload w, run the pass once, return numpy outputs and the status bits.

    split_calls=True runs tav_tree_prep, tav_tree_attention and tav_tree_verify /
    tav_presto_accept on two streams with their own workspaces; otherwise one
    tav_tree_attn_verify call (the benchmark's launch configuration)."""
    import tree_masked_verification_attn_amd as tav

    d = wdev.upload(w, "cuda", with_verify=with_verify, with_presto=with_presto, max_path=max_path)
    if split_calls:
        sa, sv = torch.cuda.Stream(), torch.cuda.Stream()
        ws2 = torch.zeros_like(d.workspace)
        tav.tav_tree_prep(d.prob, d.tree, d.tree_out, d.workspace, sa)
        tav.tav_tree_attention(d.prob, d.tree, d.attn, d.workspace, sa)
        if d.verify is not None:
            tav.tav_tree_verify(d.prob, d.tree, d.verify, ws2, sv)
        if d.presto is not None:
            tav.tav_presto_accept(d.presto, ws2, sv)
        torch.cuda.synchronize()
        status = tav.tav_read_status(d.workspace) | tav.tav_read_status(ws2)
    else:
        sv = torch.cuda.Stream() if two_streams else None
        tav.tav_tree_attn_verify(d.prob, d.tree, d.attn, d.verify, d.presto, d.tree_out, d.workspace,
                                 None, sv)
        status = tav.tav_read_status(d.workspace)
    torch.cuda.synchronize()
    out = {"status": status, "dev": d}
    out["out"] = d.attn.out.float().cpu().numpy().astype(np.float64)
    out["lse"] = d.attn.lse.cpu().numpy().astype(np.float64)
    out["depth"] = d.tree_out.depth.cpu().numpy()
    out["position"] = d.tree_out.position.cpu().numpy()
    out["mask"] = d.tree_out.mask.cpu().numpy().view(np.uint64)
    out["is_chain"] = d.tree_out.is_chain.cpu().numpy()
    if d.verify is not None:
        v = d.verify
        out["node_status"] = v.node_status.cpu().numpy()
        out["path"] = v.path.cpu().numpy()
        out["path_len"] = v.path_len.cpu().numpy()
        out["bonus"] = v.bonus_token.cpu().numpy()
        out["stats"] = v.node_stats.cpu().numpy().astype(np.float64)
        out["term"] = v.node_term_token.cpu().numpy()
    if d.presto is not None:
        out["logA"] = d.presto.log_accept.cpu().numpy().astype(np.float64)
        out["pf_path"] = d.presto.pf_path.cpu().numpy()
        out["pf_path_len"] = int(d.presto.pf_path_len.cpu().numpy()[0])
    return out


def check_tree_prep(w, got):
    prep = oracle.tree_prep(w.parent, w.node_offsets, w.prefix_len)
    np.testing.assert_array_equal(got["depth"], prep["depth"])
    np.testing.assert_array_equal(got["position"], prep["pos"])
    np.testing.assert_array_equal(got["is_chain"].astype(bool), prep["is_chain"])
    for b in range(w.B):
        for v in w.seq_nodes(b):
            want = np.zeros(4, np.uint64) if prep["is_chain"][b] else oracle.ancestor_words(prep["anc"][v], 4)
            np.testing.assert_array_equal(got["mask"][v], want, err_msg=f"mask of node {v}")


def check_attention(w, got, nodes=None, tol=None, prep=None):
    if tol is None:
        tol = 2e-2 if w.dtype == "bf16" else 1e-5
    ref_out, ref_lse = oracle.tree_attention(w, nodes, prep)
    idx = list(range(w.N)) if nodes is None else list(nodes)
    o = got["out"][idx]
    l = got["lse"][idx]
    np.testing.assert_allclose(o, ref_out, rtol=tol, atol=tol)
    np.testing.assert_allclose(l, ref_lse, rtol=tol, atol=tol)
    return float(np.abs(o - ref_out).max())


def gpu_decisions(w, b, status, path, plen, bonus):
    """Decision sequence implied by the library's outputs, in the walk's test order."""
    s, e = int(w.node_offsets[b]), int(w.node_offsets[b + 1])
    n = e - s
    kids = [[] for _ in range(n)]
    for c in range(1, n):
        kids[int(w.parent[s + c])].append(c)
    dec = []
    pth = [int(x) for x in path[:plen]]
    for i, v in enumerate(pth):
        order = [c for c in kids[v] if w.sampled[s + c]] + [c for c in kids[v] if not w.sampled[s + c]]
        nxt = pth[i + 1] if i + 1 < len(pth) else None
        for c in order:
            if c == nxt:
                dec.append(("test", c, True))
                break
            dec.append(("test", c, False))
        if nxt is None:
            dec.append(("sample", v, int(bonus)))
    # statuses must be exactly those implied by the decisions
    want = np.zeros(n, np.uint8)
    want[0] = 1
    for kind, node, outcome in dec:
        if kind == "test":
            want[node] = 1 if outcome else 2
    np.testing.assert_array_equal(status[s:e], want, err_msg=f"seq {b}: statuses vs path")
    return dec


def check_verify(w, got, seqs=None):
    """Compare the walk decision by decision with the oracle up to its first near-tie."""
    if seqs is None:
        seqs = range(w.B)
    res = oracle.verify_workload(w, seqs)
    n_flagged = 0
    for b, r in zip(seqs, res):
        dec_g = gpu_decisions(w, b, got["node_status"], got["path"][b], int(got["path_len"][b]),
                              int(got["bonus"][b]))
        dec_o = r["decisions"]
        for k, d in enumerate(dec_o):
            kind, node, outcome, flagged, extra = d
            if k >= len(dec_g):
                raise AssertionError(f"seq {b}: library stopped after {len(dec_g)} decisions, oracle has {len(dec_o)}")
            kg, ng, og = dec_g[k]
            assert (kg, ng) == (kind, node), f"seq {b} decision {k}: {dec_g[k]} vs oracle {d[:3]}"
            if kind == "sample" and extra is None:      # greedy: the argmax, exactly
                assert og == outcome, f"seq {b}: bonus {og} vs oracle {outcome}"
                break
            if kind == "sample":
                lo, hi, _F = extra
                u = float(w.uniforms[int(w.node_offsets[b]) + node][1])
                if og != outcome:
                    # the library's token is fine if u falls in its CDF step up to the tie band
                    Fj = _F[og] if og < len(_F) else 1.0
                    Fj1 = _F[og - 1] if og > 0 else 0.0
                    assert Fj1 - TIE <= u < Fj + TIE, f"seq {b}: bonus {og} vs oracle {outcome}"
                    n_flagged += 1
                break
            if flagged:
                n_flagged += 1
                break
            assert og == outcome, f"seq {b} decision {k} at node {node}: library {og} oracle {outcome}"
        else:
            assert len(dec_g) == len(dec_o), f"seq {b}: {len(dec_g)} decisions vs oracle {len(dec_o)}"
    return n_flagged


def check_node_stats(w, got, nodes):
    """M, S, Z and the would-be final draw of the given nodes against the oracle."""
    for v in nodes:
        b = int(np.searchsorted(w.node_offsets, v, side="right") - 1)
        s = int(w.node_offsets[b])
        kids = [c for c in range(s + 1, int(w.node_offsets[b + 1])) if int(w.parent[c]) == v - s]
        det = [int(w.token[c]) for c in kids if not w.sampled[c]]
        has_s = any(w.sampled[c] for c in kids)
        dr = int(w.draft_row[v])
        qt = oracle.dense_draft_row(w, dr) if (has_s and dr >= 0) else None
        row = oracle.verify._logits_f64(w, v)
        if float(w.temperature[b]) == 0.0:              # greedy: M = max l, S = 1, Z = 0, argmax
            gm, gs, gz = got["stats"][v]
            assert gm == row.max() and gs == 1.0 and gz == 0.0, (v, gm, gs, gz)
            assert int(got["term"][v]) == oracle.argmax_token(row), (v, int(got["term"][v]))
            continue
        M, S, Z, tok, (lo, hi) = node_terminal_stats(row, float(w.temperature[b]), qt, det,
                                                     float(w.uniforms[v][1]))
        gm, gs, gz = got["stats"][v]
        assert abs(gm - M) <= 1e-5 * max(1.0, abs(M)), (v, gm, M)
        assert abs(gs - S) <= 1e-5 * S, (v, gs, S)
        assert abs(gz - Z) <= 1e-5, (v, gz, Z)
        gt = int(got["term"][v])
        if gt != tok:
            # accept a neighbouring token only inside the tie band of the oracle CDF
            r = np.exp(row / float(w.temperature[b]) - row.max() / float(w.temperature[b]))
            p = r / r.sum()
            wts = np.maximum(0.0, p - qt) if qt is not None else p.copy()
            for t in det:
                wts[t] = 0.0
            F = np.cumsum(wts) / wts.sum()
            u = float(w.uniforms[v][1])
            Fj1 = F[gt - 1] if gt > 0 else 0.0
            assert gt >= 0 and Fj1 - TIE <= u < F[gt] + TIE, (v, gt, tok)


def check_presto(w, got):
    ref = oracle.presto_workload(w.presto)
    la = ref["logA"]
    ok = ~np.isnan(la)
    np.testing.assert_allclose(got["logA"][ok], la[ok], rtol=1e-3, atol=1e-3)
    path = [int(x) for x in got["pf_path"][: got["pf_path_len"]]]
    # decisions must match up to the first near-tie of the oracle
    for k, (node, go, flagged) in enumerate(ref["decisions"]):
        if flagged:
            return
        assert path[k] == node, (k, path, ref["path"])
    assert path == ref["path"], (path, ref["path"])
