"""Upload a generated workload to the GPU as torch tensors laid out for libtav,
with output buffers and a workspace.  Plumbing only: no arithmetic of the method.
"""

from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import torch


def _t(x, dtype, device):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).to(device)


def _store_tensor(arr, dtype: str, device):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def upload(w, device="cuda", with_verify=True, with_presto=True, max_path=None):
    import tree_masked_verification_attn_amd as tav

    tdtype = tav.TAV_BF16 if w.dtype == "bf16" else tav.TAV_F32
    out_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    N, B = w.N, w.B
    ns = SimpleNamespace()
    if B > 0:
        ns.prob = tav.Problem(
            node_offsets=torch.from_numpy(w.node_offsets.astype(np.int32)),
            prefix_len=torch.from_numpy(w.prefix_len.astype(np.int32)),
            num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D, dtype=tdtype,
            block_size=w.block_size, num_blocks=int(w.k_cache.shape[0]),
            max_blocks_per_seq=int(w.block_table.shape[1]),
            vocab=int(w.V) if (with_verify and w.logits is not None) else 0,
            sm_scale=float(w.sm_scale), device=device)
        ns.tree = SimpleNamespace(
            parent=_t(w.parent, torch.int32, device),
            token=_t(w.token, torch.int32, device) if w.token is not None else torch.zeros(N, dtype=torch.int32, device=device),
            sampled=_t(w.sampled, torch.uint8, device) if w.sampled is not None else torch.zeros(N, dtype=torch.uint8, device=device))
        ns.attn = SimpleNamespace(
            q=_store_tensor(w.q, w.dtype, device), k_node=_store_tensor(w.k_node, w.dtype, device),
            v_node=_store_tensor(w.v_node, w.dtype, device), k_cache=_store_tensor(w.k_cache, w.dtype, device),
            v_cache=_store_tensor(w.v_cache, w.dtype, device), block_table=_t(w.block_table, torch.int32, device),
            out=torch.zeros((N, w.Hq, w.D), dtype=out_dtype, device=device),
            lse=torch.zeros((N, w.Hq), dtype=torch.float32, device=device))
        ns.tree_out = SimpleNamespace(
            depth=torch.full((N,), -7, dtype=torch.int32, device=device),
            position=torch.full((N,), -7, dtype=torch.int32, device=device),
            mask=torch.zeros((N, 4), dtype=torch.int64, device=device),
            is_chain=torch.zeros((B,), dtype=torch.uint8, device=device))
    ns.verify = None
    if with_verify and w.logits is not None:
        mp = max_path or 64
        R = int(w.draft.shape[0]) if w.draft is not None else 0
        K = int(getattr(w, "draft_k", 0) or 0)
        sparse = K > 0
        R = int(w.draft_idx.shape[0]) if sparse else R
        ns.verify = SimpleNamespace(
            logits=_store_tensor(w.logits, w.dtype, device),
            temperature=_t(w.temperature, torch.float32, device),
            draft=None if sparse else _t(w.draft if R else np.zeros((1, w.V), np.float32), torch.float32, device),
            draft_idx=_t(w.draft_idx if R else np.zeros((1, K), np.int32), torch.int32, device) if sparse else None,
            draft_val=_t(w.draft_val if R else np.zeros((1, K), np.float32), torch.float32, device) if sparse else None,
            draft_k=K,
            num_draft_rows=R, draft_row=_t(w.draft_row, torch.int32, device),
            uniforms=_t(w.uniforms, torch.float32, device),
            node_status=torch.full((N,), 9, dtype=torch.uint8, device=device),
            path=torch.full((B, mp), -9, dtype=torch.int32, device=device), max_path=mp,
            path_len=torch.full((B,), -9, dtype=torch.int32, device=device),
            bonus_token=torch.full((B,), -9, dtype=torch.int32, device=device),
            node_stats=torch.zeros((N, 3), dtype=torch.float32, device=device),
            node_term_token=torch.full((N,), -9, dtype=torch.int32, device=device))
    ns.presto = None
    if with_presto and w.presto is not None:
        pr = w.presto
        M = len(pr.pf_parent)
        ns.presto = SimpleNamespace(
            T=int(pr.T), alpha=float(pr.alpha),
            root_lp0=_t(pr.root_lp0, torch.float32, device), root_lq=_t(pr.root_lq, torch.float32, device),
            num_requests=int(len(pr.cut)), cut=_t(pr.cut, torch.int32, device),
            suffix_off=_t(pr.suffix_off, torch.int32, device),
            lp0=_t(pr.lp0, torch.float32, device), lq=_t(pr.lq, torch.float32, device),
            num_nodes=M, pf_parent=_t(pr.pf_parent, torch.int32, device),
            pf_is_accept=_t(pr.pf_is_accept, torch.uint8, device),
            pf_request=_t(pr.pf_request, torch.int32, device), u=_t(pr.u, torch.float32, device),
            max_transitions=int(pr.max_transitions),
            log_accept=torch.full((len(pr.cut),), float("nan"), dtype=torch.float32, device=device),
            pf_path=torch.full((M,), -9, dtype=torch.int32, device=device),
            pf_path_len=torch.full((1,), -9, dtype=torch.int32, device=device))
    if B > 0:
        nbytes = tav.tav_workspace_size(ns.prob, ns.presto)
    else:
        nbytes = 256 + ((8 * len(w.presto.cut) + 255) // 256) * 256
    ns.workspace = torch.zeros(((nbytes + 255) // 256) * 256 // 8 + 32, dtype=torch.float64, device=device)
    ns.ws_bytes = nbytes
    return ns
