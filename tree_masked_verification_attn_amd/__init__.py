"""Python binding of libtav, the tree-masked scoring pass for MI355X (gfx950).

Argument marshalling only: every function here packs torch tensors (device
memory) and host integers into the C structs of ``include/tav.h`` and calls the
library entry point of the same name.  All computation happens in the HIP
kernels; if ``libtav.so`` is missing the import of any entry point raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtav.so")

TAV_F32, TAV_BF16 = 0, 1
STATUS_NAMES = {0: "TAV_OK", 1: "TAV_ERR_NULL_POINTER", 2: "TAV_ERR_BAD_SHAPE", 3: "TAV_ERR_UNSUPPORTED",
                4: "TAV_ERR_WORKSPACE", 5: "TAV_ERR_HIP", 6: "TAV_ERR_INVALID_ARGUMENT"}
DEVICE_BITS = {
    0: "BAD_PARENT", 1: "TREE_TOO_LARGE", 2: "BAD_BLOCK", 3: "BAD_TOKEN", 4: "DUP_SIBLING_TOKEN",
    5: "MULTI_SAMPLED", 6: "NO_DRAFT", 7: "ZERO_DRAFT_MASS", 8: "NONFINITE_LOGITS",
    9: "EMPTY_RESIDUAL", 10: "PATH_OVERFLOW", 11: "TOO_MANY_CHILDREN", 12: "PRESTO_BAD_TREE",
    13: "PLAN_MISMATCH", 14: "BAD_TEMPERATURE", 15: "BAD_DRAFT",
}
ENTRY_POINTS = ("tav_workspace_size", "tav_tree_prep", "tav_tree_attention", "tav_tree_verify",
                "tav_presto_accept", "tav_tree_attn_verify", "tav_read_status", "tav_kernel_timing",
                "tav_kernel_timing_read", "tav_tree_attn_verify_noalloc", "tav_token_scores",
                "tav_prefetch_build", "tav_prefetch_reach", "tav_draft_workspace_size", "tav_draft_expand",
                "tav_draft_prune", "tav_status_string", "tav_last_error")
TAV_DRAFT_HYBRID_NONE, TAV_DRAFT_HYBRID_FIRST, TAV_DRAFT_HYBRID_ALL = 0, 1, 2
TAV_PREFETCH_BFS, TAV_PREFETCH_PREDICTIVE = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20   # TAV_NOALLOC_SCRATCH_BYTES

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_f32 = ctypes.c_float


class tav_problem(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("node_offsets_host", _p), ("node_offsets", _p),
                ("prefix_len_host", _p), ("prefix_len", _p), ("num_q_heads", _i32),
                ("num_kv_heads", _i32), ("head_dim", _i32), ("dtype", _i32), ("sm_scale", _f32),
                ("block_size", _i32), ("num_blocks", _i32), ("max_blocks_per_seq", _i32),
                ("vocab", _i32)]


class tav_tree(ctypes.Structure):
    _fields_ = [("parent", _p), ("token", _p), ("sampled", _p)]


class tav_tree_out(ctypes.Structure):
    _fields_ = [("depth", _p), ("position", _p), ("mask", _p), ("is_chain", _p)]


class tav_attn_io(ctypes.Structure):
    _fields_ = [("q", _p), ("k_node", _p), ("v_node", _p), ("k_cache", _p), ("v_cache", _p),
                ("block_table", _p), ("out", _p), ("lse", _p)]


class tav_verify_io(ctypes.Structure):
    _fields_ = [("logits", _p), ("temperature", _p), ("draft", _p), ("num_draft_rows", _i32),
                ("draft_row", _p), ("draft_idx", _p), ("draft_val", _p), ("draft_k", _i32), ("uniforms", _p), ("node_status", _p), ("path", _p),
                ("max_path", _i32), ("path_len", _p), ("bonus_token", _p), ("node_stats", _p),
                ("node_term_token", _p)]


class tav_presto_io(ctypes.Structure):
    _fields_ = [("T", _i32), ("alpha", _f32), ("root_lp0", _p), ("root_lq", _p),
                ("num_requests", _i32), ("cut", _p), ("suffix_off", _p), ("lp0", _p), ("lq", _p),
                ("num_nodes", _i32), ("pf_parent", _p), ("pf_is_accept", _p), ("pf_request", _p),
                ("u", _p), ("max_transitions", _i32), ("log_accept", _p), ("pf_path", _p),
                ("pf_path_len", _p)]


class tav_score_io(ctypes.Structure):
    _fields_ = [("num_rows", _i32), ("vocab", _i32), ("dtype", _i32), ("logits", _p), ("token", _p),
                ("tau", _f32), ("log_p0", _p), ("log_q", _p), ("entropy", _p), ("argmax", _p)]


class tav_prefetch_params(ctypes.Structure):
    _fields_ = [("T", _i32), ("budget", _i32), ("depth_cap", _i32), ("rule", _i32), ("seed", ctypes.c_uint64),
                ("class_w", _f32 * 6)]


class tav_prefetch_out(ctypes.Structure):
    _fields_ = [("capacity", _i32), ("num_nodes", _i32), ("num_requests", _i32), ("parent", _p),
                ("is_accept", _p), ("request", _p), ("cut", _p), ("heap", _p), ("request_cut", _p),
                ("predicted_transitions", ctypes.c_double)]


class tav_draft_params(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("vocab", _i32), ("depth", _i32), ("expand_k", _i32), ("slots", _i32),
                ("lead_m", _i32), ("hybrid", _i32), ("support", _i32), ("budget", _i32),
                ("temperature", _f32), ("eps", _f32)]


class TavError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libtav.so (raises FileNotFoundError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(f"{LIB_PATH} is missing: build it with "
                                    "tree_masked_verification_attn_amd/build.py")
        lib = ctypes.CDLL(LIB_PATH)
        for name in ENTRY_POINTS:
            getattr(lib, name)
        lib.tav_workspace_size.argtypes = [ctypes.POINTER(tav_problem), ctypes.POINTER(tav_presto_io),
                                           ctypes.POINTER(ctypes.c_size_t)]
        lib.tav_tree_prep.argtypes = [ctypes.POINTER(tav_problem), ctypes.POINTER(tav_tree),
                                      ctypes.POINTER(tav_tree_out), _p, ctypes.c_size_t, _p]
        lib.tav_tree_attention.argtypes = [ctypes.POINTER(tav_problem), ctypes.POINTER(tav_tree),
                                           ctypes.POINTER(tav_attn_io), _p, ctypes.c_size_t, _p]
        lib.tav_tree_verify.argtypes = [ctypes.POINTER(tav_problem), ctypes.POINTER(tav_tree),
                                        ctypes.POINTER(tav_verify_io), _p, ctypes.c_size_t, _p]
        lib.tav_presto_accept.argtypes = [ctypes.POINTER(tav_presto_io), _p, ctypes.c_size_t, _p]
        lib.tav_tree_attn_verify.argtypes = [
            ctypes.POINTER(tav_problem), ctypes.POINTER(tav_tree), ctypes.POINTER(tav_attn_io),
            ctypes.POINTER(tav_verify_io), ctypes.POINTER(tav_presto_io), ctypes.POINTER(tav_tree_out),
            _p, ctypes.c_size_t, _p, _p]
        lib.tav_tree_attn_verify_noalloc.argtypes = [
            ctypes.POINTER(tav_problem), ctypes.POINTER(tav_tree), ctypes.POINTER(tav_attn_io),
            ctypes.POINTER(tav_verify_io), ctypes.POINTER(tav_presto_io), ctypes.POINTER(tav_tree_out),
            _p, _p, _p]
        lib.tav_token_scores.argtypes = [ctypes.POINTER(tav_score_io), _p, ctypes.c_size_t, _p]
        lib.tav_prefetch_build.argtypes = [ctypes.POINTER(tav_prefetch_params), ctypes.POINTER(tav_prefetch_out)]
        lib.tav_prefetch_reach.argtypes = [_i32, _p, _p, _p, _i32, _p, _f32, _p, ctypes.POINTER(ctypes.c_double)]
        lib.tav_draft_workspace_size.argtypes = [ctypes.POINTER(tav_draft_params), ctypes.POINTER(ctypes.c_size_t)]
        lib.tav_draft_expand.argtypes = [ctypes.POINTER(tav_draft_params), _i32, _p, _p, _p, _p, ctypes.c_size_t, _p]
        lib.tav_draft_prune.argtypes = [ctypes.POINTER(tav_draft_params), _p, _p, _p, _p, _p, _p, _p, _p,
                                        ctypes.c_size_t, _p]
        lib.tav_read_status.argtypes = [_p, _p, ctypes.POINTER(ctypes.c_uint32)]
        lib.tav_kernel_timing.argtypes = [ctypes.c_int]
        lib.tav_kernel_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i32)]
        lib.tav_status_string.argtypes = [ctypes.c_int]
        lib.tav_status_string.restype = ctypes.c_char_p
        lib.tav_last_error.restype = ctypes.c_char_p
        for name in ENTRY_POINTS[:16]:
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libtav must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _check(status: int):
    if status != 0:
        raise TavError(status, load().tav_last_error().decode())


def _stream(s) -> Optional[ctypes.c_void_p]:
    if s is None:
        s = torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class Problem:
    """Host description of a batch; node_offsets / prefix_len are int32 CPU tensors,
    and their device copies are made once here."""
    node_offsets: torch.Tensor
    prefix_len: torch.Tensor
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    vocab: int = 0
    sm_scale: float = 0.0
    device: str = "cuda"

    def __post_init__(self):
        self.node_offsets = self.node_offsets.to("cpu", torch.int32).contiguous()
        self.prefix_len = self.prefix_len.to("cpu", torch.int32).contiguous()
        self.node_offsets_dev = self.node_offsets.to(self.device)
        self.prefix_len_dev = self.prefix_len.to(self.device)

    def struct(self) -> tav_problem:
        return tav_problem(
            num_seqs=self.node_offsets.numel() - 1,
            node_offsets_host=_ptr(self.node_offsets), node_offsets=_ptr(self.node_offsets_dev),
            prefix_len_host=_ptr(self.prefix_len), prefix_len=_ptr(self.prefix_len_dev),
            num_q_heads=self.num_q_heads, num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
            dtype=self.dtype, sm_scale=self.sm_scale, block_size=self.block_size,
            num_blocks=self.num_blocks, max_blocks_per_seq=self.max_blocks_per_seq, vocab=self.vocab)


def _struct_of(cls, obj, **scalars):
    """Build a ctypes struct from an object whose attributes are tensors / ints."""
    if obj is None:
        return None
    vals = {}
    for name, typ in cls._fields_:
        if name in scalars:
            vals[name] = scalars[name]
            continue
        v = getattr(obj, name, None)
        vals[name] = _ptr(v) if (typ is _p and isinstance(v, torch.Tensor)) else (v if v is not None else (None if typ is _p else 0))
    return cls(**vals)


def _ref(s):
    return ctypes.byref(s) if s is not None else None


def tav_workspace_size(prob: Problem, presto=None) -> int:
    n = ctypes.c_size_t(0)
    ps = prob.struct()
    pr = _struct_of(tav_presto_io, presto)
    _check(load().tav_workspace_size(ctypes.byref(ps), _ref(pr), ctypes.byref(n)))
    return n.value


def tav_tree_prep(prob: Problem, tree, tree_out, workspace: torch.Tensor, stream=None):
    ps, ts, to = prob.struct(), _struct_of(tav_tree, tree), _struct_of(tav_tree_out, tree_out)
    _check(load().tav_tree_prep(ctypes.byref(ps), ctypes.byref(ts), _ref(to), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))


def tav_tree_attention(prob: Problem, tree, attn, workspace: torch.Tensor, stream=None):
    ps, ts, ai = prob.struct(), _struct_of(tav_tree, tree), _struct_of(tav_attn_io, attn)
    _check(load().tav_tree_attention(ctypes.byref(ps), ctypes.byref(ts), ctypes.byref(ai), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))


def tav_tree_verify(prob: Problem, tree, verify, workspace: torch.Tensor, stream=None):
    ps, ts, vi = prob.struct(), _struct_of(tav_tree, tree), _struct_of(tav_verify_io, verify)
    _check(load().tav_tree_verify(ctypes.byref(ps), ctypes.byref(ts), ctypes.byref(vi), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def tav_presto_accept(presto, workspace: torch.Tensor, stream=None):
    pr = _struct_of(tav_presto_io, presto)
    _check(load().tav_presto_accept(ctypes.byref(pr), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))


def tav_tree_attn_verify(prob: Problem, tree, attn, verify, presto, tree_out, workspace: torch.Tensor,
                         attn_stream=None, verify_stream=None):
    ps = prob.struct()
    ts = _struct_of(tav_tree, tree)
    ai = _struct_of(tav_attn_io, attn)
    vi = _struct_of(tav_verify_io, verify)
    pr = _struct_of(tav_presto_io, presto)
    to = _struct_of(tav_tree_out, tree_out)
    sa = _stream(attn_stream)
    sv = _stream(verify_stream) if verify_stream is not None else sa
    _check(load().tav_tree_attn_verify(ctypes.byref(ps), ctypes.byref(ts), ctypes.byref(ai), _ref(vi),
                                       _ref(pr), _ref(to), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), sa, sv))


def tav_tree_attn_verify_noalloc(prob: Problem, tree, attn, verify, presto, tree_out,
                                 status_out: Optional[torch.Tensor] = None, attn_stream=None,
                                 verify_stream=None):
    """The whole pass on the library's own device array (no workspace argument, no allocation);
    status_out: optional int32/uint32 device tensor of one element that receives the status word."""
    ps = prob.struct()
    ts = _struct_of(tav_tree, tree)
    ai = _struct_of(tav_attn_io, attn)
    vi = _struct_of(tav_verify_io, verify)
    pr = _struct_of(tav_presto_io, presto)
    to = _struct_of(tav_tree_out, tree_out)
    sa = _stream(attn_stream)
    sv = _stream(verify_stream) if verify_stream is not None else sa
    _check(load().tav_tree_attn_verify_noalloc(ctypes.byref(ps), ctypes.byref(ts), ctypes.byref(ai), _ref(vi),
                                               _ref(pr), _ref(to), _ptr(status_out), sa, sv))


def tav_token_scores(logits: torch.Tensor, token: Optional[torch.Tensor], tau: float, workspace: torch.Tensor,
                     log_p0=None, log_q=None, entropy=None, argmax=None, stream=None):
    """Per-token log p0, log q_tau, entropy of p0 and argmax of each row of logits [N, V]
    (bfloat16 or float32); outputs are caller tensors of N elements (None: not written)."""
    if logits.dim() != 2:
        raise ValueError("logits must be [rows, vocab]")
    dt = TAV_BF16 if logits.dtype == torch.bfloat16 else TAV_F32
    io = tav_score_io(num_rows=logits.shape[0], vocab=logits.shape[1], dtype=dt, logits=_ptr(logits),
                      token=_ptr(token), tau=float(tau), log_p0=_ptr(log_p0), log_q=_ptr(log_q),
                      entropy=_ptr(entropy), argmax=_ptr(argmax))
    _check(load().tav_token_scores(ctypes.byref(io), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)))


def tav_prefetch_build(T: int, budget: int, depth_cap: int, rule: int, seed: int, class_w, capacity=None):
    """PreSTO's prefetching tree for one batch (host only).  Returns a dict of numpy arrays:
    parent, is_accept, request, cut, heap (one entry per node, ascending heap index),
    request_cut, and predicted_transitions."""
    import numpy as np

    if capacity is None:   # BFS expansions whose request is deferred add nodes but no request
        capacity = 2 * int(budget) + 1 if rule == TAV_PREFETCH_PREDICTIVE else 64 * int(budget) + 1024
    cap = int(capacity)
    arr = {"parent": np.zeros(cap, np.int32), "is_accept": np.zeros(cap, np.uint8),
           "request": np.zeros(cap, np.int32), "cut": np.zeros(cap, np.int32),
           "heap": np.zeros(cap, np.int64), "request_cut": np.zeros(max(1, int(budget)), np.int32)}
    prm = tav_prefetch_params(T=int(T), budget=int(budget), depth_cap=int(depth_cap), rule=int(rule),
                              seed=int(seed) & ((1 << 64) - 1), class_w=(_f32 * 6)(*[float(x) for x in class_w]))
    out = tav_prefetch_out(capacity=cap, **{k: v.ctypes.data for k, v in arr.items()})
    _check(load().tav_prefetch_build(ctypes.byref(prm), ctypes.byref(out)))
    res = {k: v[: out.num_nodes].copy() for k, v in arr.items() if k != "request_cut"}
    res["request_cut"] = arr["request_cut"][: out.num_requests].copy()
    res["predicted_transitions"] = out.predicted_transitions
    return res


def tav_prefetch_reach(parent, is_accept, request, log_accept, eps: float):
    """Epsilon-rounded reaching weights of a scored prefetching tree (host only): (reach, F)."""
    import numpy as np

    parent = np.ascontiguousarray(parent, np.int32)
    is_accept = np.ascontiguousarray(is_accept, np.uint8)
    request = np.ascontiguousarray(request, np.int32)
    log_accept = np.ascontiguousarray(log_accept, np.float32)
    reach = np.zeros(len(parent), np.float64)
    F = ctypes.c_double(0.0)
    _check(load().tav_prefetch_reach(len(parent), parent.ctypes.data, is_accept.ctypes.data, request.ctypes.data,
                                     len(log_accept), log_accept.ctypes.data if len(log_accept) else None,
                                     float(eps), reach.ctypes.data, ctypes.byref(F)))
    return reach, F.value


def draft_params(**kw) -> tav_draft_params:
    """tav_draft_params from keyword arguments (the C field names)."""
    return tav_draft_params(**kw)


def tav_draft_workspace_size(params: tav_draft_params) -> int:
    n = ctypes.c_size_t(0)
    _check(load().tav_draft_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def tav_draft_expand(params: tav_draft_params, d: int, draft_logits: torch.Tensor, uniforms: torch.Tensor,
                     frontier_out: Optional[torch.Tensor], workspace: torch.Tensor, stream=None):
    """Depth d of the draft-tree construction: draft_logits [B, K_d, V] bf16, uniforms [B, K_d] f32;
    frontier_out [B, expand_k] int32 receives the next parents' candidate ids."""
    _check(load().tav_draft_expand(ctypes.byref(params), int(d), _ptr(draft_logits), _ptr(uniforms),
                                   _ptr(frontier_out), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def tav_draft_prune(params: tav_draft_params, parent, token, sampled, cand_id, draft_row, draft_idx, draft_val,
                    workspace: torch.Tensor, stream=None):
    _check(load().tav_draft_prune(ctypes.byref(params), _ptr(parent), _ptr(token), _ptr(sampled), _ptr(cand_id),
                                  _ptr(draft_row), _ptr(draft_idx), _ptr(draft_val), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def tav_read_status(workspace: torch.Tensor, stream=None) -> int:
    bits = ctypes.c_uint32(0)
    _check(load().tav_read_status(_ptr(workspace), _stream(stream), ctypes.byref(bits)))
    return bits.value


def tav_kernel_timing(which):
    """0 / False: off; 1 / True: the attention kernel; 2: the vocabulary workers' kernel."""
    _check(load().tav_kernel_timing(int(which)))


def tav_kernel_timing_read():
    """(summed milliseconds, launches) of the attention kernel since the previous read."""
    ms, n = ctypes.c_double(0.0), _i32(0)
    _check(load().tav_kernel_timing_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def device_status_names(bits: int):
    return [name for i, name in DEVICE_BITS.items() if bits >> i & 1]


def tav_status_string(status: int) -> str:
    return load().tav_status_string(status).decode()


def tav_last_error() -> str:
    return load().tav_last_error().decode()
