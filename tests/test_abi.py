"""The C ABI without a GPU: libtav.so loads, exports every entry point that
include/tav.h declares, and its host-side validation returns the documented
status codes before any HIP call is made."""

import ctypes
import os
import re

import numpy as np
import pytest

import tree_masked_verification_attn_amd as tav

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tav.h")).read()
    return sorted(set(re.findall(r"^\s*(?:tav_status|const char\*)\s+(tav_\w+)\s*\(", src, re.M)))


def test_header_declares_the_binding_entry_points():
    assert _declared() == sorted(tav.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    lib = tav.load()
    for name in _declared():
        assert hasattr(lib, name), name
        assert callable(getattr(tav, name)), name


class _Host:
    """A problem whose 'device' arrays are host arrays: fine for host-side validation."""

    def __init__(self, offsets=(0, 5, 9), prefix=(16, 40), Hq=32, Hkv=8, D=128, dtype=tav.TAV_BF16,
                 block_size=16, num_blocks=8, max_blocks=4, vocab=0):
        self.off = np.array(offsets, np.int32)
        self.pre = np.array(prefix, np.int32)
        self.p = tav.tav_problem(
            num_seqs=len(offsets) - 1,
            node_offsets_host=self.off.ctypes.data, node_offsets=self.off.ctypes.data,
            prefix_len_host=self.pre.ctypes.data, prefix_len=self.pre.ctypes.data,
            num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype, sm_scale=0.0,
            block_size=block_size, num_blocks=num_blocks, max_blocks_per_seq=max_blocks, vocab=vocab)


def _ws_size(h, presto=None):
    n = ctypes.c_size_t(0)
    st = tav.load().tav_workspace_size(ctypes.byref(h.p), presto, ctypes.byref(n))
    return st, n.value


def test_workspace_size_ok_and_grows_with_nodes():
    st, a = _ws_size(_Host())
    assert st == 0 and a > 0
    st, b = _ws_size(_Host(offsets=(0, 5, 300)))
    assert st == 0 and b > a


@pytest.mark.parametrize("kw,code", [
    (dict(offsets=(0,)), 2),                     # no sequences
    (dict(offsets=(1, 5, 9)), 2),                # offsets must start at 0
    (dict(offsets=(0, 5, 5)), 2),                # empty sequence
    (dict(Hq=30, Hkv=8), 2),                     # heads not a multiple
    (dict(Hq=24, Hkv=8), 3),                     # group size 3
    (dict(Hq=64, Hkv=2), 3),                     # group size 32
    (dict(D=96), 3),                             # head_dim
    (dict(dtype=7), 3),                          # dtype
    (dict(block_size=12), 3),                    # block size
    (dict(prefix=(16, 65), max_blocks=4), 2),    # prefix longer than the block table row
    (dict(prefix=(-1, 3)), 2),                   # negative prefix
])
def test_problem_validation_codes(kw, code):
    st, _ = _ws_size(_Host(**kw))
    assert st == code, (st, tav.tav_last_error())
    assert tav.tav_last_error() != ""


def test_null_pointers_and_workspace_checks():
    lib = tav.load()
    h = _Host()
    n = ctypes.c_size_t(0)
    assert lib.tav_workspace_size(None, None, ctypes.byref(n)) == 1
    assert lib.tav_workspace_size(ctypes.byref(h.p), None, None) == 1
    st, need = _ws_size(h)
    parent = np.array([-1, 0, 0, 1, 1, -1, 0, 1, 2], np.int32)
    tree = tav.tav_tree(parent=parent.ctypes.data, token=None, sampled=None)
    buf = np.zeros(need + 512, np.uint8)
    base = buf.ctypes.data
    ws = base + (-base) % 256
    attn = tav.tav_attn_io()                      # all NULL
    assert lib.tav_tree_attention(ctypes.byref(h.p), ctypes.byref(tree), ctypes.byref(attn), ws, need, None) == 1
    dummy = np.zeros(64, np.float32)
    d = dummy.ctypes.data + (-dummy.ctypes.data) % 16
    attn = tav.tav_attn_io(q=d, k_node=d, v_node=d, k_cache=d, v_cache=d, block_table=d, out=d, lse=None)
    assert lib.tav_tree_attention(ctypes.byref(h.p), ctypes.byref(tree), ctypes.byref(attn), None, need, None) == 4
    assert lib.tav_tree_attention(ctypes.byref(h.p), ctypes.byref(tree), ctypes.byref(attn), ws, need - 1, None) == 4
    assert lib.tav_tree_attention(ctypes.byref(h.p), ctypes.byref(tree), ctypes.byref(attn), ws + 16, need, None) == 4
    attn_mis = tav.tav_attn_io(q=d + 2, k_node=d, v_node=d, k_cache=d, v_cache=d, block_table=d, out=d)
    assert lib.tav_tree_attention(ctypes.byref(h.p), ctypes.byref(tree), ctypes.byref(attn_mis), ws, need, None) == 6
    notree = tav.tav_tree(parent=None)
    assert lib.tav_tree_attention(ctypes.byref(h.p), ctypes.byref(notree), ctypes.byref(attn), ws, need, None) == 1


def test_verify_validation_codes():
    lib = tav.load()
    dummy = np.zeros(64, np.float32)
    d = dummy.ctypes.data + (-dummy.ctypes.data) % 16
    parent = np.array([-1, 0, 0, 1, 1, -1, 0, 1, 2], np.int32)
    tree = tav.tav_tree(parent=parent.ctypes.data, token=d, sampled=d)

    def status(h, **kw):
        _, need = _ws_size(h)
        buf = np.zeros(need + 512, np.uint8)
        ws = buf.ctypes.data + (-buf.ctypes.data) % 256
        fields = dict(logits=d, temperature=d, draft=d, num_draft_rows=1, draft_row=d, uniforms=d,
                      node_status=d, path=d, max_path=8, path_len=d, bonus_token=d)
        fields.update(kw)
        io = tav.tav_verify_io(**fields)
        return lib.tav_tree_verify(ctypes.byref(h.p), ctypes.byref(tree), ctypes.byref(io), ws, need, None)

    assert status(_Host(vocab=0)) == 2                       # no vocabulary
    assert status(_Host(vocab=1001)) == 3                    # not a multiple of 8 for bf16 logits
    assert status(_Host(vocab=1048584)) == 3                 # beyond 64 slices of 16384 tokens
    assert status(_Host(vocab=1000, dtype=tav.TAV_F32), max_path=0) == 2
    assert status(_Host(vocab=1000), logits=None) == 1
    assert status(_Host(vocab=1000), num_draft_rows=2, draft=None) == 1
    tree_nt = tav.tav_tree(parent=parent.ctypes.data, token=None, sampled=d)
    h = _Host(vocab=1000)
    _, need = _ws_size(h)
    buf = np.zeros(need + 512, np.uint8)
    ws = buf.ctypes.data + (-buf.ctypes.data) % 256
    io = tav.tav_verify_io(logits=d, temperature=d, draft=d, num_draft_rows=1, draft_row=d, uniforms=d,
                           node_status=d, path=d, max_path=8, path_len=d, bonus_token=d)
    assert lib.tav_tree_verify(ctypes.byref(h.p), ctypes.byref(tree_nt), ctypes.byref(io), ws, need, None) == 1


def test_presto_validation_codes():
    lib = tav.load()
    dummy = np.zeros(64, np.float32)
    d = dummy.ctypes.data + (-dummy.ctypes.data) % 16
    buf = np.zeros(4096, np.uint8)
    ws = buf.ctypes.data + (-buf.ctypes.data) % 256
    full = dict(T=8, alpha=4.0, root_lp0=d, root_lq=d, num_requests=2, cut=d, suffix_off=d, lp0=d, lq=d,
                num_nodes=5, pf_parent=d, pf_is_accept=d, pf_request=d, u=d, max_transitions=3,
                log_accept=d, pf_path=d, pf_path_len=d)
    for k, code in [("lq", 1), ("pf_path", 1)]:
        io = tav.tav_presto_io(**{**full, k: None})
        assert lib.tav_presto_accept(ctypes.byref(io), ws, 2048, None) == code
    for k, v in [("T", 0), ("num_requests", 0), ("num_nodes", 0), ("max_transitions", -1)]:
        io = tav.tav_presto_io(**{**full, k: v})
        assert lib.tav_presto_accept(ctypes.byref(io), ws, 2048, None) == 2
    io = tav.tav_presto_io(**{**full, "alpha": float("inf")})
    assert lib.tav_presto_accept(ctypes.byref(io), ws, 2048, None) == 6
    io = tav.tav_presto_io(**full)
    assert lib.tav_presto_accept(ctypes.byref(io), ws, 100, None) == 4


def test_status_strings():
    assert tav.tav_status_string(0) == "TAV_OK"
    assert tav.tav_status_string(4) == "TAV_ERR_WORKSPACE"


def test_kernel_timing_state_without_gpu_work():
    """Enabling, reading an empty record and disabling touch no device."""
    tav.tav_kernel_timing(True)
    assert tav.tav_kernel_timing_read() == (0.0, 0)
    tav.tav_kernel_timing(False)
    assert tav.tav_kernel_timing_read() == (0.0, 0)


def test_noalloc_rejects_problems_beyond_its_array():
    """The allocation-free call checks the problem's workspace against its fixed device array
    before any HIP call: a problem needing more returns TAV_ERR_WORKSPACE and enqueues nothing."""
    lib = tav.load()
    big = _Host(offsets=(0, 200000), prefix=(16,), max_blocks=4)          # a 200000-token chain
    st, need = _ws_size(big)
    assert st == 0 and need > tav.NOALLOC_SCRATCH_BYTES
    parent = np.arange(-1, 199999, dtype=np.int32)
    tree = tav.tav_tree(parent=parent.ctypes.data, token=None, sampled=None)
    dummy = np.zeros(64, np.float32)
    d = dummy.ctypes.data + (-dummy.ctypes.data) % 16
    attn = tav.tav_attn_io(q=d, k_node=d, v_node=d, k_cache=d, v_cache=d, block_table=d, out=d, lse=None)
    st = lib.tav_tree_attn_verify_noalloc(ctypes.byref(big.p), ctypes.byref(tree), ctypes.byref(attn), None,
                                          None, None, None, None, None)
    assert st == 4, tav.tav_last_error()
    assert "allocation-free" in tav.tav_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), 3), (dict(vocab=1001), 3), (dict(vocab=0), 2), (dict(num_rows=-1), 2),
    (dict(tau=0.0), 6), (dict(tau=float("nan")), 6), (dict(logits=None), 1),
])
def test_token_scores_validation_codes(kw, code):
    lib = tav.load()
    buf = np.zeros(4096, np.uint8)
    d = buf.ctypes.data + (-buf.ctypes.data) % 256
    args = dict(num_rows=4, vocab=1024, dtype=tav.TAV_BF16, logits=d, token=None, tau=0.25, log_p0=None,
                log_q=None, entropy=None, argmax=None)
    args.update(kw)
    io = tav.tav_score_io(**args)
    st = lib.tav_token_scores(ctypes.byref(io), d, 256, None)
    assert st == code, (st, tav.tav_last_error())
    io = tav.tav_score_io(**dict(args, **{"logits": d}))
    if code != 1:
        assert lib.tav_token_scores(ctypes.byref(io), d, 100, None) in (code, 4)
