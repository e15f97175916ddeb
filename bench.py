"""Throughput of the tree-masked scoring pass on one MI355X.

Headline workload (default): 16 sequences, prefix lengths uniform in [1024, 8192] in
a paged KV cache (block 16, shuffled block table), 64-node random trees of depth <= 8,
32 query / 8 KV heads, head_dim 128, bf16, vocabulary 151936, T = 1.0, seed 10086 --
the batched verification shape.  Inputs are synthetic (seeded).

One step = one whole pass, one tav_tree_attn_verify call: the call's start with tree
preparation (the attention work plan, node packing and the verification workers' node
order), split-KV tree attention, the verification's vocabulary workers and pick, then the
walk with the merge of the attention row blocks cut between workgroups, all on one stream.  Inputs are resident in HBM; two
input copies alternate so consecutive steps do not re-read one step's data from the
256 MB last-level cache.  The K timed steps carry no events.

Prints one JSON line:  value = tree nodes scored per second (attention +
verification) on the headline workload, plus
  * the step's algorithmic HBM GB/s;
  * roofline: the dominant kernel (the verification's vocabulary workers), timed per
    launch by HIP events the library records around it on its own stream, with the HBM
    traffic measured by counters for the same kernel source (or null);
  * attention_kernel: the attention kernel's roofline from attention-only calls;
  * achievable: a streaming-read kernel's HBM bandwidth and a matrix-core kernel's bf16
    rate on this GPU (the fractions of those beside the fractions of the published peaks);
  * sub_records: the same measurements for the long-context workload (4 x 32768 prefix,
    128-node depth-10 trees), the PreSTO prefetch batch (attention MFMA utilisation,
    log A + walk time), the per-token scorer over that batch's scored tokens, the headline
    workload with sparse top-128 draft rows and at temperature 0 (greedy verification), the
    host prefetch-tree builder and the GPU draft-tree construction;
  * cpu_baseline: the oracle on a bounded sample of the headline workload, on the host.
"""

import argparse
import copy
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
# Counter data of the vocabulary workers' kernel (FETCH_SIZE / WRITE_SIZE per dispatch, scaled by a
# plain copy of known size), valid while the kernel sources are the ones it was taken from.
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_vocab_worker_batched_verify.json")
KERNEL_SOURCES = [os.path.join(ROOT, "tree_masked_verification_attn_amd", "csrc", f)
                  for f in ("vocab_worker.h", "k_verify.hip")]


def _used_draft_rows(w):
    """Nodes whose draft row verification reads: a sampled child and a draft row, in a sequence
    verified at a temperature above 0 (greedy verification reads no draft row)."""
    import numpy as np

    has_s = np.zeros(w.N, bool)
    for b in range(w.B):
        if w.temperature is not None and float(w.temperature[b]) == 0.0:
            continue
        s = int(w.node_offsets[b])
        for c in range(s + 1, int(w.node_offsets[b + 1])):
            if w.sampled[c]:
                has_s[s + int(w.parent[c])] = True
    return int(np.sum(has_s & (w.draft_row >= 0)))


def algorithmic_bytes(w):
    """Bytes the pass must move: each prefix KV row once per (sequence, KV head), each node's
    q / k / v / out once, each logits row once, each draft row that verification uses once
    (V floats dense, K ids + K floats sparse), small per-node arrays."""
    eb = 2 if w.dtype == "bf16" else 4
    kv = int(sum(int(L) for L in w.prefix_len)) * w.Hkv * w.D * eb * 2
    nodes = w.N * (w.Hq * w.D * eb * 2 + w.Hkv * w.D * eb * 2 + w.Hq * 4)
    attn = kv + nodes + int(w.block_table.size) * 4
    verify = 0
    if w.logits is not None:
        row = w.draft_k * 8 if w.draft_k else w.V * 4
        verify = w.N * w.V * eb + _used_draft_rows(w) * row + w.N * (4 + 1 + 4 + 1 + 8)
    return attn, verify


def depths(w):
    """Depth of every node (parents are earlier nodes of the same sequence)."""
    import numpy as np

    d = np.zeros(w.N, np.int64)
    for b in range(w.B):
        s = int(w.node_offsets[b])
        for v in range(s + 1, int(w.node_offsets[b + 1])):
            d[v] = d[s + int(w.parent[v])] + 1
    return d


def attention_flops(w):
    """4 d flops per (query row, visible key): QK^T and PV over prefix + ancestors + self."""
    import numpy as np

    seq = np.repeat(np.arange(w.B), np.diff(w.node_offsets))
    keys = int(np.sum(np.asarray(w.prefix_len, np.int64)[seq] + depths(w) + 1))
    return 4 * w.D * w.Hq * keys


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, threads, min_seconds=8.0, max_passes=4):
    """The oracle, as it is, on the headline workload (attention of every node + verification
    walk of every sequence), with `threads` BLAS threads, repeated to about min_seconds."""
    from threadpoolctl import threadpool_limits

    import oracle

    seqs = list(range(w.B))
    nodes = [v for b in seqs for v in w.seq_nodes(b)]
    passes, dt = 0, 0.0
    with threadpool_limits(threads):
        while passes < max_passes and (passes == 0 or dt < min_seconds):
            t0 = time.perf_counter()
            oracle.tree_attention(w, nodes)
            oracle.verify_workload(w, seqs)
            dt += time.perf_counter() - t0
            passes += 1
    return {"value": round(passes * len(nodes) / dt, 1), "unit": "nodes/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"the whole workload ({w.B} sequences, {len(nodes)} nodes: attention of every "
                      f"node + verification walk) x {passes} passes, {dt:.1f} s"}


def kernel_source_sha256():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the vocabulary workers' kernel from the committed counter data, or
    None when the counters were taken on another workload or the kernel sources have changed
    since."""
    if not os.path.exists(PMC_FILE):
        return None
    rec = json.load(open(PMC_FILE))
    if rec.get("workload") != workload or rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return int(rec["hbm_bytes_per_launch"])


# ----------------------------------------------------------------------------------------------
# GPU measurements
# ----------------------------------------------------------------------------------------------

def achievable(tav_dir):
    """Streaming-read bandwidth (4 GiB read once, median of 5) and bf16 MFMA rate (256 x 4 waves,
    median of 5) measured by the probe library on this GPU."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(tav_dir, "libtavprobe.so"))
    lib.tavprobe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_void_p]
    lib.tavprobe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    s = torch.cuda.Stream()
    nbytes = 4 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    grid = 256 * 16
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
    times = []
    for i in range(7):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        assert lib.tavprobe_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), grid, s.cuda_stream) == 0
        e1.record(s)
        torch.cuda.synchronize()
        if i >= 2:
            times.append(e0.elapsed_time(e1))
    del src
    read_gbs = nbytes / (sorted(times)[len(times) // 2] * 1e-3) / 1e9
    mgrid, iters = 1024, 20000
    msink = torch.zeros(mgrid * 256, dtype=torch.float32, device="cuda")
    times = []
    for i in range(7):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        assert lib.tavprobe_mfma(msink.data_ptr(), iters, mgrid, s.cuda_stream) == 0
        e1.record(s)
        torch.cuda.synchronize()
        if i >= 2:
            times.append(e0.elapsed_time(e1))
    flops = mgrid * 4 * 4 * iters * 32768.0        # waves x chains x rounds x flops per MFMA
    mfma_tflops = flops / (sorted(times)[len(times) // 2] * 1e-3) / 1e12
    return {"hbm_read_gbs": round(read_gbs, 1), "hbm_read_frac_of_peak": round(read_gbs / HBM_PEAK_GBS, 4),
            "mfma_bf16_tflops": round(mfma_tflops, 1),
            "mfma_frac_of_peak": round(mfma_tflops / BF16_PEAK_TFLOPS, 4),
            "how": "stream_read_kernel: 4 GiB read once with 16-byte loads, 8 in flight per thread; "
                   "mfma_kernel: 4 independent v_mfma_f32_32x32x16_bf16 chains per wave, 1024 x 4 waves; "
                   "medians of 5 timed launches"}


class Pass:
    """A workload uploaded twice, timed as whole passes and per kernel."""

    def __init__(self, w, copies=2):
        import torch

        from workloads import device as wdev

        self.w = w
        self.copies = [wdev.upload(w, "cuda") for _ in range(max(1, copies))]
        self.sa = torch.cuda.Stream()
        torch.cuda.synchronize()

    def step(self, i, presto=False):
        import tree_masked_verification_attn_amd as tav

        c = self.copies[i % len(self.copies)]
        tav.tav_tree_attn_verify(c.prob, c.tree, c.attn, c.verify, c.presto if presto else None, None,
                                 c.workspace, self.sa, self.sa)

    def time_steps(self, steps, warmup, presto=False):
        import torch

        import tree_masked_verification_attn_amd as tav

        for i in range(warmup):
            self.step(i, presto)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i, presto)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        for c in self.copies:
            bits = tav.tav_read_status(c.workspace)
            if bits:
                raise RuntimeError(f"device status bits set: {tav.device_status_names(bits)}")
        return ms

    def kernel_ms(self, which, steps, call="pass"):
        """Average launch time of one kernel (1 attention, 2 vocabulary workers) from the library's
        own events over `steps` calls (whole passes, or attention-only calls)."""
        import torch

        import tree_masked_verification_attn_amd as tav

        def run(i):
            if call == "pass":
                self.step(i)
            else:
                c = self.copies[i % len(self.copies)]
                tav.tav_tree_attention(c.prob, c.tree, c.attn, c.workspace, self.sa)

        for i in range(2):
            run(i)
        torch.cuda.synchronize()
        tav.tav_kernel_timing(which)
        for i in range(steps):
            run(i)
        torch.cuda.synchronize()
        total, n = tav.tav_kernel_timing_read()
        tav.tav_kernel_timing(0)
        return total / max(1, n), n

    def presto_ms(self, steps):
        import torch

        import tree_masked_verification_attn_amd as tav

        c = self.copies[0]
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        tav.tav_presto_accept(c.presto, c.workspace, self.sa)
        for e0, e1 in ev:
            e0.record(self.sa)
            tav.tav_presto_accept(c.presto, c.workspace, self.sa)
            e1.record(self.sa)
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in ev) / steps


def roofline_hbm(kernel, bytes_, ms, ach=None, traffic=None, launches=None):
    gbs = bytes_ / (ms * 1e-3) / 1e9
    r = {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "avg_launch_ms": round(ms, 4),
         "launches_timed": launches, "algorithmic_bytes": bytes_}
    if ach:
        r["frac_of_achievable"] = round(gbs / ach["hbm_read_gbs"], 4)
    return r


def attention_record(p, flops, attn_b, steps, ach):
    a_ms, n = p.kernel_ms(1, steps, call="attention")
    rec = roofline_hbm("attn_bf16_kernel (tree-masked attention, bf16 MFMA), attention-only calls",
                       attn_b, a_ms, ach, launches=n)
    tf = flops / (a_ms * 1e-3) / 1e12
    rec.update({"algorithmic_flops": flops, "mfma_tflops": round(tf, 1),
                "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
                "roofline_frac": round(max(attn_b / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
                                       / (a_ms * 1e-3), 4)})
    if ach:
        rec["mfma_frac_of_achievable"] = round(tf / ach["mfma_bf16_tflops"], 4)
    return rec


def tree_sub_record(w, steps, warmup, ach, label):
    p = Pass(w)
    ms = p.time_steps(steps, warmup)
    attn_b, ver_b = algorithmic_bytes(w)
    flops = attention_flops(w)
    k_ms, kn = p.kernel_ms(2, min(steps, 10))
    rec = {"workload": label, "nodes": w.N, "sequences": w.B, "ms_per_pass": round(ms, 4),
           "nodes_per_s": round(w.N / (ms * 1e-3), 1), "algorithmic_bytes": attn_b + ver_b,
           "algorithmic_flops": flops, "pass_gbs": round((attn_b + ver_b) / (ms * 1e-3) / 1e9, 1),
           "pass_roofline_frac": round(max((attn_b + ver_b) / (HBM_PEAK_GBS * 1e9),
                                           flops / (BF16_PEAK_TFLOPS * 1e12)) / (ms * 1e-3), 4),
           "draft_rows_used": _used_draft_rows(w), "draft_k": int(w.draft_k),
           "vocab_workers": roofline_hbm("vocab_worker_kernel + pick_kernel", ver_b, k_ms, ach, launches=kn),
           "attention_kernel": attention_record(p, flops, attn_b, min(steps, 10), ach)}
    del p
    return rec


def presto_sub_record(w, steps, warmup, ach):
    """The PreSTO batch: the whole pass (tree attention of every suffix token + log A + walk), the
    attention kernel alone, tav_presto_accept alone."""
    p = Pass(w)
    ms = p.time_steps(steps, warmup, presto=True)
    attn_b, _ = algorithmic_bytes(w)
    flops = attention_flops(w)
    rec = {"workload": "c4: " + w.info.get("description", ""), "requests": int(len(w.presto.cut)),
           "query_tokens": w.N, "ms_per_pass": round(ms, 4), "algorithmic_bytes": attn_b,
           "algorithmic_flops": flops,
           "attention_kernel": attention_record(p, flops, attn_b, min(steps, 10), ach),
           "presto_accept_ms": round(p.presto_ms(20), 4),
           "note": "the 32 requests are 32 sequences whose block-table rows name the same prefix blocks"}
    del p
    return rec


def scorer_record(seed, rows, V=151936, tau=0.25, reps=5):
    """tav_token_scores over `rows` bf16 logits rows of V tokens drawn on the device (the PreSTO
    batch's scored tokens: every suffix token and every token of the state), one launch per rep."""
    import numpy as np
    import torch

    import tree_masked_verification_attn_amd as tav
    from workloads import gen

    logits = gen.device_logits(seed, rows, V)
    tok = torch.from_numpy(np.random.default_rng(seed).integers(0, V, rows).astype(np.int32)).cuda()
    outs = [torch.empty(rows, device="cuda") for _ in range(3)]
    am = torch.empty(rows, dtype=torch.int32, device="cuda")
    ws = torch.zeros(64, dtype=torch.float64, device="cuda")
    s = torch.cuda.Stream()
    tav.tav_token_scores(logits, tok, tau, ws, *outs, am, stream=s)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(s)
        tav.tav_token_scores(logits, tok, tau, ws, *outs, am, stream=s)
        e1.record(s)
    torch.cuda.synchronize()
    if tav.tav_read_status(ws, s):
        raise RuntimeError("token scorer status bits set")
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]
    nbytes = rows * V * 2 + rows * (4 + 3 * 4 + 4)
    del logits
    torch.cuda.empty_cache()
    rec = roofline_hbm("score_kernel (log p0, log q_tau, entropy, argmax per row)", nbytes, ms, None,
                       launches=reps)
    rec.update({"rows": rows, "vocab": V, "tau": tau, "tokens_per_s": round(rows / (ms * 1e-3), 1)})
    return rec


def draft_tree_record(seed, reps=10):
    """tav_draft_expand x D + tav_draft_prune at the long-context workload's tree shape (4 trees,
    depth 10, 8 parents x 8 slots, hybrid pools with one lead token, top-128 sparse draft, 127 nodes
    kept, V = 151936): the drafter's logits of each depth resident in HBM (drawn on the device)."""
    import torch

    import tree_masked_verification_attn_amd as tav
    from workloads import gen

    B, V, D, K, slots, S, R = 4, 151936, 10, 8, 8, 128, 127
    prm = tav.draft_params(num_seqs=B, vocab=V, depth=D, expand_k=K, slots=slots, lead_m=1,
                           hybrid=tav.TAV_DRAFT_HYBRID_ALL, support=S, budget=R, temperature=1.0, eps=1e-6)
    ws = torch.zeros((tav.tav_draft_workspace_size(prm) + 7) // 8, dtype=torch.float64, device="cuda")
    lg = gen.device_logits(seed, B * K, V).view(B, K, V)
    lg1 = lg[:, :1].contiguous()
    uni = torch.rand((B, K), generator=torch.Generator(device="cuda").manual_seed(seed), device="cuda")
    uni1 = uni[:, :1].contiguous()
    n = R + 1
    outs = [torch.empty(B * n, dtype=torch.int32, device="cuda") for _ in range(2)]
    smp = torch.empty(B * n, dtype=torch.uint8, device="cuda")
    drow = torch.empty(B * n, dtype=torch.int32, device="cuda")
    didx = torch.empty((B * n, S), dtype=torch.int32, device="cuda")
    dval = torch.empty((B * n, S), dtype=torch.float32, device="cuda")
    front = torch.empty((B, K), dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()

    def build():
        for d in range(1, D + 1):
            tav.tav_draft_expand(prm, d, lg1 if d == 1 else lg, uni1 if d == 1 else uni, front, ws, s)
        tav.tav_draft_prune(prm, outs[0], outs[1], smp, None, drow, didx, dval, ws, s)

    build()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        build()
    e1.record(s)
    torch.cuda.synchronize()
    if tav.tav_read_status(ws, s):
        raise RuntimeError("draft-tree status bits set")
    ms = e0.elapsed_time(e1) / reps
    nbytes = B * V * 2 * (1 + (D - 1) * K)
    rec = roofline_hbm("draft_expand_kernel x depth + frontier + prune (GPU draft-tree construction)", nbytes, ms,
                       None, launches=reps)
    rec.update({"trees": B, "depth": D, "parents_per_depth": K, "slots": slots, "support": S, "kept": R,
                "ms_per_build": round(ms, 4), "us_per_depth": round(ms * 1e3 / D, 1),
                "note": "latency-bound: 32 rows per depth on 256 compute units; each depth reads 8 logits rows "
                        "per tree (9.7 MB) from HBM once (the per-thread maxima) and again from the cache (the "
                        "gather of the pairs at or above the bound)"})
    return rec


def call_latency_record(seed, steps=50, warmup=5):
    """The two launch-latency configurations (c1: one 15-node tree in fp32; c2: one 60-node tree
    behind a 2048-token prefix, bf16): microseconds per whole-pass call, launched eagerly and as a
    HIP-graph replay of the same call (one graph per input copy, captured once)."""
    import torch

    import tree_masked_verification_attn_amd as tav
    from workloads import gen

    rec = {}
    for name in ("c1", "c2"):
        w = gen.make(name, seed)
        p = Pass(w)
        eager_ms = p.time_steps(steps, warmup)
        s = torch.cuda.Stream()
        graphs = []
        for c in p.copies:
            with torch.cuda.stream(s):
                tav.tav_tree_attn_verify(c.prob, c.tree, c.attn, c.verify, None, None, c.workspace, s, s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                tav.tav_tree_attn_verify(c.prob, c.tree, c.attn, c.verify, None, None, c.workspace, s, s)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / steps
        for c in p.copies:
            bits = tav.tav_read_status(c.workspace)
            if bits:
                raise RuntimeError(f"device status bits set: {tav.device_status_names(bits)}")
        attn_b, ver_b = algorithmic_bytes(w)
        rec[name] = {"workload": f"{name}: {w.info['description']}", "nodes": int(w.N),
                     "us_per_call_eager": round(eager_ms * 1e3, 1), "us_per_call_graph": round(graph_ms * 1e3, 1),
                     "algorithmic_bytes": attn_b + ver_b}
        del graphs, p
        torch.cuda.empty_cache()
    rec["note"] = "launch-latency configurations: microseconds per call, not a bandwidth result"
    return rec


def prefetch_builder_record(seed, reps=200):
    """Host time of tav_prefetch_build at the PreSTO batch's shape (T = 4096, N_pf = 32, K' = 100),
    both rules, and each tree's predicted transition count."""
    import tree_masked_verification_attn_amd as tav

    w = [1.0, -3.0, -1.0, 2.5, 0.0, 0.0]
    rec = {"shape": "T = 4096, N_pf = 32, depth cap 100; class weights (bias, slope) = "
                    "(1, -3) reject, (-1, 2.5) accept, (0, 0) uncertain"}
    for name, rule in (("bfs", tav.TAV_PREFETCH_BFS), ("predictive", tav.TAV_PREFETCH_PREDICTIVE)):
        t0 = time.perf_counter()
        for i in range(reps):
            t = tav.tav_prefetch_build(4096, 32, 100, rule, seed + i, w)
        us = (time.perf_counter() - t0) * 1e6 / reps
        rec[name] = {"us_per_build": round(us, 1), "nodes": int(len(t["parent"])),
                     "requests": int(len(t["request_cut"])),
                     "predicted_transitions": round(float(t["predicted_transitions"]), 4)}
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=10086)
    ap.add_argument("--workload", default="c3", choices=["c2", "c3", "c5"])
    ap.add_argument("--draft-support", type=int, default=0,
                    help="headline workload with sparse draft rows of this support (0: dense)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub", action="store_true", help="headline workload only (profiling runs)")
    ap.add_argument("--sub", default="",
                    help="comma-separated sub-record names to run (default: all of them)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--kernel-steps", type=int, default=20,
                    help="passes / attention-only calls timed by the library's kernel events")
    ap.add_argument("--print-sha", action="store_true",
                    help="print the SHA-256 of the vocabulary workers' sources and exit")
    args = ap.parse_args()
    if args.print_sha:
        print(kernel_source_sha256())
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the scoring pass has no multi-GPU path "
              "(each configuration is one GPU's share); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tree_masked_verification_attn_amd as tav
    from workloads import gen

    tav.load()
    torch.cuda.set_device(0)
    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib * 262144, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ach = None if args.no_sub else achievable(os.path.dirname(tav.LIB_PATH))

    w = gen.make(args.workload, args.seed, draft_support=args.draft_support or None)
    p = Pass(w)
    ms = p.time_steps(args.steps, args.warmup)
    kern_ms, kern_n = p.kernel_ms(2, min(args.steps, args.kernel_steps))
    attn_b, ver_b = algorithmic_bytes(w)
    flops = attention_flops(w)
    attn_rec = attention_record(p, flops, attn_b, args.kernel_steps, ach) if args.kernel_steps > 0 else None
    del p
    step_gbs = (attn_b + ver_b) / (ms * 1e-3) / 1e9
    roof = roofline_hbm("vocab_worker_kernel + pick_kernel (verification: logits and draft rows streamed "
                        "per node, then the pick of every node)",
                        ver_b, kern_ms, ach, traffic=measured_traffic(args.workload), launches=kern_n)

    subs = {}
    if not args.no_sub:
        sub_steps = max(5, min(args.steps, 20))
        only = set(filter(None, args.sub.split(",")))

        def want(name):
            return not only or name in only

        if want("c5_long_context"):
            subs["c5_long_context"] = tree_sub_record(gen.make("c5", args.seed), sub_steps, 3, ach,
                                                      "c5: " + gen.CONFIG_DESCRIPTIONS["c5"])
        if want("c4_presto") or want("c4_token_scores"):
            w4 = gen.make("c4", args.seed)
            if want("c4_presto"):
                subs["c4_presto"] = presto_sub_record(w4, sub_steps, 3, ach)
            if want("c4_token_scores"):
                subs["c4_token_scores"] = scorer_record(args.seed, w4.N + w4.presto.T)
            del w4
        if want("c3_greedy"):
            wg = copy.copy(w)
            wg.temperature = np.zeros_like(w.temperature)
            subs["c3_greedy"] = tree_sub_record(wg, sub_steps, 3, ach,
                                                "c3 at temperature 0: greedy verification (argmax verification tokens)")
        if args.workload == "c3" and not args.draft_support and want("c3_sparse_draft_k128"):
            subs["c3_sparse_draft_k128"] = tree_sub_record(
                gen.make("c3", args.seed, draft_support=128), sub_steps, 3, ach,
                "c3 with sparse draft rows: top-128 support per row (RheoSampling's sparse draft)")
        if want("c1_c2_call_latency"):
            subs["c1_c2_call_latency"] = call_latency_record(args.seed)
        if want("prefetch_builder_host"):
            subs["prefetch_builder_host"] = prefetch_builder_record(args.seed)
        if want("draft_tree_gpu"):
            subs["draft_tree_gpu"] = draft_tree_record(args.seed)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, 1)
        ncores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        cpu["all_cores_run"] = cpu_baseline(w, ncores, min_seconds=5.0, max_passes=2)

    line = {
        "metric": "tree nodes scored/sec (attn+verify) and achieved HBM GB/s vs MI355X peak",
        "value": round(w.N / (ms * 1e-3), 1), "unit": "nodes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": {"workload": f"{args.workload}: {w.info['description']}", "seed": args.seed, "nodes": w.N,
                   "sequences": w.B, "prefix_rows": int(np.sum(w.prefix_len)),
                   "draft_rows_used": _used_draft_rows(w)},
        "step_gbs": round(step_gbs, 1), "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes": attn_b + ver_b,
        "roofline": roof, "attention_kernel": attn_rec, "achievable": ach, "sub_records": subs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
