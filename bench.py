"""Throughput of the tree-masked scoring pass on one MI355X.

Workload (default): 16 sequences, prefix lengths uniform in [1024, 8192] in a
paged KV cache (block 16, shuffled block table), 64-node random trees of depth
<= 8, 32 query / 8 KV heads, head_dim 128, bf16, vocabulary 151936, T = 1.0,
seed 10086 -- the batched verification shape.  Inputs are synthetic (seeded).

One step = one whole pass, one tav_tree_attn_verify call: the call's start
kernel (status reset, the verification workers' node order), tree preparation
(with the attention work plan and node packing), split-KV tree attention and its
merge, then the verification's vocabulary workers and the walk, all on one
stream.  With --separate the step is tav_tree_attention and tav_tree_verify on
their own streams and workspaces instead (which also times each half).  Inputs
are resident in HBM; two input copies alternate so consecutive steps do not
re-read one step's data from the 256 MB last-level cache.

Prints one JSON line:  value = tree nodes scored per second (attention +
verification), plus the step's algorithmic HBM GB/s, the roofline of the
dominant kernel -- the vocabulary workers of the verification, the longest
kernel of the pass and an HBM stream, timed per launch by HIP events the
library records around it on its own stream over the timed region -- with the
HBM traffic measured by counters for the same kernel source (or null), the
attention kernel's roofline from a second timed loop of attention-only calls,
and the oracle's throughput on the same workload on one host core.
"""

import argparse
import json
import os
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


def algorithmic_bytes(w):
    """Bytes the pass must move: each prefix KV row once per (sequence, KV head),
    each node's q / k / v / out once, each logits row once, each draft row that
    verification uses once (nodes with a sampled child), small per-node arrays."""
    import numpy as np

    eb = 2 if w.dtype == "bf16" else 4
    kv = int(sum(int(L) for L in w.prefix_len)) * w.Hkv * w.D * eb * 2
    nodes = w.N * (w.Hq * w.D * eb * 2 + w.Hkv * w.D * eb * 2 + w.Hq * 4)
    attn = kv + nodes + int(w.block_table.size) * 4
    verify = 0
    if w.logits is not None:
        has_s = np.zeros(w.N, bool)
        for b in range(w.B):
            s = int(w.node_offsets[b])
            for c in range(s + 1, int(w.node_offsets[b + 1])):
                if w.sampled[c]:
                    has_s[s + int(w.parent[c])] = True
        used = int(np.sum(has_s & (w.draft_row >= 0)))
        verify = w.N * w.V * eb + used * w.V * 4 + w.N * (4 + 1 + 4 + 1 + 8)
    return attn, verify


def attention_flops(w):
    import oracle

    prep = oracle.tree_prep(w.parent, w.node_offsets, w.prefix_len)
    keys = 0
    for b in range(w.B):
        for v in w.seq_nodes(b):
            keys += int(w.prefix_len[b]) + int(prep["depth"][v]) + 1
    return 4 * w.D * w.Hq * keys


def cpu_baseline(w, min_seconds=10.0, max_passes=4):
    """The oracle, as it is, on the whole workload (attention of every node + verification
    walk of every sequence), one thread, repeated until about min_seconds of CPU work."""
    from threadpoolctl import threadpool_limits

    import oracle

    seqs = list(range(w.B))
    nodes = [v for b in seqs for v in w.seq_nodes(b)]
    passes, dt = 0, 0.0
    with threadpool_limits(1):
        while passes < max_passes and (passes == 0 or dt < min_seconds):
            t0 = time.perf_counter()
            oracle.tree_attention(w, nodes)
            oracle.verify_workload(w, seqs)
            dt += time.perf_counter() - t0
            passes += 1
    return {"value": passes * len(nodes) / dt, "unit": "nodes/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole workload ({w.B} sequences, {len(nodes)} nodes: attention of every "
                      f"node + verification walk) x {passes} passes, {dt:.1f} s"}


def kernel_source_sha256():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the vocabulary workers' kernel from the committed counter data, or
    None when the kernel sources have changed since the counters were taken."""
    if not os.path.exists(PMC_FILE):
        return None
    rec = json.load(open(PMC_FILE))
    if rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return int(rec["hbm_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=10086)
    ap.add_argument("--workload", default="c3", choices=["c2", "c3", "c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=2)
    ap.add_argument("--separate", action="store_true",
                    help="attention and verification as two calls with their own workspaces")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--attn-steps", type=int, default=20,
                    help="attention-only calls timed after the main loop (the attention kernel's roofline)")
    ap.add_argument("--print-sha", action="store_true",
                    help="print the SHA-256 of the vocabulary workers' sources and exit")
    args = ap.parse_args()
    if args.print_sha:
        print(kernel_source_sha256())
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the scoring pass has no multi-GPU path in this build "
              "(each configuration is one GPU's share); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tree_masked_verification_attn_amd as tav
    from workloads import device as wdev
    from workloads import gen

    torch.cuda.set_device(0)
    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib * 262144, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = gen.make(args.workload, args.seed)
    copies = [wdev.upload(w, "cuda") for _ in range(max(1, args.copies))]
    # verification's own workspaces (separate calls only)
    ws_v = [torch.zeros_like(c.workspace) for c in copies] if args.separate else [None] * len(copies)
    sa = torch.cuda.Stream()
    sv = torch.cuda.Stream()
    torch.cuda.synchronize()

    def step(i, ev=None):
        c = copies[i % len(copies)]
        if not args.separate:
            if ev is not None:
                ev[0].record(sa)
            tav.tav_tree_attn_verify(c.prob, c.tree, c.attn, c.verify, None, None, c.workspace, sa, sv)
            if ev is not None:
                ev[1].record(sa)
            return
        if ev is not None:
            ev[0].record(sa)
        tav.tav_tree_attention(c.prob, c.tree, c.attn, c.workspace, sa)
        if ev is not None:
            ev[1].record(sa)
            ev[2].record(sv)
        tav.tav_tree_verify(c.prob, c.tree, c.verify, ws_v[i % len(copies)], sv)
        if ev is not None:
            ev[3].record(sv)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the timed steps: nothing but the calls (events between kernels cost a few microseconds each)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for c, wv in zip(copies, ws_v):
        bits = tav.tav_read_status(c.workspace) | (tav.tav_read_status(wv) if wv is not None else 0)
        if bits:
            raise RuntimeError(f"device status bits set: {tav.device_status_names(bits)}")

    # then the same steps again with events: around each call, and (in the library) around the
    # vocabulary workers' kernel on its stream, for that kernel's launch time
    n_ev = min(args.steps, 20)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_ev)]
    tav.tav_kernel_timing(2)
    torch.cuda.synchronize()
    for i in range(n_ev):
        step(i, events[i])
    torch.cuda.synchronize()
    kern_ms_total, kern_launches = tav.tav_kernel_timing_read()
    tav.tav_kernel_timing(0)
    kern_ms = kern_ms_total / max(1, kern_launches)
    attn_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    ver_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events])) if args.separate else None

    # the attention kernel alone: attention-only calls on one stream, events around the kernel
    a_ms = None
    if args.attn_steps > 0:
        for i in range(2):
            c = copies[i % len(copies)]
            tav.tav_tree_attention(c.prob, c.tree, c.attn, c.workspace, sa)
        torch.cuda.synchronize()
        tav.tav_kernel_timing(1)
        for i in range(args.attn_steps):
            c = copies[i % len(copies)]
            tav.tav_tree_attention(c.prob, c.tree, c.attn, c.workspace, sa)
        torch.cuda.synchronize()
        a_total, a_n = tav.tav_kernel_timing_read()
        tav.tav_kernel_timing(0)
        a_ms = a_total / max(1, a_n)

    ms = wall * 1e3 / args.steps
    attn_b, ver_b = algorithmic_bytes(w)
    flops = attention_flops(w)
    step_gbs = (attn_b + ver_b) / (ms * 1e-3) / 1e9

    # roofline of the dominant kernel: the vocabulary workers (per launch = one step's verification)
    kern_gbs = ver_b / (kern_ms * 1e-3) / 1e9
    roof = {"kernel": "vocab_worker_kernel (verification: logits and draft rows streamed per node)",
            "bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
            "avg_launch_ms": round(kern_ms, 4), "launches_timed": kern_launches,
            "algorithmic_bytes": ver_b}
    attn_roof = None
    if a_ms is not None:
        a_gbs = attn_b / (a_ms * 1e-3) / 1e9
        attn_roof = {"kernel": "attn_bf16_kernel (tree-masked attention, bf16 MFMA), attention-only calls",
                     "bound": "hbm", "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(a_gbs / HBM_PEAK_GBS, 4), "avg_launch_ms": round(a_ms, 4),
                     "launches_timed": args.attn_steps, "algorithmic_bytes": attn_b,
                     "mfma_tflops": round(flops / (a_ms * 1e-3) / 1e12, 1),
                     "mfma_frac": round(flops / (a_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    if args.separate:
        other = {"mode": "separate calls", "attention_half_ms": round(attn_ms, 4),
                 "attention_half_gbs": round(attn_b / (attn_ms * 1e-3) / 1e9, 1),
                 "verify_half_ms": round(ver_ms, 4),
                 "verify_half_gbs": round(ver_b / (ver_ms * 1e-3) / 1e9, 1)}
    else:
        other = {"mode": "one tav_tree_attn_verify call", "pass_event_ms": round(attn_ms, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w)

    desc = gen.CONFIG_DESCRIPTIONS[args.workload]
    line = {
        "metric": "tree nodes scored/sec (attn+verify) and achieved HBM GB/s vs MI355X peak",
        "value": round(w.N / (ms * 1e-3), 1), "unit": "nodes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": {"workload": f"{args.workload}: {desc}", "seed": args.seed, "nodes": w.N,
                   "sequences": w.B, "prefix_rows": int(np.sum(w.prefix_len)),
                   "draft_rows": int(w.draft.shape[0]) if w.draft is not None else 0},
        "step_gbs": round(step_gbs, 1), "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes": attn_b + ver_b,
        "roofline": roof, "attention_kernel": attn_roof, "kernels": other, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
