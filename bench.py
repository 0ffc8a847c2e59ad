"""Benchmark: one decode step of query-aware sparse paged attention on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is the whole hot path for one batch of decode queries: page scoring
against key min/max metadata (with the GQA group-mean query), top-k page
selection, and sparse attention over the selected pages (split-KV partials
and their online-softmax combine).  Page metadata is built once beforehand,
as it is during prefill.

Default workload: Quest-style GQA decode, batch 1, 32 q / 8 KV heads,
head_dim 128, 32768-token context in 16-token pages, 256-page budget, bf16
KV.  Inputs are seeded synthetic data already resident in HBM.  Each timed
step reads a different replica of the KV pool and metadata (R copies at
distinct addresses, R * per-step bytes > 1 GiB), so the 256 MB Infinity
Cache cannot serve repeated steps.

Output: one JSON line with queries/s, the per-step algorithmic HBM bytes and
rate, a roofline entry for the dominant kernel call (timed with HIP events
on its stream) and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "sparse decode attn+select: queries/sec and achieved HBM GB/s (% of peak)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="quest_gqa_32k", choices=["quest_gqa_32k"])
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough for > 1 GiB per rotation")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 10 plain device copies of BYTES (HBM counter calibration) and exit")
    return ap.parse_args()


def copy_calibration(nbytes: int):
    """A plain device-to-device copy of known size: its FETCH_SIZE/WRITE_SIZE
    readings per dispatch calibrate the HBM traffic counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "dispatches": 10}))


def algorithmic_bytes(bt, k_pages):
    """Bytes a step must move from HBM: every valid page's metadata for the
    scoring, plus K and V of the selected pages."""
    elem = 2 if bt.dtype == "bf16" else 4
    g = bt.page_size // bt.logical_page
    units = bt.batch * bt.n_kv_heads
    n_pages = min(bt.max_pages, -(-int(bt.seq_lens[0]) // bt.page_size))
    meta = units * n_pages * g * 2 * bt.head_dim * elem
    kv = units * min(k_pages, n_pages) * bt.page_size * bt.head_dim * 2 * elem
    return meta, kv


def cpu_baseline(bt, k_pages, budget_s):
    """The oracle as it stands, single-threaded: whole decode steps of the
    same workload (score every page of every (sequence, KV head), top-k,
    attention of the group's q heads) repeated for about `budget_s` seconds;
    queries/s = sequences * steps / time."""
    import oracle
    from threadpoolctl import threadpool_limits
    meta, has = oracle.page_meta(bt)          # prefill-time work, not timed
    steps, t_used = 0, 0.0
    with threadpool_limits(1):
        while t_used < budget_s:
            t0 = time.perf_counter()
            scores = oracle.page_scores(bt, meta=meta, has=has)
            ids = oracle.select_topk(bt, scores, k_pages)
            oracle.sparse_decode(bt, ids)
            t_used += time.perf_counter() - t0
            steps += 1
    return {"value": bt.batch * steps / t_used, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} whole decode steps of the workload ({bt.batch * bt.n_kv_heads} (sequence, KV head) "
                      f"units each), {t_used:.1f} s single-threaded fp64 numpy"}


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, if the kernel sources still hash to what was profiled."""
    import glob
    import hashlib
    import re
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        m = re.search(r"```json\n(\{.*?\})\n```", open(path).read(), re.S)
        if not m:
            continue
        rec = json.loads(m.group(1))
        if rec.get("kernel") != kernel or rec.get("workload") != workload:
            continue
        h = hashlib.sha256()
        for f in rec["source_files"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest()[:16] == rec["source_sha256"]:
            return rec["traffic_bytes_per_launch"]
    return None


def main():
    a = parse()
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; multi-GPU sharding is described "
                                   "in the design notes but not built", "n_gpus": a.gpus}))
        sys.exit(2)
    import torch
    import workloads as wl
    import dynamic_sparse_attention_page_amd as dsa

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    bt = wl.make(a.workload)
    k_pages = bt.topk
    meta_b, kv_b = algorithmic_bytes(bt, k_pages)
    step_bytes = meta_b + kv_b
    R = a.replicas or max(1, math.ceil((1 << 30) / step_bytes))

    # --- resident inputs: R replicas of pool, tables and metadata ---------
    q = dsa.upload_q(bt.q, bt.dtype)
    base = dsa.PagedKV.from_numpy(bt.k, bt.v, bt.page_table, bt.seq_lens, bt.dtype)
    S = base.num_slots
    kbig = base.k.repeat(R, 1, 1, 1)
    vbig = base.v.repeat(R, 1, 1, 1)
    pts = torch.cat([base.page_table + r * S for r in range(R)], 0).contiguous()
    pts = torch.where(base.page_table.repeat(R, 1) < 0, torch.full_like(pts, -1), pts).contiguous()
    sls = base.seq_lens.repeat(R).contiguous()
    allkv = dsa.PagedKV(kbig, vbig, pts, sls)
    meta = dsa.page_meta_build(allkv, bt.logical_page)
    del base
    B = bt.batch
    kvs = [dsa.PagedKV(kbig, vbig, pts[r * B:(r + 1) * B].contiguous(), sls[r * B:(r + 1) * B].contiguous())
           for r in range(R)]
    Hq, Hkv, D, N = bt.n_q_heads, bt.n_kv_heads, bt.head_dim, bt.max_pages
    scores = torch.empty((B, Hkv, N), dtype=torch.float32, device=dev)
    ids = torch.empty((B, Hkv, k_pages), dtype=torch.int32, device=dev)
    counts = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    O = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    l = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    m = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.zeros(dsa.workspace_bytes(dsa.OP_SPARSE_DECODE_ATTN, kvs[0], Hq, k_pages), dtype=torch.uint8,
                     device=dev)
    scale = float(bt.scale)

    def step(r):
        kv = kvs[r % R]
        dsa.page_score(q, kv, meta, bt.logical_page, scores=scores)
        dsa.page_select_topk(scores, kv.seq_lens, bt.page_size, k_pages, ids=ids, counts=counts)
        dsa.sparse_decode_attn(q, kv, ids, counts, scale=scale, out=(O, l, m), ws=ws)

    op_fns = {
        "page_score": lambda r: dsa.page_score(q, kvs[r % R], meta, bt.logical_page, scores=scores),
        "page_select_topk": lambda r: dsa.page_select_topk(scores, kvs[r % R].seq_lens, bt.page_size, k_pages,
                                                           ids=ids, counts=counts),
        "sparse_decode_attn": lambda r: dsa.sparse_decode_attn(q, kvs[r % R], ids, counts, scale=scale,
                                                               out=(O, l, m), ws=ws),
    }

    def capture(fn, n):
        """A HIP graph of n calls (replica r = 0..n-1); launches stay on the
        capture stream, no memset nodes."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(n):
                fn(r)
        return g

    def time_graph(g, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # eager (host-launched) step rate, for reference
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(a.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    eager_ms_step = e0.elapsed_time(e1) / a.steps

    # timed region: exactly K steps (replica i mod R) replayed from one graph
    g_step = capture(step, a.steps)
    g_step.replay()                       # untimed warm replay
    torch.cuda.synchronize()
    ms = time_graph(g_step, 1)
    n_steps = a.steps
    ms_step = ms / n_steps
    reps = max(1, math.ceil(a.steps / R))

    # per-call durations: a graph of R launches of one call, timed with
    # events on the stream it replays on
    ops = {}
    for name, fn in op_fns.items():
        g = capture(fn, R)
        g.replay()
        torch.cuda.synchronize()
        ops[name] = time_graph(g, reps) / (reps * R) * 1e3   # us per call
    bytes_of = {"page_score": meta_b, "sparse_decode_attn": kv_b}
    dom = max(bytes_of, key=lambda k: ops[k])
    dur_us, dom_bytes = ops[dom], bytes_of[dom]
    achieved = dom_bytes / (dur_us * 1e-6) / 1e9

    res = {
        "metric": METRIC,
        "value": B * n_steps / (ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": a.workload, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D,
                   "seq_len": int(bt.seq_lens[0]), "page_size": bt.page_size, "topk_pages": k_pages,
                   "replicas": R, "parallelism": "single GPU"},
        "step_bytes": step_bytes,
        "step_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "op_us": {k: round(v, 3) for k, v in ops.items()},
        "eager_ms_per_step": eager_ms_step,
        "timing": "HIP graph of one step per replica, replayed; events on the replay stream",
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": profiled_traffic(dom, a.workload),
                     "bytes_per_launch": dom_bytes, "avg_launch_us": dur_us},
    }
    if not a.no_cpu:
        res["cpu_baseline"] = cpu_baseline(bt, k_pages, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
