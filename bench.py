"""Benchmark: one decode step of query-aware sparse paged attention on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is the whole hot path for one batch of decode queries on inputs
already resident in HBM; page metadata is built beforehand (prefill work).

With no --workload (or --workload all) every workload below runs, each in a
child process of its own and one after the other, and one JSON line is
printed: the headline fields are those of psa_mha_64k, the largest workload
(8 sequences, an 8 GiB bf16 pool, about 0.56 GB of algorithmic bytes per
step), and "workloads" holds the full result of each of the others, timed in
the same run the same way.

  psa_mha_64k (headline)   psa_decode = page_score -> page_select_progressive (threshold
      0.95) in one call: one launch, each (sequence, head) workgroup scoring its own row;
      the two separate calls are timed beside it
      batch 8, 32 heads MHA, d=128, 65536 tokens in 16-token pages, bf16
  quest_gqa_32k            page_score -> sparse_decode_attn_topk (top-k selection + sparse
      attention in one call; the separate page_select_topk and sparse_decode_attn are
      timed beside it)
      batch 1, 32 q / 8 KV heads, d=128, 32768 tokens in 16-token pages, top-256, bf16
  lserve_hier_128k         the same calls with 64/16 hierarchical paging and
      4 of 8 KV heads streaming (sink 128 + local 256); batch 4, 131072 tokens, top-64
  prr_512k                 PRR speculative step in one call (dsa_prr_decode_step): the scores
      (with the EMA update) beside the speculative attention over P in one launch, the
      selection of A, M = A \\ P and the next P, then the speculative combine beside the
      repair's partials, then the repair's fold;
      batch 1, 32 q / 2 KV heads, 524288 tokens, top-2048, 64-step query trace
  tiny_f32                 score, top-8, attention and PSA on one fp32 head
  lserve_prefill_16k       LServe block-sparse prefill of one 16K-token prompt

Each timed step reads a different replica of the KV pool and metadata (R
copies at distinct addresses, R * per-step bytes > 1 GiB) so the 256 MB
Infinity Cache cannot serve repeated steps; PRR replicas run interleaved
64-step traces.  Exactly K steps are captured in one HIP graph and replayed
between HIP events; per-call durations come from graphs of R launches of
one call, timed the same way.

Output: one JSON line (queries/s; one query = one sequence's decode token
through all heads of one layer), the per-step algorithmic HBM bytes and
rate, a roofline entry for the dominant call and the CPU oracle's rate.
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
# calls timed beside the step but not part of it: the roofline names the
# dominant call of the step only
SIDE_OPS = {"kv_append", "prr_calibrate"}
PREFILL = "lserve_prefill_16k"   # the block-sparse prefill workload
MFMA_BF16_TFLOPS = 2500.0        # dense bf16 matrix-core peak
T_CAL = 32   # steps of the score trace the PRR calibration searches over
REUSE_CHUNK = 4   # LServe's default selector-reuse interval
WORKLOADS = ["quest_gqa_32k", "lserve_hier_128k", "psa_mha_64k", "prr_512k", "tiny_f32"]
HEADLINE = "psa_mha_64k"   # the largest workload: its fields head the line
SUB_WORKLOADS = ["quest_gqa_32k", "lserve_hier_128k", "prr_512k", "tiny_f32", PREFILL]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="all", choices=["all"] + list(WORKLOADS) + [PREFILL])
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough for > 1 GiB per rotation")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU oracle sample")
    ap.add_argument("--sub-cpu-seconds", type=float, default=5.0,
                    help="budget of each CPU oracle sample of the workloads after the headline (--workload all)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=min(16, len(os.sched_getaffinity(0))),
                    help="processes of the parallel oracle sample (1: single-threaded only)")
    ap.add_argument("--delta-profile", action="store_true",
                    help="prr_512k: also run PRR's offline speculation-budget profile (4K-64K contexts)")
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


# --------------------------------------------------------------------------
# algorithmic bytes
# --------------------------------------------------------------------------
def _elem(bt):
    return 2 if bt.dtype == "bf16" else 4


def _units(bt):
    """(dense units, streaming units) as (sequence, KV head) counts."""
    n_stream = 0 if bt.streaming is None else int(np.count_nonzero(bt.streaming))
    return bt.batch * (bt.n_kv_heads - n_stream), bt.batch * n_stream


def meta_bytes(bt):
    """kmin + kmax of every valid logical page of every scored (dense) unit."""
    dense, _ = _units(bt)
    n_pages = min(bt.max_pages, -(-int(bt.seq_lens[0]) // bt.page_size))
    return dense * n_pages * (bt.page_size // bt.logical_page) * 2 * bt.head_dim * _elem(bt)


def page_kv_bytes(bt, pages_per_unit, units):
    return int(units * pages_per_unit * bt.page_size * bt.head_dim * 2 * _elem(bt))


def streaming_bytes(bt):
    """K and V of the pages the streaming heads read (sink + local pages)."""
    _, streaming_units = _units(bt)
    if not streaming_units:
        return 0
    L = int(bt.seq_lens[0])
    toks = set(range(min(bt.sink, L))) | set(range(max(0, L - bt.local), L))
    pages = len({t // bt.page_size for t in toks})
    return page_kv_bytes(bt, pages, streaming_units)


# --------------------------------------------------------------------------
# CPU baseline (the oracle as it stands)
# --------------------------------------------------------------------------
def _cpu_sample(bt):
    """Units the oracle runs on: all of them, or a fixed sample of 16 for
    larger batches (scaled by the fraction)."""
    units = None
    if bt.batch * bt.n_kv_heads > 16:
        rng = np.random.default_rng(0)
        all_units = [(b, h) for b in range(bt.batch) for h in range(bt.n_kv_heads)]
        units = set(all_units[i] for i in rng.choice(len(all_units), 16, replace=False))
    frac = 1.0 if units is None else len(units) / (bt.batch * bt.n_kv_heads)
    return units, frac


def _oracle_unit(bt, meta, has, b, h, scores=None):
    """One (sequence, KV head) of a decode step through the oracle: scores,
    selection, attention (PSA: the progressive walk)."""
    import oracle
    if scores is None:
        scores = oracle.page_scores(bt, meta=meta, has=has, units={(b, h)})
    if bt.topk is None:
        oracle.psa_progressive(bt, b, h, scores[b, h], bt.threshold, 0)
        return
    n = oracle.n_pages(bt.seq_lens[b], bt.page_size)
    if bt.streaming is not None and bt.streaming[h]:
        ids = oracle.streaming_pages(bt.seq_lens[b], bt.page_size, bt.sink, bt.local)
    else:
        ids = oracle.topk_pages(scores[b, h], n, bt.topk)
    oracle.attend_pages(bt, b, h, ids)
    if bt.threshold is not None:
        oracle.psa_progressive(bt, b, h, scores[b, h], bt.threshold, 0)


def cpu_baseline(bt, budget_s):
    """The oracle, single-threaded, on whole decode steps of the workload
    (PRR: the plain selection + attention its repair reproduces), repeated
    for about `budget_s` seconds; queries/s = sequences * steps / time.
    Batches of more than 16 (sequence, KV head) units run a fixed sample of
    16 units and scale by the fraction."""
    import oracle
    from threadpoolctl import threadpool_limits
    units, frac = _cpu_sample(bt)
    meta, has = oracle.page_meta(bt, units)          # prefill-time work, not timed
    steps, t_used = 0, 0.0
    with threadpool_limits(1):
        while t_used < budget_s:
            t0 = time.perf_counter()
            scores = oracle.page_scores(bt, meta=meta, has=has, units=units)
            for b in range(bt.batch):
                for h in range(bt.n_kv_heads):
                    if units is not None and (b, h) not in units:
                        continue
                    _oracle_unit(bt, meta, has, b, h, scores)
            t_used += time.perf_counter() - t0
            steps += 1
    sample = (f"{steps} whole decode steps" if units is None else
              f"{steps} decode steps of {len(units)} sampled (sequence, KV head) units, scaled by "
              f"{1 / frac:.0f},")
    return {"value": bt.batch * steps * frac / t_used, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{sample} of the workload; {t_used:.1f} s single-threaded fp64 numpy"}


_PAR = None   # (batch, meta, has) inherited by the forked oracle workers


def _par_unit(u):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        _oracle_unit(*_PAR, *u)


def cpu_baseline_parallel(bt, budget_s, workers):
    """The same oracle steps with the (sequence, KV head) units spread over a
    pool of `workers` single-threaded processes (fork: call it before the GPU
    is touched); wall time per step."""
    import multiprocessing as mp

    import oracle
    global _PAR
    units, frac = _cpu_sample(bt)
    ulist = sorted(units) if units is not None else [(b, h) for b in range(bt.batch) for h in range(bt.n_kv_heads)]
    workers = min(workers, len(ulist))
    if workers < 2:
        return None
    meta, has = oracle.page_meta(bt, units)
    _PAR = (bt, meta, has)
    steps, t_used = 0, 0.0
    with mp.get_context("fork").Pool(workers) as pool:
        pool.map(_par_unit, ulist[:workers], chunksize=1)          # start-up, untimed
        while t_used < budget_s:
            t0 = time.perf_counter()
            pool.map(_par_unit, ulist, chunksize=1)
            t_used += time.perf_counter() - t0
            steps += 1
    _PAR = None
    return {"value": bt.batch * steps * frac / t_used, "unit": "queries/s", "cores": workers, "kind": "oracle",
            "sample": f"{steps} decode steps of {len(ulist)} (sequence, KV head) units"
                      f"{'' if units is None else f' (sampled, scaled by {1 / frac:.0f})'} over {workers} "
                      f"single-threaded processes; {t_used:.1f} s wall"}


# --------------------------------------------------------------------------
# GPU timing
# --------------------------------------------------------------------------
def reuse_coverage(dsa, torch, wl, bt, kv, meta, st, q, steps=8, theta=0.1):
    """Share of a fresh top-k that the reused pages cover, on a drifting
    query trace (angle theta per step), averaged over the steps that reuse;
    dense heads only."""
    qs = wl.query_drift(91, bt.q, steps, theta, bt.dtype)
    from dynamic_sparse_attention_page_amd.reuse import ChunkedReuseDecoder
    dec = ChunkedReuseDecoder(kv, meta, bt.n_q_heads, bt.topk, chunk=REUSE_CHUNK, logical_page=bt.logical_page,
                              streaming=st)
    cov = []
    for t in range(steps):
        qt = dsa.upload_q(qs[t], bt.dtype)
        dec.step(qt)
        sc = dsa.page_score(qt, kv, meta, bt.logical_page, streaming=st)
        ids_f, cnt_f = dsa.page_select_topk(sc, kv.seq_lens, bt.page_size, bt.topk, streaming=st)
        if t % REUSE_CHUNK == 0:
            continue
        a, ca, r, cr = (x.cpu().numpy() for x in (ids_f, cnt_f, dec.ids, dec.counts))
        for b in range(bt.batch):
            for h in range(bt.n_kv_heads):
                if bt.streaming is not None and bt.streaming[h]:
                    continue
                fresh = set(a[b, h, :ca[b, h]].tolist())
                cov.append(len(fresh & set(r[b, h, :cr[b, h]].tolist())) / max(1, len(fresh)))
    return {"theta_per_step": theta, "mean": float(np.mean(cov)), "min": float(np.min(cov))}


def host_signal_latency(dsa, torch, ops, counts, iters=30):
    """Host wall time from enqueueing a PSA step (scores + progressive
    selection) to holding its page counts: through the zero-copy signal
    (dsa_signal_host + polling a pinned flag) vs a synchronising copy.
    Medians in microseconds."""
    import time
    host = torch.zeros(counts.numel(), dtype=torch.int32, pin_memory=True)
    flag = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    res = {}
    for kind in ("signal", "sync_copy"):
        ts = []
        for it in range(iters):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            ops["page_score"](0)
            ops["page_select_progressive"](0)
            if kind == "signal":
                dsa.signal_host(counts.view(-1), host, flag, 1000 + it)
                if not dsa.wait_host_flag(flag, 1000 + it, timeout_s=10.0):
                    raise RuntimeError("host signal never arrived")
            else:
                counts.view(-1).cpu()
            ts.append((time.perf_counter() - t0) * 1e6)
        res[kind + "_us"] = float(np.median(ts))
    return res


def replicate(dsa, torch, bt, R):
    """R copies of pool, page table and metadata at distinct addresses;
    returns one PagedKV view per replica and the metadata."""
    base = dsa.PagedKV.from_numpy(bt.k, bt.v, bt.page_table, bt.seq_lens, bt.dtype)
    S = base.num_slots
    kbig = base.k.repeat(R, 1, 1, 1)
    vbig = base.v.repeat(R, 1, 1, 1)
    pts = torch.cat([torch.where(base.page_table < 0, base.page_table, base.page_table + r * S) for r in range(R)],
                    0).contiguous()
    sls = base.seq_lens.repeat(R).contiguous()
    meta = dsa.page_meta_build(dsa.PagedKV(kbig, vbig, pts, sls), bt.logical_page)
    B = bt.batch
    kvs = [dsa.PagedKV(kbig, vbig, pts[r * B:(r + 1) * B].contiguous(), sls[r * B:(r + 1) * B].contiguous())
           for r in range(R)]
    return kvs, meta


def prefill_pairs(L: int, streaming, sink: int, local: int, G: int) -> int:
    """(query, key) pairs the prefill attends to, over all q heads."""
    i = np.arange(L, dtype=np.int64)
    dense = int(((i + 1)).sum())
    lam = np.minimum(i + 1, sink) + np.maximum(0, i - np.maximum(sink, i - local + 1) + 1)
    return G * sum(int(lam.sum()) if s else dense for s in streaming)


def run_prefill(a, dsa, torch, wl):
    """LServe's block-sparse prefill on the 16K-token prompt: prefill tokens
    per second, against the bf16 matrix-core peak on the attended pairs."""
    import time
    cfg = wl.PREFILL_16K
    L, Hq, Hkv, D = cfg["L"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    q, k, v = wl.prefill_inputs(cfg["seed"], L, Hq, Hkv, D, "bf16")
    qd, kd, vd = (dsa.upload_q(x, "bf16") for x in (q, k, v))
    st = dsa.Streaming(cfg["streaming"], cfg["sink"], cfg["local"])
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = dsa.block_sparse_prefill(qd, kd, vd, streaming=st, scale=scale)
    for _ in range(a.warmup):
        dsa.block_sparse_prefill(qd, kd, vd, streaming=st, scale=scale, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(a.steps):
            dsa.block_sparse_prefill(qd, kd, vd, streaming=st, scale=scale, out=out)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    G = Hq // Hkv
    pairs = prefill_pairs(L, cfg["streaming"], cfg["sink"], cfg["local"], G)
    flops = 4.0 * D * pairs                      # q.k and p.v, 2 flops per multiply-add
    n_qt = -(-L // 64)
    dense_tiles = n_qt * (n_qt + 1) // 2
    res = {
        "metric": "block-sparse prefill: prompt tokens/s",
        "value": L / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL, "seq_len": L, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D,
                   "streaming_kv_heads": int(np.count_nonzero(cfg["streaming"])), "sink": cfg["sink"],
                   "local": cfg["local"], "tile": 64, "parallelism": "single GPU"},
        "attended_pairs": pairs,
        "block_sparsity_vs_causal": 1.0 - pairs / (G * Hkv * L * (L + 1) / 2),
        "dense_head_tiles": dense_tiles,
        "roofline": {"bound": "mfma", "kernel": "block_sparse_prefill", "achieved": flops / (ms * 1e-3) / 1e12,
                     "peak": MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_TFLOPS, "traffic": None,
                     "flops_per_launch": flops, "avg_launch_us": ms * 1e3},
    }
    if not a.no_cpu:   # the oracle on a bounded sample of queries (all heads of each)
        import oracle
        qf, kf, vf = (oracle.widen(x, "bf16") for x in (q, k, v))
        rng = np.random.default_rng(0)
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < a.cpu_seconds:
            i = int(rng.integers(0, L))
            for hq in range(Hq):
                hk = hq // G
                j = oracle.prefill_keys(i, L, bool(cfg["streaming"][hk]), cfg["sink"], cfg["local"])
                oracle.attention(qf[i, hq], kf[j, hk], vf[j, hk], scale)
            n += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": n / dt, "unit": "tokens/s (uniformly sampled query positions)",
                               "cores": 1, "kind": "oracle", "sample": f"{n} query tokens x {Hq} heads"}
    print(json.dumps(res), flush=True)


def run_all(a):
    """Every workload in a child process of its own, one after the other
    (each forks its CPU oracle pool before touching the GPU; this process
    never touches it); prints the headline workload's line with the other
    results under "workloads"."""
    import subprocess
    results = {}
    for w in [HEADLINE] + SUB_WORKLOADS:
        cmd = [sys.executable, os.path.abspath(__file__), "--workload", w, "--steps", str(a.steps), "--warmup",
               str(a.warmup), "--cpu-workers", str(a.cpu_workers),
               "--cpu-seconds", str(a.cpu_seconds if w == HEADLINE else a.sub_cpu_seconds)]
        if a.no_cpu:
            cmd.append("--no-cpu")
        if a.replicas:
            cmd += ["--replicas", str(a.replicas)]
        print(f"bench: {w} ...", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
        lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
        if r.returncode != 0 or not lines:
            sys.stderr.write(r.stdout)
            print(f"bench: {w} failed (exit {r.returncode})", file=sys.stderr, flush=True)
            sys.exit(r.returncode or 1)
        results[w] = json.loads(lines[-1])
        print(f"bench: {w} done in {time.perf_counter() - t0:.1f} s: {results[w]['value']:.1f} "
              f"{results[w]['unit']}", file=sys.stderr, flush=True)
    head = dict(results[HEADLINE])
    head["workloads"] = {w: results[w] for w in SUB_WORKLOADS}
    print(json.dumps(head), flush=True)


def main():
    a = parse()
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; multi-GPU sharding is described "
                                   "in the design notes but not built", "n_gpus": a.gpus}))
        sys.exit(2)
    if a.workload == "all":
        run_all(a)
        return
    import torch
    import workloads as wl
    import dynamic_sparse_attention_page_amd as dsa

    if a.workload == PREFILL:
        torch.cuda.set_device(0)
        run_prefill(a, dsa, torch, wl)
        return
    bt = wl.make(a.workload)
    cpu_par = None
    if not a.no_cpu and a.cpu_workers > 1:   # forks: before the GPU is initialised
        cpu_par = cpu_baseline_parallel(bt, a.cpu_seconds, a.cpu_workers)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    B, Hq, Hkv, D, N = bt.batch, bt.n_q_heads, bt.n_kv_heads, bt.head_dim, bt.max_pages
    scale = float(bt.scale)
    st = None if bt.streaming is None else dsa.Streaming(bt.streaming, bt.sink, bt.local)
    dense_units, _ = _units(bt)
    mb = meta_bytes(bt)
    f32, i32 = torch.float32, torch.int32
    scores = torch.empty((B, Hkv, N), dtype=f32, device=dev)
    O = torch.empty((B, Hq, D), dtype=f32, device=dev)
    l = torch.empty((B, Hq), dtype=f32, device=dev)
    m = torch.empty((B, Hq), dtype=f32, device=dev)

    # per-step byte estimate for the replica count (refined below)
    if a.workload == "prr_512k":
        est = mb + 2 * page_kv_bytes(bt, bt.topk, B * Hkv)
    elif a.workload == "psa_mha_64k":
        est = mb
    else:
        est = mb + page_kv_bytes(bt, bt.topk, dense_units) + streaming_bytes(bt)
    R = a.replicas or max(1, math.ceil((1 << 30) / est))
    kvs, meta = replicate(dsa, torch, bt, R)
    q = dsa.upload_q(bt.q, bt.dtype)

    extra = {}
    step_end = None
    reuse_step = None
    if a.workload == "prr_512k":
        from dynamic_sparse_attention_page_amd.prr import PRRDecoder
        a_, b_, g_ = bt.extra["ema"]
        T = bt.extra["steps"]
        qt = torch.from_numpy(bt.extra["q_trace"].view(np.int16)).to(dev).view(torch.bfloat16)
        decs = [PRRDecoder(kv, meta, Hq, bt.topk, a_, b_, g_, bt.extra["delta"], scale=scale) for kv in kvs]

        def step(i):   # step i: replica i mod R at trace step 1 + (i // R) mod (T - 1), a speculative step
            r = i % R
            decs[r].t = 1 + (i // R) % (T - 1)
            decs[r].step(qt[decs[r].t])

        def step_end():   # the side streams' last predictor updates join the caller's stream
            for d in decs:
                d.join()
        # one pass over the traces: predictor state and the measured miss rate
        miss, prev_p = [], None
        for t in range(T):
            for r in range(R):
                decs[r].t = t
                decs[r].step(qt[t])
            step_end()
            torch.cuda.synchronize()
            A = decs[0].a_ids.cpu().numpy()
            if prev_p is not None:
                miss.append(np.mean([len(set(A[0, h].tolist()) - set(prev_p[0, h].tolist())) / bt.topk
                                     for h in range(Hkv)]))
            prev_p = decs[0].p_ids.cpu().numpy()
        miss_rate = float(np.mean(miss))
        extra["prr_miss_rate"] = {"mean": miss_rate, "min": float(np.min(miss)), "max": float(np.max(miss))}
        kvb = page_kv_bytes(bt, bt.topk, B * Hkv)
        step_bytes = mb + kvb + miss_rate * kvb + B * Hkv * N * (24 + 8)
        sel_ws = torch.empty(dsa.prr_select_workspace_bytes(B, Hkv, N), dtype=torch.uint8, device=dev)
        ops = {
            "page_score": lambda r: dsa.page_score(q, kvs[r], meta, scores=decs[r].scores),
            "page_select_topk": lambda r: dsa.page_select_topk(decs[r].scores, kvs[r].seq_lens, bt.page_size,
                                                               bt.topk, ids=decs[r].a_ids, counts=decs[r].a_counts),
            "sparse_decode_attn": lambda r: dsa.sparse_decode_attn(q, kvs[r], decs[r].p_ids, decs[r].p_counts,
                                                                   scale=scale, out=(O, l, m), ws=decs[r].ws),
            # the repair as the decoder runs it: over the missing set M = A \ P the selection wrote
            "attn_repair": lambda r: dsa.attn_repair(q, kvs[r], decs[r].m_ids, decs[r].m_counts, None, None, O, l,
                                                     m, scale=scale, ws=decs[r].ws),
            # the same repair given A and P (M formed inside, through an LDS bitmap of P)
            "attn_repair_filter": lambda r: dsa.attn_repair(q, kvs[r], decs[r].a_ids, decs[r].a_counts,
                                                            decs[r].p_ids, decs[r].p_counts, O, l, m, scale=scale,
                                                            ws=decs[r].ws),
            "ema_predict_update": lambda r: dsa.ema_predict_update(decs[r].scores, decs[r].level, decs[r].trend,
                                                                   decs[r].pred, a_, b_, g_),
            "prr_select": lambda r: dsa.prr_select(decs[r].scores, kvs[r].seq_lens, bt.page_size, bt.topk,
                                                   decs[r].level, decs[r].trend, decs[r].pred, a_, b_, g_, False,
                                                   decs[r].k_spec, decs[r].a_ids, decs[r].a_counts,
                                                   decs[r].p_ids, decs[r].p_counts, split=False),
            # the same call with a workspace: the split-row selection (many CUs)
            "prr_select_split": lambda r: dsa.prr_select(decs[r].scores, kvs[r].seq_lens, bt.page_size, bt.topk,
                                                         decs[r].level, decs[r].trend, decs[r].pred, a_, b_, g_,
                                                         False, decs[r].k_spec, decs[r].a_ids, decs[r].a_counts,
                                                         decs[r].p_ids, decs[r].p_counts, ws=sel_ws),
        }
        if decs[0].one_stream:
            # the whole speculative step as the decoder runs it: one call, four launches
            ops["prr_decode_step"] = lambda r: dsa.prr_decode_step(
                q, kvs[r], meta, decs[r].scores, decs[r].level, decs[r].trend, decs[r].pred, a_, b_, g_, bt.topk,
                decs[r]._p[0], (decs[r].a_ids, decs[r].a_counts), (decs[r].m_ids, decs[r].m_counts), decs[r]._p[1],
                O, l, m, scale=scale, ws=decs[r].step_ws)
        op_bytes = {"page_score": mb, "sparse_decode_attn": kvb, "ema_predict_update": B * Hkv * N * 24,
                    "attn_repair": int(miss_rate * kvb)}
        # online calibration of (alpha, beta, gamma) over the 80-candidate grid
        # on a score trace of T_CAL steps (runs beside prefill, not in the step)
        cal_trace = torch.from_numpy(wl.score_trace(77, T_CAL, B * Hkv, N)).to(dev)
        cal_nv = torch.full((B * Hkv,), N, dtype=i32, device=dev)
        cal_H = torch.empty((B * Hkv, dsa.CALIB_CANDIDATES), dtype=f32, device=dev)
        cal_best = torch.empty((B * Hkv,), dtype=i32, device=dev)
        cal_ws = torch.empty(int(dsa.lib.dsa_prr_calibrate_workspace_bytes(T_CAL, B * Hkv, N)), dtype=torch.uint8,
                             device=dev)
        ops["prr_calibrate"] = lambda r: dsa.prr_calibrate(cal_trace, cal_nv, bt.topk, decs[r].k_spec, H=cal_H,
                                                           best=cal_best, ws=cal_ws)
        op_bytes["prr_calibrate"] = T_CAL * B * Hkv * N * 4
        if a.delta_profile:   # section 3.4: the offline profile behind the speculation budget (opt-in: it
            # launches the attention kernels at other shapes, which would blend into their trace averages)
            from dynamic_sparse_attention_page_amd.prr import profile_delta_table
            _, extra["prr_delta_profile"] = profile_delta_table(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                                                                page_size=bt.page_size)
    elif bt.topk is None or a.workload == "tiny_f32":   # PSA (and the tiny workload: top-k and PSA)
        ids_p = torch.empty((B, Hkv, N), dtype=i32, device=dev)
        cnt_p = torch.empty((B, Hkv), dtype=i32, device=dev)
        Op = (torch.empty_like(O), torch.empty_like(l), torch.empty_like(m))
        ops = {
            "page_score": lambda r: dsa.page_score(q, kvs[r], meta, scores=scores),
            "page_select_progressive": lambda r: dsa.page_select_progressive(
                q, kvs[r], scores, bt.threshold, 0, scale, out=(ids_p, cnt_p, *Op)),
        }
        if bt.topk is None:
            # the step: both calls in one (one launch when the rows cover the CUs);
            # the two calls are timed beside it
            ops["psa_decode"] = lambda r: dsa.psa_decode(q, kvs[r], meta, bt.threshold, 0, scale,
                                                         out=(scores, ids_p, cnt_p, *Op))
        if bt.topk is not None:
            ids = torch.empty((B, Hkv, bt.topk), dtype=i32, device=dev)
            cnt = torch.empty((B, Hkv), dtype=i32, device=dev)
            ws = torch.zeros(dsa.workspace_bytes(dsa.OP_SPARSE_DECODE_ATTN, kvs[0], Hq, bt.topk), dtype=torch.uint8,
                             device=dev)
            ops["page_select_topk"] = lambda r: dsa.page_select_topk(scores, kvs[r].seq_lens, bt.page_size,
                                                                     bt.topk, ids=ids, counts=cnt)
            ops["sparse_decode_attn"] = lambda r: dsa.sparse_decode_attn(q, kvs[r], ids, cnt, scale=scale,
                                                                         out=(O, l, m), ws=ws)

        def step(i):
            if "psa_decode" in ops:
                ops["psa_decode"](i % R)
            else:
                for fn in ops.values():
                    fn(i % R)
        step(0)
        torch.cuda.synchronize()
        visited = float(cnt_p.float().mean().item())
        extra["psa_pages_visited"] = {"mean": visited, "max": int(cnt_p.max().item())}
        extra["psa_host_signal"] = host_signal_latency(dsa, torch, ops, cnt_p)
        step_bytes = mb + page_kv_bytes(bt, visited, B * Hkv)
        op_bytes = {"page_score": mb, "page_select_progressive": page_kv_bytes(bt, visited, B * Hkv)}
        if bt.topk is None:
            op_bytes["psa_decode"] = mb + page_kv_bytes(bt, visited, B * Hkv)
        if bt.topk is not None:
            step_bytes += page_kv_bytes(bt, bt.topk, B * Hkv)
            op_bytes["sparse_decode_attn"] = page_kv_bytes(bt, bt.topk, B * Hkv)
    else:   # quest_gqa_32k, lserve_hier_128k
        k_pages = bt.topk
        ids = torch.empty((B, Hkv, k_pages), dtype=i32, device=dev)
        cnt = torch.empty((B, Hkv), dtype=i32, device=dev)
        ws = torch.zeros(dsa.workspace_bytes(dsa.OP_SPARSE_DECODE_ATTN, kvs[0], Hq, k_pages), dtype=torch.uint8,
                         device=dev)
        ops = {
            "page_score": lambda r: dsa.page_score(q, kvs[r], meta, bt.logical_page, streaming=st, scores=scores),
            "sparse_decode_attn_topk": lambda r: dsa.sparse_decode_attn_topk(
                q, kvs[r], scores, k_pages, streaming=st, scale=scale, out=(O, l, m), ids=ids, counts=cnt, ws=ws),
            # the two calls the fused one stands for, timed on their own (not part of the step)
            "page_select_topk": lambda r: dsa.page_select_topk(scores, kvs[r].seq_lens, bt.page_size, k_pages,
                                                               streaming=st, ids=ids, counts=cnt),
            "sparse_decode_attn": lambda r: dsa.sparse_decode_attn(q, kvs[r], ids, cnt, streaming=st, scale=scale,
                                                                   out=(O, l, m), ws=ws),
        }

        def step(i):   # score -> top-k selection + sparse attention (one call)
            ops["page_score"](i % R)
            ops["sparse_decode_attn_topk"](i % R)

        # LServe's reusable selector (section 4.3): the selector runs on the
        # first token of every chunk of REUSE_CHUNK steps, later tokens reuse
        # its pages; timed over a whole number of chunks per replica
        from dynamic_sparse_attention_page_amd.reuse import ChunkedReuseDecoder
        reuse_decs = [ChunkedReuseDecoder(kv_r, meta, Hq, k_pages, chunk=REUSE_CHUNK, logical_page=bt.logical_page,
                                          streaming=st, scale=scale) for kv_r in kvs]
        reuse_steps = REUSE_CHUNK * R * max(1, round(a.steps / (REUSE_CHUNK * R)))

        def reuse_step(i):
            reuse_decs[i % R].step(q)
        kvb = page_kv_bytes(bt, k_pages, dense_units) + streaming_bytes(bt)
        step_bytes = mb + kvb
        op_bytes = {"page_score": mb, "sparse_decode_attn_topk": kvb + 4 * N * B * Hkv, "sparse_decode_attn": kvb}

    # decode-time append, timed on its own (it precedes the step and is not
    # part of it): each sequence's last token is written again at its own
    # position (lengths one short, new lengths into a side buffer), which
    # leaves the cache as it was
    P_, Pl_ = bt.page_size, bt.logical_page
    app_lens = torch.empty((B,), dtype=i32, device=dev)
    app = []
    for kv_r in kvs:
        lens = kv_r.seq_lens.cpu().numpy()
        pt = kv_r.page_table.cpu().numpy()
        rows = [(int(pt[b, (int(L) - 1) // P_]), (int(L) - 1) % P_) for b, L in enumerate(lens)]
        kn = torch.stack([kv_r.k[s, :, o] for s, o in rows]).contiguous()
        vn = torch.stack([kv_r.v[s, :, o] for s, o in rows]).contiguous()
        app.append((dsa.PagedKV(kv_r.k, kv_r.v, kv_r.page_table, (kv_r.seq_lens - 1).contiguous()), kn, vn))
    ops["kv_append"] = lambda r: dsa.kv_append(app[r][0], app[r][1], app[r][2], meta, Pl_, new_seq_lens=app_lens)
    op_bytes["kv_append"] = B * Hkv * 8 * D * _elem(bt)   # k/v rows in and out, kmin/kmax read and written

    def capture(fn, n, end=None):
        """A HIP graph of n calls fn(0..n-1) on the capture stream (no memset nodes)."""
        torch.cuda.synchronize()
        if end is not None:
            end()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
            if end is not None:
                end()
        return g

    def time_graph(g, reps):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # eager (host-launched) steps: warmup, and the reference eager rate
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(a.steps):
        step(i)
    if step_end is not None:
        step_end()
    e1.record()
    torch.cuda.synchronize()
    eager_ms_step = e0.elapsed_time(e1) / a.steps

    # timed region: exactly K steps replayed from one graph
    g_step = capture(step, a.steps, step_end)
    g_step.replay()                       # untimed warm replay
    ms = time_graph(g_step, 1)
    ms_step = ms / a.steps

    if reuse_step is not None:
        g_reuse = capture(reuse_step, reuse_steps)
        g_reuse.replay()
        ms_reuse = time_graph(g_reuse, 1)
        extra["chunked_reuse"] = {"chunk": REUSE_CHUNK, "steps": reuse_steps,
                                  "ms_per_step": ms_reuse / reuse_steps,
                                  "queries_per_s": B * reuse_steps / (ms_reuse * 1e-3),
                                  "speedup_vs_step": ms_step / (ms_reuse / reuse_steps),
                                  "coverage": reuse_coverage(dsa, torch, wl, bt, kvs[0], meta, st, q)}

    # per-call durations: graphs of R launches of one call
    reps = max(1, math.ceil(a.steps / R))
    op_us = {}
    for name, fn in ops.items():
        g = capture(fn, R)
        g.replay()
        op_us[name] = time_graph(g, reps) / (reps * R) * 1e3
    dom = max((k for k in op_bytes if k not in SIDE_OPS), key=lambda k: op_us[k])
    dur_us, dom_bytes = op_us[dom], op_bytes[dom]
    achieved = dom_bytes / (dur_us * 1e-6) / 1e9

    cfg = {"workload": a.workload, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D,
           "seq_len": int(bt.seq_lens[0]), "page_size": bt.page_size, "logical_page": bt.logical_page,
           "topk_pages": bt.topk, "threshold": bt.threshold, "kv_dtype": bt.dtype, "replicas": R,
           "parallelism": "single GPU"}
    if bt.streaming is not None:
        cfg.update(streaming_kv_heads=int(np.count_nonzero(bt.streaming)), sink=bt.sink, local=bt.local)
    res = {
        "metric": METRIC,
        "value": B * a.steps / (ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": bt.dtype,
        "data": "synthetic",
        "config": cfg,
        "step_bytes": int(step_bytes),
        "step_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "op_us": {k: round(v, 3) for k, v in op_us.items()},
        "eager_ms_per_step": eager_ms_step,
        "timing": "HIP graph of K steps replayed once between events; per-call graphs of R launches",
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": profiled_traffic(dom, a.workload),
                     "bytes_per_launch": int(dom_bytes), "avg_launch_us": dur_us},
    }
    res.update(extra)
    if not a.no_cpu:
        res["cpu_baseline"] = cpu_baseline(bt, a.cpu_seconds)
        if cpu_par is not None:
            res["cpu_baseline_parallel"] = cpu_par
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
