"""The fused calls captured in a HIP graph give the eager result on every
replay: psa_decode (scores, progressive selection and attention in one
launch), sparse_decode_attn_topk with hierarchical paging and streaming
heads, attn_repair folding into its caller's (O, l, m) in place (compacted M
and P filtered), and the block-sparse prefill.  Before each replay the pure
outputs are poisoned and the in-place operands restored; eager work and
synchronisations run between replays.  The comparison is bit for bit (the
same kernels on the same inputs); each call is checked against the oracle
elsewhere (test_gpu_parity, test_gpu_fused, test_gpu_psa_fused,
test_gpu_prefill)."""
import numpy as np
import pytest
import torch

import workloads as wl
from parity_util import to_device

pytestmark = pytest.mark.gpu


def _same(x: torch.Tensor, y: torch.Tensor) -> bool:
    if x.dtype == torch.float32:
        return torch.equal(x.view(torch.int32), y.view(torch.int32))
    return torch.equal(x, y)


def _poison(ts):
    for t in ts:
        if t.dtype == torch.float32:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


def _check_replays(name, step, outs, restore=lambda: None, reps=4):
    print(f"[case] graph replay {name}", flush=True)
    restore()
    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(reps):
        restore()
        _poison([x for x in outs if not getattr(x, "_in_place", False)])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, r) in enumerate(zip(outs, ref)):
            assert _same(x, r), f"{name}: replay {rep}, output {i}"
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()   # eager work between replays


@pytest.mark.parametrize("wide", [False, True])
def test_graph_psa_decode(gpu_lib, wide):
    """Few rows: the score and progressive launches; rows that cover the
    CUs: one launch."""
    dsa = gpu_lib
    if wide:
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        Hkv = 32
        B = max(8, -(-n_cu // Hkv))
        rng = np.random.default_rng(951)
        lens = [0, 5] + [int(x) for x in rng.integers(16 * 40, 16 * 120, size=B - 2)]
    else:
        Hkv, B = 4, 3
        lens = [16 * 900 + 3, 16 * 40, 5]
    bt = wl.random_batch(951, lens, n_q_heads=Hkv, n_kv_heads=Hkv, head_dim=128, page_size=16)
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv)
    dev = q.device
    out = (torch.empty((B, Hkv, kv.max_pages), device=dev),
           torch.empty((B, Hkv, kv.max_pages), dtype=torch.int32, device=dev),
           torch.empty((B, Hkv), dtype=torch.int32, device=dev),
           torch.empty((B, Hkv, 128), device=dev), torch.empty((B, Hkv), device=dev),
           torch.empty((B, Hkv), device=dev))
    for thr, mode in ((0.95, 0), (0.6, 1)):
        _check_replays(f"psa_decode thr={thr} mode={mode}",
                       lambda: dsa.psa_decode(q, kv, meta, thr, mode, float(bt.scale), out=out), list(out))


def test_graph_topk_hierarchical_streaming(gpu_lib):
    dsa = gpu_lib
    flags = np.array([1, 0, 0, 1], np.uint8)
    bt = wl.random_batch(952, [64 * 300 + 17, 64 * 7, 0, 64 * 120], n_q_heads=16, n_kv_heads=4, head_dim=128,
                         page_size=64, logical_page=16, streaming=flags, sink=128, local=256)
    q, kv, st = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, 16)
    dev = q.device
    B, Hkv, k = kv.batch, kv.n_kv_heads, 24
    sc = torch.empty((B, Hkv, kv.max_pages), device=dev)
    ids = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    O, l, m = (torch.empty((B, 16, 128), device=dev), torch.empty((B, 16), device=dev),
               torch.empty((B, 16), device=dev))
    ws = torch.zeros(dsa.workspace_bytes(dsa.OP_SPARSE_DECODE_ATTN, kv, 16, k), dtype=torch.uint8, device=dev)

    def step():
        dsa.page_score(q, kv, meta, 16, streaming=st, scores=sc)
        dsa.sparse_decode_attn_topk(q, kv, sc, k, streaming=st, scale=float(bt.scale), out=(O, l, m), ids=ids,
                                    counts=cnt, ws=ws)

    _check_replays("page_score + sparse_decode_attn_topk (64/16 pages, streaming heads)", step,
                   [sc, ids, cnt, O, l, m])


@pytest.mark.parametrize("filtered", [False, True])
def test_graph_repair_in_place(gpu_lib, filtered):
    dsa = gpu_lib
    bt = wl.random_batch(953, [16 * 2000 + 9, 16 * 600], n_q_heads=32, n_kv_heads=2, head_dim=128,
                         page_size=16)
    q, kv, _ = to_device(dsa, bt)
    dev = q.device
    B, Hkv, k = kv.batch, kv.n_kv_heads, 256
    rng = np.random.default_rng(5)
    a = np.full((B, Hkv, k), -1, np.int32)
    p = np.full((B, Hkv, k), -1, np.int32)
    ac = np.zeros((B, Hkv), np.int32)
    pc = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        npg = -(-int(bt.seq_lens[b]) // 16)
        for h in range(Hkv):
            sel = np.sort(rng.choice(npg, size=min(k, npg), replace=False))
            a[b, h, :len(sel)] = sel
            ac[b, h] = len(sel)
            keep = np.sort(rng.choice(sel, size=len(sel) * 3 // 4, replace=False))   # P shares 3/4 of A
            extra = np.setdiff1d(np.arange(npg), sel)[: len(sel) - len(keep)]
            ps = np.sort(np.concatenate([keep, extra]))
            p[b, h, :len(ps)] = ps
            pc[b, h] = len(ps)
    if not filtered:   # the compacted missing set M = A \ P
        for b in range(B):
            for h in range(Hkv):
                msk = np.setdiff1d(a[b, h, :ac[b, h]], p[b, h, :pc[b, h]])
                a[b, h] = -1
                a[b, h, :len(msk)] = msk
                ac[b, h] = len(msk)
    t = lambda x: torch.from_numpy(x).to(dev)
    a_ids, a_cnt, p_ids, p_cnt = t(a), t(ac), t(p), t(pc)
    # the caller's speculative result over P
    O0, l0, m0 = dsa.sparse_decode_attn(q, kv, p_ids, p_cnt, scale=float(bt.scale))
    O, l, m = O0.clone(), l0.clone(), m0.clone()
    for x in (O, l, m):
        x._in_place = True
    ws = torch.zeros(dsa.workspace_bytes(dsa.OP_ATTN_REPAIR, kv, 32, k), dtype=torch.uint8, device=dev)

    def restore():
        O.copy_(O0)
        l.copy_(l0)
        m.copy_(m0)

    if filtered:
        step = lambda: dsa.attn_repair(q, kv, a_ids, a_cnt, p_ids, p_cnt, O, l, m, scale=float(bt.scale), ws=ws)
    else:
        step = lambda: dsa.attn_repair(q, kv, a_ids, a_cnt, None, None, O, l, m, scale=float(bt.scale), ws=ws)
    _check_replays(f"attn_repair ({'P filtered' if filtered else 'compacted M'})", step, [O, l, m], restore)


def test_graph_prefill(gpu_lib):
    dsa = gpu_lib
    L, Hq, Hkv, D = 700, 8, 4, 128
    g = torch.Generator(device="cpu").manual_seed(954)
    q, k, v = (torch.randn((L, h, D), generator=g).to(torch.bfloat16).cuda() for h in (Hq, Hkv, Hkv))
    st = dsa.Streaming(np.array([0, 1, 0, 1], np.uint8), 64, 200)
    dev = q.device
    out = (torch.empty((L, Hq, D), device=dev), torch.empty((L, Hq), device=dev), torch.empty((L, Hq), device=dev))
    _check_replays("block_sparse_prefill (streaming heads)",
                   lambda: dsa.block_sparse_prefill(q, k, v, streaming=st, out=out), list(out))
