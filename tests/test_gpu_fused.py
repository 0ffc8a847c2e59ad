"""GPU parity of dsa_sparse_decode_attn_topk (selection recomputed inside
the attention workgroups) against the two separate calls it replaces and
against the fp64 oracle: ids and counts bit-exact with dsa_page_select_topk
(same fp32 scores), (O, l, m) to the attention tolerance of the oracle over
those pages.  Covers both row widths of the fused path (<= 2048 and <= 4096
pages), streaming heads, k above the valid page count, empty sequences,
fp32 KV, and the fallback (16 heads per KV head; rows above 4096 pages)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import check_selected_attention, check_selection, np_, to_device

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _run(dsa, bt, k, st=None):
    q, kv, st0 = to_device(dsa, bt)
    st = st or st0
    meta = dsa.page_meta_build(kv, bt.logical_page)
    sc = dsa.page_score(q, kv, meta, bt.logical_page, streaming=st)
    ids_f, cnt_f, O, l, m = dsa.sparse_decode_attn_topk(q, kv, sc, k, streaming=st)
    ids_s, cnt_s = dsa.page_select_topk(sc, kv.seq_lens, bt.page_size, k, streaming=st)
    O2, l2, m2 = dsa.sparse_decode_attn(q, kv, ids_s, cnt_s, streaming=st)
    torch.cuda.synchronize()
    assert np.array_equal(np_(cnt_f), np_(cnt_s)), "counts differ from dsa_page_select_topk"
    assert np.array_equal(np_(ids_f), np_(ids_s)), "ids differ from dsa_page_select_topk"
    # same pages, same kernels: the outputs of the two routes agree to rounding
    np.testing.assert_allclose(np_(O), np_(O2), rtol=0, atol=1e-6)
    # against the oracle: its scores and its selection (boundary rule), and
    # the outputs against its attention over its own selection
    ref = oracle.page_scores(bt)
    idn, cn = np_(ids_f), np_(cnt_f)
    units = [(b, h) for b in range(bt.batch) for h in range(bt.n_kv_heads)]
    for b, h in units:
        if bt.streaming is None or not bt.streaming[h]:
            check_selection(idn[b, h], int(cn[b, h]), ref[b, h], oracle.n_pages(bt.seq_lens[b], bt.page_size), k,
                            f"fused (b={b}, h={h})")
    check_selected_attention(dsa, bt, q, kv, st, idn, cn, (O, l, m), oracle.select_topk(bt, ref, k), units, "fused")


@pytest.mark.parametrize("dtype,D,P,G,max_pages,k", [
    ("bf16", 128, 16, 4, 2048, 256),     # quest shape, 8 scores per thread
    ("bf16", 128, 16, 4, 3000, 100),     # 16 scores per thread
    ("bf16", 64, 16, 2, 500, 37),
    ("f32", 64, 16, 1, 700, 64),
    ("bf16", 128, 16, 16, 600, 48),      # fallback: two launches
    ("bf16", 128, 16, 4, 5000, 64),      # fallback: row above 4096 pages
])
def test_fused_topk_attention(gpu_lib, dtype, D, P, G, max_pages, k):
    dsa = gpu_lib
    _banner(f"fused {dtype} D={D} P={P} G={G} N={max_pages} k={k}")
    lens = [0, 5, P * 3 + 1, P * (max_pages // 3) + 7, P * max_pages]
    bt = wl.random_batch(81, lens, n_q_heads=2 * G, n_kv_heads=2, head_dim=D, page_size=P, dtype=dtype,
                         max_pages=max_pages)
    _run(dsa, bt, k)


def test_fused_streaming_heads(gpu_lib):
    dsa = gpu_lib
    _banner("fused streaming heads")
    bt = wl.random_batch(82, [64 * 20 + 30, 64 * 8, 200, 64 * 300], n_q_heads=8, n_kv_heads=4, head_dim=128,
                         page_size=64, logical_page=16, streaming=[1, 0, 0, 1], sink=128, local=256)
    _run(dsa, bt, 8)


def test_fused_quest_workload(gpu_lib):
    dsa = gpu_lib
    _banner("fused quest_gqa_32k")
    bt = wl.make("quest_gqa_32k")
    _run(dsa, bt, bt.topk)


def test_fused_exact_ties(gpu_lib):
    dsa = gpu_lib
    _banner("fused exact score ties")
    bt = wl.random_batch(83, [16 * 900 + 5, 16 * 400], n_q_heads=8, n_kv_heads=2, head_dim=128, max_pages=1000,
                         dup_pages=40)
    _run(dsa, bt, 30)


def _host_scores(rng, B, H, N, kind):
    """Adversarial float32 score rows for the selection inside the fused
    call: exact ties (with -0 and +0), wide magnitude ranges with -inf,
    +inf entries, a constant row and a two-valued row."""
    if kind == "ties":
        s = rng.integers(-3, 4, size=(B, H, N)).astype(np.float32)
        s[s == 0] = np.where(rng.random((s == 0).sum()) < 0.5, -0.0, 0.0)
    elif kind == "mixed":
        s = (rng.standard_normal((B, H, N)) * 10.0 ** rng.integers(-3, 4, size=(B, H, N))).astype(np.float32)
        s[rng.random((B, H, N)) < 0.02] = -np.inf
        s[rng.random((B, H, N)) < 0.005] = np.inf
    elif kind == "constant":
        s = np.full((B, H, N), 7.25, np.float32)
    else:  # two values, far apart
        s = np.where(rng.random((B, H, N)) < 0.3, np.float32(1e30), np.float32(-1e-30)).astype(np.float32)
    return s


@pytest.mark.parametrize("N", [5, 64, 65, 700, 2048, 4096])
@pytest.mark.parametrize("kind", ["ties", "mixed", "constant", "two"])
def test_fused_selection_exact(gpu_lib, N, kind):
    """Host-made scores fed to the fused call: its ids and counts equal the
    oracle's top-k (ties to the lower index) bit for bit, for k in
    {1, 63, 64, 65, N/16, N-1, N, N+5}, with ragged lengths; the attention is
    checked against the oracle over those pages."""
    dsa = gpu_lib
    rng = np.random.default_rng(N * 13 + len(kind))
    P = 16
    lens = [N * P, max(0, N * P - 37), 3]
    bt = wl.random_batch(91, lens, n_q_heads=8, n_kv_heads=2, head_dim=128, page_size=P, dtype="bf16",
                         max_pages=N)
    q, kv, _ = to_device(dsa, bt)
    B, H = bt.batch, bt.n_kv_heads
    s = _host_scores(rng, B, H, N, kind)
    sc = torch.from_numpy(s).cuda()
    for k in sorted({1, 63, 64, 65, max(1, N // 16), max(1, N - 1), N, N + 5}):
        _banner(f"fused selection N={N} kind={kind} k={k}")
        ids, cnt, O, l, m = dsa.sparse_decode_attn_topk(q, kv, sc, k)
        torch.cuda.synchronize()
        ids, cnt = np_(ids), np_(cnt)
        ref_sel = {}
        for b in range(B):
            nv = oracle.n_pages(bt.seq_lens[b], P)
            for h in range(H):
                ref = oracle.topk_pages(s[b, h].astype(np.float64), nv, k)
                assert cnt[b, h] == len(ref), (b, h, k)
                assert np.array_equal(ids[b, h, :len(ref)], ref), (b, h, k)
                assert np.all(ids[b, h, len(ref):] == -1)
                ref_sel[(b, h)] = ref
        if k in (64, N + 5):
            units = [(b, h) for b in range(B) for h in range(H)]
            ref_ids = [[ref_sel[(b, h)] for h in range(H)] for b in range(B)]
            check_selected_attention(dsa, bt, q, kv, None, ids, cnt, (O, l, m), ref_ids, units,
                                     f"fused selection N={N} {kind} k={k}")
