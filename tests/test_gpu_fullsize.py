"""Full-size parity: the five workloads at their real shapes, run through the
C ABI with the same calls bench.py times, checked against the oracle on
every output the oracle can afford (all units for the smaller workloads,
sampled (sequence, KV head) units for the large ones), plus properties that
hold at any size."""
import math
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import (check_attention, check_selected_attention, check_selection, np_, to_device,
                         upload_ids)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"[full] {msg}", flush=True)


def _gen(name):
    t = time.time()
    bt = wl.make(name)
    _log(f"{name}: generated in {time.time() - t:.1f} s")
    return bt


def _sample_units(bt, n, seed, dense_only=False):
    rng = np.random.default_rng(seed)
    units = [(b, h) for b in range(bt.batch) for h in range(bt.n_kv_heads)
             if not (dense_only and bt.streaming is not None and bt.streaming[h])]
    pick = rng.choice(len(units), size=min(n, len(units)), replace=False)
    return sorted(units[i] for i in pick)


def _check_meta(dsa, bt, meta_gpu, units):
    ref, has = oracle.page_meta(bt, set(units))
    got = np_(meta_gpu.float()).astype(np.float64)
    for b, h in units:
        slots = bt.page_table[b, :oracle.n_pages(bt.seq_lens[b], bt.page_size)]
        sel = has[slots, h]
        assert np.array_equal(got[slots, h][sel], ref[slots, h][sel]), f"meta (b={b}, h={h})"


def _check_scores(sc_gpu, ref, units):
    for b, h in units:
        g, r = sc_gpu[b, h].astype(np.float64), ref[b, h]
        assert np.array_equal(np.isneginf(g), np.isneginf(r)), f"score -inf pattern (b={b}, h={h})"
        fin = np.isfinite(r)
        err = np.abs(g[fin] - r[fin]) / np.maximum(1.0, np.abs(r[fin]))
        assert err.max() <= 2e-6, f"score error {err.max():.3g} at (b={b}, h={h})"


def test_tiny_f32_full(gpu_lib):
    """1 query, 1 head, fp32: top-8, PSA at 0.95 (both stop rules), and the
    dense limits k = N and threshold = 1."""
    dsa = gpu_lib
    bt = _gen("tiny_f32")
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv)
    sc = dsa.page_score(q, kv, meta)
    ref = oracle.page_scores(bt)
    _check_meta(dsa, bt, meta, [(0, 0)])
    _check_scores(np_(sc), ref, [(0, 0)])
    N = bt.max_pages
    for k in (bt.topk, N):
        ids, cnt = dsa.page_select_topk(sc, kv.seq_lens, bt.page_size, k)
        idn, cn = np_(ids), np_(cnt)
        check_selection(idn[0, 0], int(cn[0, 0]), ref[0, 0], N, k, f"tiny top-{k}")
        O, l, m = dsa.sparse_decode_attn(q, kv, ids, cnt)
        check_selected_attention(dsa, bt, q, kv, None, idn, cn, (O, l, m), oracle.select_topk(bt, ref, k),
                                 [(0, 0)], f"tiny attention k={k}")
    dO, dl, dm = oracle.dense_attention(bt)
    check_attention("f32", np_(O), np_(l), np_(m), dO, dl, dm, "tiny k=N is dense")
    # the progressive selection takes the oracle's scores (rounded to float32)
    # as its input, and the oracle ranks the same values
    s32 = ref.astype(np.float32)
    scn = s32.astype(np.float64)
    for thr, mode in ((0.95, 0), (0.95, 1), (1.0, 0)):
        ids, cnt, O, l, m = dsa.page_select_progressive(q, kv, torch.from_numpy(s32).cuda(), thr, mode)
        n = int(np_(cnt)[0, 0])
        rid, rn, *_ = oracle.psa_progressive(bt, 0, 0, scn[0, 0], thr, mode)
        assert n == rn, (thr, mode, n, rn)
        assert np.array_equal(np_(ids)[0, 0, :n], rid)
        ref_att = oracle.attend_pages(bt, 0, 0, rid)
        check_attention("f32", np_(O)[0], np_(l)[0], np_(m)[0], *ref_att, f"tiny psa thr={thr} mode={mode}")
        if mode == 0 and thr < 1:
            assert n <= math.ceil(thr / (1 - thr))
    check_attention("f32", np_(O), np_(l), np_(m), dO, dl, dm, "tiny threshold 1 is dense")


def test_quest_gqa_32k_full(gpu_lib):
    """Every unit of the quest workload: metadata, scores, selection, outputs."""
    dsa = gpu_lib
    bt = _gen("quest_gqa_32k")
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv)
    sc = dsa.page_score(q, kv, meta)
    ids, cnt = dsa.page_select_topk(sc, kv.seq_lens, bt.page_size, bt.topk)
    O, l, m = dsa.sparse_decode_attn(q, kv, ids, cnt)
    torch.cuda.synchronize()
    units = [(0, h) for h in range(bt.n_kv_heads)]
    t = time.time()
    ref_meta, has = oracle.page_meta(bt)
    ref = oracle.page_scores(bt, meta=ref_meta, has=has)
    _log(f"quest oracle scores in {time.time() - t:.1f} s")
    _check_meta(dsa, bt, meta, units)
    scn, idn, cn = np_(sc), np_(ids), np_(cnt)
    _check_scores(scn, ref, units)
    swaps = 0
    for b, h in units:
        swaps += check_selection(idn[b, h], int(cn[b, h]), ref[b, h], bt.max_pages, bt.topk, f"quest h={h}")
        # the biased pages (cosine 0.4 to the group query) are all selected
        assert set(bt.extra["biased_pages"][b, h]) <= set(idn[b, h, :cn[b, h]].tolist())
    reruns = check_selected_attention(dsa, bt, q, kv, None, idn, cn, (O, l, m), oracle.select_topk(bt, ref, bt.topk),
                                      units, "quest attention")
    _log(f"quest: {swaps} exempted boundary swaps, {reruns} units checked on the oracle's ids")


def test_lserve_hier_128k_full(gpu_lib):
    """Hierarchical 64/16 paging with streaming heads, sampled units."""
    dsa = gpu_lib
    bt = _gen("lserve_hier_128k")
    q, kv, st = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, bt.logical_page)
    sc = dsa.page_score(q, kv, meta, bt.logical_page, streaming=st)
    ids, cnt = dsa.page_select_topk(sc, kv.seq_lens, bt.page_size, bt.topk, streaming=st)
    O, l, m = dsa.sparse_decode_attn(q, kv, ids, cnt, streaming=st)
    torch.cuda.synchronize()
    dense = _sample_units(bt, 4, 7, dense_only=True)
    stream_units = [(b, h) for b in range(bt.batch) for h in range(bt.n_kv_heads) if bt.streaming[h]][:3]
    t = time.time()
    ref = oracle.page_scores(bt, units=set(dense))
    _log(f"lserve oracle scores ({len(dense)} units) in {time.time() - t:.1f} s")
    _check_meta(dsa, bt, meta, dense)
    scn, idn, cn = np_(sc), np_(ids), np_(cnt)
    _check_scores(scn, ref, dense)
    for b, h in stream_units:
        assert np.all(np.isneginf(scn[b, h]))
        exp = oracle.streaming_pages(bt.seq_lens[b], bt.page_size, bt.sink, bt.local)
        assert np.array_equal(idn[b, h, :cn[b, h]], exp)
    for b, h in dense:
        check_selection(idn[b, h], int(cn[b, h]), ref[b, h], bt.max_pages, bt.topk, f"lserve (b={b}, h={h})")
    check_selected_attention(dsa, bt, q, kv, st, idn, cn, (O, l, m), oracle.select_topk(bt, ref, bt.topk),
                             dense + stream_units, "lserve attention")


def test_psa_mha_64k_full(gpu_lib):
    """PSA progressive selection at 0.95 on the MHA workload: every unit's
    stop count obeys the printed rule's bound; sampled units match the oracle
    (stop count, rank order, output), for both stop rules."""
    dsa = gpu_lib
    bt = _gen("psa_mha_64k")
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv)
    sc = dsa.page_score(q, kv, meta)
    res = {mode: dsa.page_select_progressive(q, kv, sc, bt.threshold, mode) for mode in (0, 1)}
    torch.cuda.synchronize()
    cnt0 = np_(res[0][1])
    assert cnt0.min() >= 1 and cnt0.max() <= math.ceil(bt.threshold / (1 - bt.threshold))
    _log(f"psa printed rule: pages visited min {cnt0.min()} mean {cnt0.mean():.1f} max {cnt0.max()}; "
         f"remaining-pages rule: mean {np_(res[1][1]).mean():.1f} max {np_(res[1][1]).max()}")
    units = _sample_units(bt, 5, 11)
    t = time.time()
    ref = oracle.page_scores(bt, units=set(units))
    _log(f"psa oracle scores ({len(units)} units) in {time.time() - t:.1f} s")
    _check_meta(dsa, bt, meta, units)
    scn = np_(sc)
    _check_scores(scn, ref, units)
    # sampled units: the progressive selection runs again with the oracle's
    # scores (rounded to float32) in their rows, and the oracle ranks the same values
    s_in = scn.copy()
    for b, h in units:
        s_in[b, h] = ref[b, h].astype(np.float32)
    s_dev = torch.from_numpy(s_in).cuda()
    for mode in (0, 1):
        ids, cnt, O, l, m = (np_(x) for x in dsa.page_select_progressive(q, kv, s_dev, bt.threshold, mode))
        for b, h in units:
            row = s_in[b, h].astype(np.float64)
            rid, rn, *_ = oracle.psa_progressive(bt, b, h, row, bt.threshold, mode)
            n = int(cnt[b, h])
            if n != rn:
                ratios = oracle.psa_ratios(bt, b, h, row, mode)
                lo, hi = min(n, rn), max(n, rn)
                assert np.any(np.abs(ratios[lo - 1:hi] - bt.threshold) <= 1e-5), (mode, b, h, n, rn)
            ranked = oracle.rank_pages(row, bt.max_pages)
            assert np.array_equal(ids[b, h, :n], ranked[:n])
            r = oracle.attend_pages(bt, b, h, ids[b, h, :n])
            check_attention("bf16", O[b, h:h + 1], l[b, h:h + 1], m[b, h:h + 1], *r,
                            f"psa mode={mode} (b={b}, h={h})")


def test_prr_512k_full(gpu_lib):
    """The 64-step PRR trace through the decoder (its speculative steps in one
    dsa_prr_decode_step call at this shape), against the
    oracle's own run of the same trace (its scores, its top-k A^t, an fp64
    EMA fed its scores, its speculative sets P^{t+1}): per step the scores,
    A^t and P^{t+1} under the boundary rule, the predictions, and (sampled
    steps) the repaired output against attention over P^t u A^t.  Reports
    the miss rate |A \\ P| / |A| of the decoder's sets."""
    dsa = gpu_lib
    from dynamic_sparse_attention_page_amd.prr import PRRDecoder
    bt = _gen("prr_512k")
    q0, kv, _ = to_device(dsa, bt)
    qt = torch.from_numpy(bt.extra["q_trace"].view(np.int16)).cuda().view(torch.bfloat16)
    meta = dsa.page_meta_build(kv)
    a_, b_, g_ = bt.extra["ema"]
    dec = PRRDecoder(kv, meta, bt.n_q_heads, bt.topk, a_, b_, g_, bt.extra["delta"])
    N, k, H = bt.max_pages, bt.topk, bt.n_kv_heads
    units = [(0, h) for h in range(H)]
    ref_meta, ref_has = oracle.page_meta(bt)
    lvl = trd = None
    ref_p = gpu_p = None
    misses, exempt = [], 0
    for t in range(bt.extra["steps"]):
        O, l, m = dec.step(qt[t])
        torch.cuda.synchronize()
        bq = wl.Batch(**{**bt.__dict__, "q": bt.extra["q_trace"][t]})
        ref = oracle.page_scores(bq, meta=ref_meta, has=ref_has)
        _check_scores(np_(dec.scores), ref, units)
        A_ids, A_cnt = np_(dec.a_ids), np_(dec.a_counts)
        ref_a = [oracle.topk_pages(ref[0, h], N, k) for h in range(H)]
        for h in range(H):
            exempt += check_selection(A_ids[0, h], int(A_cnt[0, h]), ref[0, h], N, k, f"prr A step {t} h={h}")
        if t % 16 == 0 or t == bt.extra["steps"] - 1:
            # P^t u A^t: the decoder's sets against the oracle's; where they
            # differ by an exempted pair the attention runs on the oracle's union
            want = [np.array(sorted(set(ref_a[h].tolist()) | (set(ref_p[h]) if ref_p is not None else set())),
                             np.int64) for h in range(H)]
            got = [np.array(sorted(set(A_ids[0, h, :A_cnt[0, h]].tolist()) | (set(gpu_p[h]) if gpu_p else set())),
                            np.int64) for h in range(H)]
            On, ln, mn = np_(O), np_(l), np_(m)
            G = bt.group
            for h in range(H):
                r = oracle.attend_pages(bq, 0, h, want[h])
                sl = slice(h * G, (h + 1) * G)
                if np.array_equal(got[h], want[h]):
                    check_attention("bf16", On[0, sl], ln[0, sl], mn[0, sl], *r, f"prr step {t} h={h}")
                else:
                    it, ct = upload_ids([want], max(len(w) for w in want))
                    O2, l2, m2 = (np_(x) for x in dsa.sparse_decode_attn(qt[t], kv, it, ct))
                    check_attention("bf16", O2[0, sl], l2[0, sl], m2[0, sl], *r, f"prr step {t} h={h}, oracle sets")
            _log(f"prr step {t}: scores, selections and repaired output match")
        # the oracle's EMA runs on its own scores
        IS = ref.reshape(-1)
        if lvl is None:
            lvl, trd = IS.copy(), np.zeros(IS.size)
        else:
            lvl, trd = oracle.ema_update(IS, lvl, trd, a_, b_)
        pred_ref = oracle.ema_predict(lvl, trd, g_)
        pred = np_(dec.pred).astype(np.float64).reshape(-1)
        # Derived bound.  The EMA is linear and contracting: a score error e
        # moves the level by at most max|e| and the trend by at most 2 max|e|,
        # so the prediction by at most (1 + 2 gamma) max|e|; the scores agree
        # to 2e-6 relative (the score parity bound) and each step's fp32
        # rounding adds under one ulp of the scale to the level (damped by
        # 1 - alpha).  (1 + 2 * 0.25) * 2e-6 + 2 * 2^-24 / 0.6 < 3.3e-6 of
        # max|IS|: checked at 1e-5 of max|pred|, a 3x margin.
        assert np.allclose(pred, pred_ref, rtol=0.0, atol=1e-5 * np.abs(pred_ref).max())
        P_ids, P_cnt = np_(dec.p_ids), np_(dec.p_counts)
        predr = pred_ref.reshape(ref.shape)
        kp = int(math.floor(dec.delta * k))
        for h in range(H):
            exempt += check_selection(P_ids[0, h], int(P_cnt[0, h]), predr[0, h], N, kp, f"prr P step {t} h={h}")
        if gpu_p is not None:
            mr = np.mean([np.setdiff1d(A_ids[0, h, :A_cnt[0, h]], gpu_p[h]).size / A_cnt[0, h] for h in range(H)])
            misses.append(mr)
        gpu_p = [P_ids[0, h, :P_cnt[0, h]].tolist() for h in range(H)]
        ref_p = [oracle.speculative_set(predr[0, h], N, k, dec.delta).tolist() for h in range(H)]
    _log(f"prr: {exempt} exempted boundary swaps over the trace")
    misses = np.array(misses)
    _log(f"prr miss rate |A\\P|/|A| over steps 1..63: min {misses.min():.3f} mean {misses.mean():.3f} "
         f"max {misses.max():.3f}")
