"""GPU parity of dsa_prr_select (A^t, the EMA update and P^{t+1}) against
the calls it stands for: dsa_page_select_topk on the scores,
dsa_ema_predict_update, dsa_page_select_topk on the prediction.
ids and counts bit-exact; level, trend and pred equal to the separate EMA
call (same float arithmetic); and the selections exact against the oracle
on the GPU's own scores / predictions."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import np_, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("max_pages,k,k_spec", [(700, 64, 64), (2048, 256, 200), (5000, 300, 300),
                                                (32768, 2048, 2048)])
def test_prr_select_matches_separate_calls(gpu_lib, max_pages, k, k_spec):
    dsa = gpu_lib
    print(f"[case] prr_select N={max_pages} k={k} k_spec={k_spec}", flush=True)
    P = 16
    lens = [P * max_pages, P * (max_pages // 2) + 5, 7]
    bt = wl.random_batch(91, lens, n_q_heads=4, n_kv_heads=2, head_dim=64, page_size=P, max_pages=max_pages)
    q, kv, _ = to_device(dsa, bt)
    B, H, N = bt.batch, bt.n_kv_heads, max_pages
    # inputs from the host: the oracle's scores (rounded to float32, -inf past
    # each sequence) and seeded EMA state
    s_h = oracle.page_scores(bt).astype(np.float32)
    hr0 = np.random.default_rng(5)
    lvl_h = hr0.standard_normal(B * H * N).astype(np.float32)
    trd_h = hr0.standard_normal(B * H * N).astype(np.float32)
    lvl0, trd0 = torch.from_numpy(lvl_h).cuda(), torch.from_numpy(trd_h).cuda()
    i32 = torch.int32
    for init in (True, False):
        sc = torch.from_numpy(s_h).cuda()
        # fused
        lv1, tr1, pr1 = lvl0.clone(), trd0.clone(), torch.empty(B * H * N, device="cuda")
        a1, ac1 = torch.empty((B, H, k), dtype=i32, device="cuda"), torch.empty((B, H), dtype=i32, device="cuda")
        p1, pc1 = torch.empty((B, H, k_spec), dtype=i32, device="cuda"), torch.empty((B, H), dtype=i32, device="cuda")
        dsa.prr_select(sc, kv.seq_lens, P, k, lv1, tr1, pr1, 0.6, 0.3, 0.25, init, k_spec, a1, ac1, p1, pc1)
        # separate calls
        lv2, tr2, pr2 = lvl0.clone(), trd0.clone(), torch.empty(B * H * N, device="cuda")
        a2, ac2 = dsa.page_select_topk(sc, kv.seq_lens, P, k)
        dsa.ema_predict_update(sc, lv2, tr2, pr2, 0.6, 0.3, 0.25, init=init)
        p2, pc2 = dsa.page_select_topk(pr2.view(B, H, N), kv.seq_lens, P, k_spec)
        torch.cuda.synchronize()
        assert np.array_equal(np_(ac1), np_(ac2)) and np.array_equal(np_(a1), np_(a2)), "A differs"
        assert np.array_equal(np_(pc1), np_(pc2)) and np.array_equal(np_(p1), np_(p2)), "P differs"
        for x, y, what in ((lv1, lv2, "level"), (tr1, tr2, "trend"), (pr1, pr2, "pred")):
            assert np.array_equal(np_(x), np_(y)), f"{what} differs from dsa_ema_predict_update"
        # the prediction in the kernel's float32 arithmetic, then both selections
        if init:
            pr_ref = s_h.reshape(-1)
        else:
            pr_ref = oracle.ema_predict_f32(*oracle.ema_step_f32(s_h.reshape(-1), lvl_h, trd_h, 0.6, 0.3), 0.25)
        assert np.array_equal(np_(pr1), pr_ref), "prediction differs from the oracle's float32 EMA"
        scn, prn = s_h.astype(np.float64), pr_ref.astype(np.float64).reshape(B, H, N)
        ref_a = {}
        for b in range(B):
            n_valid = oracle.n_pages(bt.seq_lens[b], P)
            for h in range(H):
                ref_a[b, h] = oracle.topk_pages(scn[b, h], n_valid, k)
                assert np.array_equal(np_(a1)[b, h, :np_(ac1)[b, h]], ref_a[b, h])
                assert np.array_equal(np_(p1)[b, h, :np_(pc1)[b, h]], oracle.topk_pages(prn[b, h], n_valid, k_spec))
        # with this step's speculative set: M = A \ P_cur, the rest unchanged
        hr = np.random.default_rng(11)
        pcur = np.full((B, H, k_spec), -1, np.int32)
        pcnt = np.zeros((B, H), np.int32)
        for b in range(B):
            n_valid = oracle.n_pages(bt.seq_lens[b], P)
            for h in range(H):
                c = max(0, min(k_spec, n_valid) - 3)
                pcur[b, h, :c] = np.sort(hr.choice(n_valid, c, replace=False))
                pcnt[b, h] = c
        lv3, tr3, pr3 = lvl0.clone(), trd0.clone(), torch.empty(B * H * N, device="cuda")
        a3, ac3 = torch.empty_like(a1), torch.empty_like(ac1)
        p3, pc3 = torch.empty_like(p1), torch.empty_like(pc1)
        m3, mc3 = torch.full((B, H, k), -7, dtype=i32, device="cuda"), torch.empty((B, H), dtype=i32, device="cuda")
        dsa.prr_select(sc, kv.seq_lens, P, k, lv3, tr3, pr3, 0.6, 0.3, 0.25, init, k_spec, a3, ac3, p3, pc3,
                       p_cur=(torch.from_numpy(pcur).cuda(), torch.from_numpy(pcnt).cuda()), m_out=(m3, mc3))
        torch.cuda.synchronize()
        assert torch.equal(a3, a1) and torch.equal(ac3, ac1) and torch.equal(p3, p1) and torch.equal(pr3, pr1)
        for b in range(B):
            for h in range(H):
                ref = oracle.missing_pages(ref_a[b, h], pcur[b, h, :pcnt[b, h]])
                n = int(np_(mc3)[b, h])
                assert n == len(ref) and np.array_equal(np_(m3)[b, h, :n], ref), f"M differs ({b}, {h})"
                assert np.all(np_(m3)[b, h, n:] == -1)


def _prr_run(dsa, sc, lens_t, P, k, k_spec, lvl0, trd0, init, pcur, pcnt, split):
    B, H, N = sc.shape
    i32 = torch.int32
    lv, tr, pr = lvl0.clone(), trd0.clone(), torch.empty(B * H * N, device="cuda")
    a, ac = torch.full((B, H, k), -7, dtype=i32, device="cuda"), torch.empty((B, H), dtype=i32, device="cuda")
    p, pc = torch.full((B, H, k_spec), -7, dtype=i32, device="cuda"), torch.empty((B, H), dtype=i32, device="cuda")
    m, mc = torch.full((B, H, k), -7, dtype=i32, device="cuda"), torch.empty((B, H), dtype=i32, device="cuda")
    dsa.prr_select(sc, lens_t, P, k, lv, tr, pr, 0.6, 0.3, 0.25, init, k_spec, a, ac, p, pc,
                   p_cur=(pcur, pcnt), m_out=(m, mc), split=split)
    torch.cuda.synchronize()
    return {n: np_(t) for n, t in (("a", a), ("ac", ac), ("p", p), ("pc", pc), ("m", m), ("mc", mc), ("lv", lv),
                                   ("tr", tr), ("pr", pr))}


@pytest.mark.parametrize("kind", ["normal", "few_values", "all_equal", "infinities"])
def test_prr_select_split_rows(gpu_lib, kind):
    """Long rows (over 4096 pages) take the split-row selection when a
    workspace is given: 2048-page chunks over many workgroups, the cut from
    the bucket holding the k-th score.  Its A, P, M, counts and EMA state
    equal the one-workgroup path's bit for bit and the oracle's top-k, on
    ragged rows (a partial last chunk, a 1-page row, an empty row, budgets
    above the valid count) and on scores with long runs of ties (few
    distinct values, all equal: the cut then falls among thousands of equal
    keys), and with +-inf scores."""
    dsa = gpu_lib
    print(f"[case] prr_select split rows kind={kind}", flush=True)
    P, N = 16, 20000
    lens = [P * N, P * 12345 + 3, 5, 0]
    B, H = len(lens), 2
    k, k_spec = 1500, 1200
    rng = np.random.default_rng(123)
    if kind == "normal":
        s = rng.standard_normal((B, H, N)).astype(np.float32)
    elif kind == "few_values":
        s = rng.integers(0, 4, (B, H, N)).astype(np.float32)
    elif kind == "all_equal":
        s = np.full((B, H, N), 0.5, np.float32)
    else:
        s = rng.standard_normal((B, H, N)).astype(np.float32)
        s[:, :, ::97] = np.inf
        s[:, :, 5::89] = -np.inf
    sc = torch.from_numpy(s).cuda()
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    lvl = rng.standard_normal(B * H * N).astype(np.float32)
    trd = rng.standard_normal(B * H * N).astype(np.float32)
    if kind == "all_equal":   # equal predictions too
        lvl[:] = 0.25
        trd[:] = 0.0
    lvl0, trd0 = torch.from_numpy(lvl).cuda(), torch.from_numpy(trd).cuda()
    pcur = np.full((B, H, k_spec), -1, np.int32)
    pcnt = np.zeros((B, H), np.int32)
    for b in range(B):
        nv = oracle.n_pages(lens[b], P)
        for h in range(H):
            c = min(k_spec, nv)
            pcur[b, h, :c] = np.sort(rng.choice(nv, c, replace=False))
            pcnt[b, h] = c
    pcur_t, pcnt_t = torch.from_numpy(pcur).cuda(), torch.from_numpy(pcnt).cuda()
    for init in (False, True):
        one = _prr_run(dsa, sc, lens_t, P, k, k_spec, lvl0, trd0, init, pcur_t, pcnt_t, split=False)
        spl = _prr_run(dsa, sc, lens_t, P, k, k_spec, lvl0, trd0, init, pcur_t, pcnt_t, split=True)
        for name in one:
            assert np.array_equal(one[name], spl[name], equal_nan=True), f"{name} differs (init={init})"
        # the EMA state and prediction: the oracle's float32 update, bit for bit
        if init:
            lv_ref, tr_ref, pr_ref = s.reshape(-1), np.zeros_like(trd), s.reshape(-1)
        else:
            lv_ref, tr_ref = oracle.ema_step_f32(s.reshape(-1), lvl, trd, 0.6, 0.3)
            pr_ref = oracle.ema_predict_f32(lv_ref, tr_ref, 0.25)
        assert np.array_equal(spl["lv"], lv_ref) and np.array_equal(spl["tr"], tr_ref)
        assert np.array_equal(spl["pr"], pr_ref)
        prn = pr_ref.astype(np.float64).reshape(B, H, N)
        for b in range(B):
            nv = oracle.n_pages(lens[b], P)
            for h in range(H):
                a = spl["a"][b, h, :spl["ac"][b, h]]
                ra = oracle.topk_pages(s[b, h].astype(np.float64), nv, k)
                assert np.array_equal(a, ra)
                assert np.all(spl["a"][b, h, spl["ac"][b, h]:] == -1)
                p = spl["p"][b, h, :spl["pc"][b, h]]
                assert np.array_equal(p, oracle.topk_pages(prn[b, h], nv, k_spec))
                assert np.all(spl["p"][b, h, spl["pc"][b, h]:] == -1)
                ref = oracle.missing_pages(ra, pcur[b, h, :pcnt[b, h]])
                n = int(spl["mc"][b, h])
                assert n == len(ref) and np.array_equal(spl["m"][b, h, :n], ref)
                assert np.all(spl["m"][b, h, n:] == -1)


@pytest.mark.parametrize("N,lens,k", [(4097, [16 * 4097, 16 * 2049 + 1], 1),      # 3 chunks, the last of 1 page
                                      (4097, [16 * 4097, 16 * 4096], 4097),        # budget = every valid page
                                      (65536, [16 * 65536], 3000)])                # the largest row: 32 chunks
def test_prr_select_split_edges(gpu_lib, N, lens, k):
    """Chunk-count edges of the split-row selection: a last chunk of one
    page, a budget covering every valid page, and the 65536-page maximum;
    bit-equal to the one-workgroup path and to the oracle's top-k."""
    dsa = gpu_lib
    print(f"[case] prr_select split edges N={N} k={k}", flush=True)
    P = 16
    B, H = len(lens), 2
    rng = np.random.default_rng(N + k)
    s = rng.standard_normal((B, H, N)).astype(np.float32)
    sc = torch.from_numpy(s).cuda()
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    lvl = rng.standard_normal(B * H * N).astype(np.float32)
    trd = rng.standard_normal(B * H * N).astype(np.float32)
    lvl0, trd0 = torch.from_numpy(lvl).cuda(), torch.from_numpy(trd).cuda()
    k_spec = k
    pcur = np.full((B, H, k_spec), -1, np.int32)
    pcnt = np.zeros((B, H), np.int32)
    for b in range(B):
        nv = oracle.n_pages(lens[b], P)
        for h in range(H):
            c = min(k_spec, nv) // 2
            pcur[b, h, :c] = np.sort(rng.choice(nv, c, replace=False))
            pcnt[b, h] = c
    pcur_t, pcnt_t = torch.from_numpy(pcur).cuda(), torch.from_numpy(pcnt).cuda()
    one = _prr_run(dsa, sc, lens_t, P, k, k_spec, lvl0, trd0, False, pcur_t, pcnt_t, split=False)
    spl = _prr_run(dsa, sc, lens_t, P, k, k_spec, lvl0, trd0, False, pcur_t, pcnt_t, split=True)
    for name in one:
        assert np.array_equal(one[name], spl[name]), f"{name} differs"
    lv_ref, tr_ref = oracle.ema_step_f32(s.reshape(-1), lvl, trd, 0.6, 0.3)
    prn = oracle.ema_predict_f32(lv_ref, tr_ref, 0.25).astype(np.float64).reshape(B, H, N)
    for b in range(B):
        nv = oracle.n_pages(lens[b], P)
        for h in range(H):
            a = spl["a"][b, h, :spl["ac"][b, h]]
            ra = oracle.topk_pages(s[b, h].astype(np.float64), nv, k)
            assert np.array_equal(a, ra)
            assert np.array_equal(spl["p"][b, h, :spl["pc"][b, h]], oracle.topk_pages(prn[b, h], nv, k_spec))
            ref = oracle.missing_pages(ra, pcur[b, h, :pcnt[b, h]])
            n = int(spl["mc"][b, h])
            assert n == len(ref) and np.array_equal(spl["m"][b, h, :n], ref)
