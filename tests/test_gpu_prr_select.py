"""GPU parity of dsa_prr_select (A^t, the EMA update and P^{t+1} in one
launch) against the calls it stands for: dsa_page_select_topk on the
scores, dsa_ema_predict_update, dsa_page_select_topk on the prediction.
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
    meta = dsa.page_meta_build(kv)
    B, H, N = bt.batch, bt.n_kv_heads, max_pages
    rng = torch.Generator(device="cuda").manual_seed(5)
    lvl0 = torch.randn(B * H * N, device="cuda", generator=rng)
    trd0 = torch.randn(B * H * N, device="cuda", generator=rng)
    i32 = torch.int32
    for init in (True, False):
        sc = dsa.page_score(q, kv, meta)
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
        scn, prn = np_(sc).astype(np.float64), np_(pr1).astype(np.float64).reshape(B, H, N)
        for b in range(B):
            n_valid = oracle.n_pages(bt.seq_lens[b], P)
            for h in range(H):
                assert np.array_equal(np_(a1)[b, h, :np_(ac1)[b, h]], oracle.topk_pages(scn[b, h], n_valid, k))
                assert np.array_equal(np_(p1)[b, h, :np_(pc1)[b, h]], oracle.topk_pages(prn[b, h], n_valid, k_spec))
