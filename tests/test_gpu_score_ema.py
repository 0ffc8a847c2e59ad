"""GPU parity of dsa_page_score_ema (page scores with PRR's EMA update in
the same launch) against the two calls it stands for, dsa_page_score and
dsa_ema_predict_update, bit for bit (the same float operations); and of
dsa_prr_select given the already-updated prediction (level = trend = NULL)
against the call that updates it itself, on both selection paths.  The
score and EMA arithmetic of the separate calls is pinned to the oracle in
test_gpu_parity.py."""
import numpy as np
import pytest
import torch

import workloads as wl
from parity_util import np_, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,D,P,Pl,G,streaming", [("bf16", 128, 16, 16, 16, None), ("bf16", 128, 16, 16, 4, None),
                                                      ("f32", 64, 16, 16, 1, None),
                                                      ("bf16", 128, 64, 16, 2, [0, 1, 1, 0])])
@pytest.mark.parametrize("init", [False, True])
def test_page_score_ema_matches_two_calls(gpu_lib, dtype, D, P, Pl, G, streaming, init):
    dsa = gpu_lib
    print(f"[case] score_ema {dtype} D={D} P={P} Pl={Pl} G={G} streaming={streaming} init={init}", flush=True)
    H = 4 if streaming else 2
    lens = [0, 3, P * 5 + 1, P * 70 + 17, P * 130]
    bt = wl.random_batch(43, lens, n_q_heads=H * G, n_kv_heads=H, head_dim=D, page_size=P, logical_page=Pl,
                         dtype=dtype, max_pages=135, streaming=streaming, sink=P, local=2 * P)
    q, kv, st = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, Pl)
    B, N = bt.batch, bt.max_pages
    rng = np.random.default_rng(7)
    lvl = torch.from_numpy(rng.standard_normal(B * H * N).astype(np.float32)).cuda()
    trd = torch.from_numpy(rng.standard_normal(B * H * N).astype(np.float32)).cuda()
    lv1, tr1, pr1 = lvl.clone(), trd.clone(), torch.empty_like(lvl)
    sc1 = dsa.page_score_ema(q, kv, meta, lv1, tr1, pr1, 0.6, 0.3, 0.25, init=init, logical_page=Pl, streaming=st)
    sc2 = dsa.page_score(q, kv, meta, Pl, streaming=st)
    lv2, tr2, pr2 = lvl.clone(), trd.clone(), torch.empty_like(lvl)
    dsa.ema_predict_update(sc2, lv2, tr2, pr2, 0.6, 0.3, 0.25, init=init)
    torch.cuda.synchronize()
    for x, y, what in ((sc1, sc2, "scores"), (lv1, lv2, "level"), (tr1, tr2, "trend"), (pr1, pr2, "pred")):
        assert np.array_equal(np_(x), np_(y), equal_nan=True), f"{what} differs"


@pytest.mark.parametrize("N,split", [(3000, False), (20000, False), (20000, True)])
def test_prr_select_with_updated_prediction(gpu_lib, N, split):
    dsa = gpu_lib
    print(f"[case] prr_select level=NULL N={N} split={split}", flush=True)
    P, k = 16, 700
    lens = [P * N, P * (N // 3) + 9]
    B, H = len(lens), 2
    rng = np.random.default_rng(19)
    sc = torch.from_numpy(rng.standard_normal((B, H, N)).astype(np.float32)).cuda()
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    lvl = torch.from_numpy(rng.standard_normal(B * H * N).astype(np.float32)).cuda()
    trd = torch.from_numpy(rng.standard_normal(B * H * N).astype(np.float32)).cuda()
    pcur = torch.from_numpy(np.stack([np.stack([np.sort(rng.choice(N // 3, k, replace=False))
                                                for _ in range(H)]) for _ in range(B)]).astype(np.int32)).cuda()
    pcnt = torch.full((B, H), k, dtype=torch.int32, device="cuda")
    i32 = torch.int32
    outs = []
    for fused in (False, True):
        lv, tr, pr = lvl.clone(), trd.clone(), torch.empty(B * H * N, device="cuda")
        if fused:   # the prediction is updated first, as page_score_ema leaves it
            dsa.ema_predict_update(sc, lv, tr, pr, 0.6, 0.3, 0.25)
        a, ac = torch.empty((B, H, k), dtype=i32, device="cuda"), torch.empty((B, H), dtype=i32, device="cuda")
        p, pc = torch.empty((B, H, k), dtype=i32, device="cuda"), torch.empty((B, H), dtype=i32, device="cuda")
        m, mc = torch.empty((B, H, k), dtype=i32, device="cuda"), torch.empty((B, H), dtype=i32, device="cuda")
        dsa.prr_select(sc, lens_t, P, k, None if fused else lv, None if fused else tr, pr, 0.6, 0.3, 0.25, False, k,
                       a, ac, p, pc, p_cur=(pcur, pcnt), m_out=(m, mc), split=split)
        torch.cuda.synchronize()
        outs.append([np_(t) for t in (a, ac, p, pc, m, mc, lv, tr, pr)])
    for x, y, what in zip(outs[0], outs[1], ("A", "A counts", "P", "P counts", "M", "M counts", "level", "trend",
                                              "pred")):
        assert np.array_equal(x, y), f"{what} differs"
