"""GPU parity: every step of the HIP path, called through the C ABI, against
the fp64 oracle on the same seeded inputs.  Sizes span several tiles and
splits with ragged tails; edge cases: empty sequences, partial pages,
k = 1 / N / > N, exact score ties, streaming heads, every group size."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import (TOL, check_attention, check_psa, check_psa_result, check_selected_attention, check_selection,
                         ids_lists, np_, to_device)

pytestmark = pytest.mark.gpu

RAGGED = [0, 5, 16, 37, 16 * 9 + 3, 16 * 40]


def _banner(msg):
    print(f"[case] {msg}", flush=True)


# ---------------------------------------------------------------- metadata
@pytest.mark.parametrize("dtype,D,P,Pl", [("bf16", 128, 16, 16), ("bf16", 64, 16, 16), ("f32", 64, 16, 16),
                                          ("f32", 128, 32, 16), ("bf16", 128, 64, 16), ("bf16", 128, 64, 32),
                                          ("bf16", 64, 64, 64)])
def test_meta_build(gpu_lib, dtype, D, P, Pl):
    dsa = gpu_lib
    _banner(f"meta {dtype} D={D} P={P} Pl={Pl}")
    bt = wl.random_batch(31, [0, 5, P, P * 3 + 7, P * 9], n_q_heads=2, n_kv_heads=2, head_dim=D, page_size=P,
                         logical_page=Pl, dtype=dtype)
    q, kv, _ = to_device(dsa, bt)
    g = P // Pl
    sentinel = torch.full((kv.num_slots, kv.n_kv_heads, g, 2, D), 7.0, dtype=kv.k.dtype, device="cuda")
    meta = dsa.page_meta_build(kv, Pl, meta=sentinel)
    torch.cuda.synchronize()
    got = np_(meta.float()).astype(np.float64)
    ref, has = oracle.page_meta(bt)
    used = np.zeros(kv.num_slots, bool)
    for b in range(bt.batch):
        used[bt.page_table[b, :oracle.n_pages(bt.seq_lens[b], P)]] = True
    assert np.array_equal(got[has], ref[has])
    for s in np.nonzero(used)[0]:
        assert np.all(got[s][~has[s]] == 0.0)           # empty sub-pages are zeros
    assert np.all(got[~used] == 7.0)                     # untouched slots


def test_meta_build_page_range(gpu_lib):
    """first_page / n_pages rebuild only that range (incremental append)."""
    dsa = gpu_lib
    bt = wl.random_batch(32, [16 * 12 + 5], n_q_heads=2, n_kv_heads=2, head_dim=128)
    q, kv, _ = to_device(dsa, bt)
    meta = torch.full((kv.num_slots, 2, 1, 2, 128), 3.0, dtype=kv.k.dtype, device="cuda")
    dsa.page_meta_build(kv, 16, meta=meta, first_page=4, n_pages=3)
    torch.cuda.synchronize()
    got = np_(meta.float())
    ref, has = oracle.page_meta(bt)
    for j in range(oracle.n_pages(bt.seq_lens[0], 16)):
        s = bt.page_table[0, j]
        if 4 <= j < 7:
            assert np.array_equal(got[s], ref[s])
        else:
            assert np.all(got[s] == 3.0)


# ---------------------------------------------------------------- scores
@pytest.mark.parametrize("dtype,D,P,Pl,G", [("bf16", 128, 16, 16, 1), ("bf16", 128, 16, 16, 4),
                                            ("bf16", 128, 16, 16, 16), ("bf16", 64, 16, 16, 2),
                                            ("f32", 64, 16, 16, 1), ("f32", 128, 16, 16, 8),
                                            ("bf16", 128, 64, 16, 4), ("bf16", 128, 32, 16, 4),
                                            ("f32", 64, 64, 32, 2)])
def test_page_score(gpu_lib, dtype, D, P, Pl, G):
    dsa = gpu_lib
    _banner(f"score {dtype} D={D} P={P} Pl={Pl} G={G}")
    lens = [0, 3, P * 5 + 1, P * 70 + 17, P * 130]
    bt = wl.random_batch(41, lens, n_q_heads=2 * G, n_kv_heads=2, head_dim=D, page_size=P, logical_page=Pl,
                         dtype=dtype, max_pages=135)
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, Pl)
    sc = np_(dsa.page_score(q, kv, meta, Pl))
    ref = oracle.page_scores(bt)
    assert np.array_equal(np.isneginf(sc), np.isneginf(ref))
    fin = np.isfinite(ref)
    err = np.abs(sc[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))
    assert err.max() <= 2e-6, err.max()


def test_page_score_streaming_heads(gpu_lib):
    dsa = gpu_lib
    bt = wl.random_batch(42, [700, 64 * 9], n_q_heads=8, n_kv_heads=4, head_dim=128, page_size=64,
                         logical_page=16, streaming=[0, 1, 1, 0], sink=64, local=128)
    q, kv, st = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, 16)
    sc = np_(dsa.page_score(q, kv, meta, 16, streaming=st))
    ref = oracle.page_scores(bt)
    assert np.all(np.isneginf(sc[:, 1:3]))
    fin = np.isfinite(ref)
    assert np.allclose(sc[fin], ref[fin], rtol=2e-6, atol=2e-6)


# ---------------------------------------------------------------- top-k on identical scores
def _score_rows(rng, B, H, N, kind):
    if kind == "ties":
        s = rng.integers(-3, 4, size=(B, H, N)).astype(np.float32)
        s[s == 0] = np.where(rng.random((s == 0).sum()) < 0.5, -0.0, 0.0)    # -0 and +0 tie
    elif kind == "spread":
        s = (100 + 5 * rng.standard_normal((B, H, N))).astype(np.float32)
    else:  # mixed magnitudes and signs, a few -inf
        s = (rng.standard_normal((B, H, N)) * 10.0 ** rng.integers(-3, 4, size=(B, H, N))).astype(np.float32)
        s[rng.random((B, H, N)) < 0.01] = -np.inf
    return s


@pytest.mark.parametrize("N", [1, 7, 128, 300, 2048, 5000, 32768])
@pytest.mark.parametrize("kind", ["ties", "spread", "mixed"])
def test_topk_exact(gpu_lib, N, kind):
    """Given the same float32 scores, the selection is bit-exact, ties to the
    lower index, for k in {1, N-1, N, N+5, N/16}."""
    dsa = gpu_lib
    rng = np.random.default_rng(N * 7 + len(kind))
    B, H = 2, 3
    s = _score_rows(rng, B, H, N, kind)
    P = 16
    lens = np.array([N * P, max(0, N * P - 37)], np.int32)
    st = torch.from_numpy(s).cuda()
    sl = torch.from_numpy(lens).cuda()
    for k in sorted({1, max(1, N - 1), N, N + 5, max(1, N // 16)}):
        _banner(f"topk N={N} kind={kind} k={k}")
        ids, counts = dsa.page_select_topk(st, sl, P, k)
        ids, counts = np_(ids), np_(counts)
        for b in range(B):
            nv = oracle.n_pages(lens[b], P)
            for h in range(H):
                ref = oracle.topk_pages(s[b, h].astype(np.float64), nv, k)
                assert counts[b, h] == len(ref)
                assert np.array_equal(ids[b, h, :len(ref)], ref), (b, h, k)
                assert np.all(ids[b, h, len(ref):] == -1)


def test_topk_streaming_lists(gpu_lib):
    dsa = gpu_lib
    N, P = 40, 64
    lens = np.array([N * P, 1000, 100, 0], np.int32)
    s = torch.zeros((4, 2, N), dtype=torch.float32, device="cuda")
    st = dsa.Streaming(np.array([1, 0], np.uint8), 128, 256)
    ids, counts = dsa.page_select_topk(s, torch.from_numpy(lens).cuda(), P, 8, streaming=st)
    ids, counts = np_(ids), np_(counts)
    for b in range(4):
        ref = oracle.streaming_pages(lens[b], P, 128, 256)
        assert counts[b, 0] == len(ref) and np.array_equal(ids[b, 0, :len(ref)], ref)
        assert np.all(ids[b, 0, len(ref):] == -1)


# ---------------------------------------------------------------- attention
@pytest.mark.parametrize("dtype,D,P,G", [("bf16", 128, 16, 1), ("bf16", 128, 16, 4), ("bf16", 128, 16, 16),
                                         ("bf16", 64, 16, 2), ("bf16", 128, 64, 4), ("bf16", 128, 32, 8),
                                         ("bf16", 128, 16, 8), ("bf16", 64, 16, 8), ("bf16", 64, 64, 16),
                                         ("f32", 64, 16, 1), ("f32", 128, 16, 4), ("f32", 64, 64, 16)])
def test_sparse_decode_attn(gpu_lib, dtype, D, P, G):
    dsa = gpu_lib
    _banner(f"attn {dtype} D={D} P={P} G={G}")
    lens = [0, 7, P * 3, P * 37 + 5, P * 300 + 1]
    bt = wl.random_batch(51, lens, n_q_heads=2 * G, n_kv_heads=2, head_dim=D, page_size=P, dtype=dtype)
    q, kv, _ = to_device(dsa, bt)
    rng = np.random.default_rng(5)
    stride = 96
    ids = np.full((bt.batch, 2, stride), -1, np.int32)
    counts = np.zeros((bt.batch, 2), np.int32)
    for b in range(bt.batch):
        n = oracle.n_pages(lens[b], P)
        for h in range(2):
            c = min(n, int(rng.integers(0, stride + 1)))
            sel = np.sort(rng.choice(n, size=c, replace=False)) if c else np.zeros(0, int)
            ids[b, h, :c] = sel
            counts[b, h] = c
    O, l, m = dsa.sparse_decode_attn(q, kv, torch.from_numpy(ids).cuda(), torch.from_numpy(counts).cuda())
    rO, rl, rm = oracle.sparse_decode(bt, ids_lists(ids, counts))
    check_attention(dtype, np_(O), np_(l), np_(m), rO, rl, rm, "attn")


def test_attention_all_pages_is_dense(gpu_lib):
    dsa = gpu_lib
    bt = wl.random_batch(52, [16 * 50 + 9, 16 * 3], n_q_heads=8, n_kv_heads=2, head_dim=128)
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv)
    sc = dsa.page_score(q, kv, meta)
    ids, counts = dsa.page_select_topk(sc, kv.seq_lens, 16, 1000)
    O, l, m = dsa.sparse_decode_attn(q, kv, ids, counts)
    rO, rl, rm = oracle.dense_attention(bt)
    check_attention("bf16", np_(O), np_(l), np_(m), rO, rl, rm, "dense")


@pytest.mark.parametrize("G", [2, 8])
def test_attention_streaming_heads(gpu_lib, G):
    dsa = gpu_lib
    bt = wl.random_batch(53, [64 * 20 + 30, 64 * 8, 200], n_q_heads=4 * G, n_kv_heads=4, head_dim=128, page_size=64,
                         logical_page=16, streaming=[1, 0, 0, 1], sink=128, local=256)
    q, kv, st = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, 16)
    sc = dsa.page_score(q, kv, meta, 16, streaming=st)
    ids, counts = dsa.page_select_topk(sc, kv.seq_lens, 64, 8, streaming=st)
    O, l, m = dsa.sparse_decode_attn(q, kv, ids, counts, streaming=st)
    idn, cn = np_(ids), np_(counts)
    ref = oracle.page_scores(bt)
    ref_ids = oracle.select_topk(bt, ref, 8)
    units = [(b, h) for b in range(bt.batch) for h in range(bt.n_kv_heads)]
    for b, h in units:
        if not bt.streaming[h]:
            check_selection(idn[b, h], int(cn[b, h]), ref[b, h], oracle.n_pages(bt.seq_lens[b], 64), 8, f"({b}, {h})")
    check_selected_attention(dsa, bt, q, kv, st, idn, cn, (O, l, m), ref_ids, units, "streaming")
    # streaming heads really see only sink + local tokens
    for b in range(bt.batch):
        for h in (0, 3):
            assert np.array_equal(idn[b, h, :cn[b, h]], ref_ids[b][h])


# ---------------------------------------------------------------- PSA
@pytest.mark.parametrize("thr,mode", [(0.95, 0), (0.95, 1), (0.8, 0), (1.0, 0), (0.0, 0)])
def test_psa_tiny(gpu_lib, thr, mode):
    dsa = gpu_lib
    _banner(f"psa tiny thr={thr} mode={mode}")
    bt = wl.tiny_heavy()
    _psa_check(dsa, bt, thr, mode)


@pytest.mark.parametrize("G,P,D,dtype", [(1, 16, 128, "bf16"), (2, 16, 64, "bf16"), (4, 64, 128, "bf16"),
                                         (1, 16, 64, "f32")])
def test_psa_random(gpu_lib, G, P, D, dtype):
    dsa = gpu_lib
    _banner(f"psa random G={G} P={P} D={D} {dtype}")
    bt = wl.random_batch(61, [0, P * 2 + 3, P * 90 + 7, P * 200], n_q_heads=2 * G, n_kv_heads=2, head_dim=D,
                         page_size=P, dtype=dtype, dup_pages=3)
    for thr, mode in ((0.9, 0), (0.6, 1), (1.0, 0)):
        _psa_check(dsa, bt, thr, mode)


def _psa_check(dsa, bt, thr, mode):
    """The progressive selection takes the oracle's scores (rounded to
    float32) as its input; the oracle ranks and walks the same values."""
    q, kv, _ = to_device(dsa, bt)
    check_psa(dsa, bt, q, kv, oracle.page_scores(bt).astype(np.float32), thr, mode, f"psa thr={thr} mode={mode}")



@pytest.mark.parametrize("G,P,mode", [(1, 16, 0), (4, 16, 1), (2, 64, 0)])
def test_psa_streaming_heads(gpu_lib, G, P, mode):
    """Progressive selection with streaming heads (LServe section 4.1): dense
    heads walk as usual, a streaming head visits its sink and local pages in
    ascending order under the token mask, with no early stop (oracle.psa_unit)."""
    dsa = gpu_lib
    _banner(f"psa streaming G={G} P={P} mode={mode}")
    lens = [P * 300 + 7, P * 40, P * 2 + 1, 0, 5]
    bt = wl.random_batch(313 + G, lens, n_q_heads=4 * G, n_kv_heads=4, head_dim=128, page_size=P,
                         streaming=[0, 1, 1, 0], sink=P + 3, local=3 * P + 2)
    q, kv, st = to_device(dsa, bt)
    s32 = oracle.page_scores(bt).astype(np.float32)
    sc = torch.from_numpy(np.ascontiguousarray(s32)).cuda()
    ids, counts, O, l, m = (np_(x) for x in dsa.page_select_progressive(q, kv, sc, 0.9, mode, float(bt.scale),
                                                                         streaming=st))
    dense = [(b, h) for b in range(bt.batch) for h in (0, 3)]
    check_psa_result(bt, s32, ids, counts, O, l, m, 0.9, mode, f"psa streaming G={G}", dense)
    for b in range(bt.batch):
        for h in (1, 2):
            rid, rn, rO, rl, rm = oracle.psa_unit(bt, b, h, s32[b, h].astype(np.float64), 0.9, mode)
            n = int(counts[b, h])
            assert n == rn and np.array_equal(ids[b, h, :n], rid), f"streaming pages (b={b}, h={h})"
            assert np.all(ids[b, h, n:] == -1)
            sl = slice(h * G, (h + 1) * G)
            check_attention("bf16", O[b, sl], l[b, sl], m[b, sl], rO, rl, rm, f"streaming (b={b}, h={h})")


@pytest.mark.parametrize("G,P", [(4, 16), (16, 16)])
def test_repair_streaming_heads(gpu_lib, G, P):
    """Repair with streaming heads: spec over P and repair over A \\ P, both
    under the token mask of a streaming head, equal attention over P u A
    with that mask (compacted M and P-filtered forms)."""
    dsa = gpu_lib
    _banner(f"repair streaming G={G} P={P}")
    lens = [P * 150 + 3, P * 64, P * 10]
    bt = wl.random_batch(75, lens, n_q_heads=2 * G, n_kv_heads=2, head_dim=128, page_size=P,
                         streaming=[1, 0], sink=P + 5, local=5 * P)
    q, kv, st = to_device(dsa, bt)
    rng = np.random.default_rng(21)
    stride = 48
    A = np.full((3, 2, stride), -1, np.int32)
    Pp = np.full((3, 2, stride), -1, np.int32)
    ac = np.zeros((3, 2), np.int32)
    pc = np.zeros((3, 2), np.int32)
    for b in range(3):
        n = oracle.n_pages(lens[b], P)
        for h in range(2):
            a = np.sort(rng.choice(n, size=min(n, 30), replace=False))
            p = np.sort(np.concatenate([a[:12], rng.choice(np.setdiff1d(np.arange(n), a), size=min(6, n - len(a)),
                                                           replace=False)]))
            A[b, h, :len(a)], ac[b, h] = a, len(a)
            Pp[b, h, :len(p)], pc[b, h] = p, len(p)
    t = lambda x: torch.from_numpy(x).cuda()
    union = [[np.array(sorted(set(A[b, h, :ac[b, h]]) | set(Pp[b, h, :pc[b, h]])), np.int64) for h in range(2)]
             for b in range(3)]
    rO, rl, rm = oracle.sparse_decode(bt, union)
    # P filtered inside the call
    O, l, m = dsa.sparse_decode_attn(q, kv, t(Pp), t(pc), streaming=st)
    dsa.attn_repair(q, kv, t(A), t(ac), t(Pp), t(pc), O, l, m, streaming=st)
    check_attention("bf16", np_(O), np_(l), np_(m), rO, rl, rm, "repair streaming (filtered)")
    # M compacted by the caller
    M = np.full((3, 2, stride), -1, np.int32)
    mc = np.zeros((3, 2), np.int32)
    for b in range(3):
        for h in range(2):
            mm = np.setdiff1d(A[b, h, :ac[b, h]], Pp[b, h, :pc[b, h]])
            M[b, h, :len(mm)], mc[b, h] = mm, len(mm)
    O, l, m = dsa.sparse_decode_attn(q, kv, t(Pp), t(pc), streaming=st)
    dsa.attn_repair(q, kv, t(M), t(mc), None, None, O, l, m, streaming=st)
    check_attention("bf16", np_(O), np_(l), np_(m), rO, rl, rm, "repair streaming (compacted)")

# ---------------------------------------------------------------- repair
@pytest.mark.parametrize("G,P", [(4, 16), (16, 16), (2, 64)])
def test_repair(gpu_lib, G, P):
    """spec over P + repair over A\\P == attention over P u A; several
    overlaps including P inside A, P disjoint from A, empty P, empty A."""
    dsa = gpu_lib
    _banner(f"repair G={G} P={P}")
    lens = [P * 150 + 3, P * 64, P * 10]
    bt = wl.random_batch(71, lens, n_q_heads=2 * G, n_kv_heads=2, head_dim=128, page_size=P)
    q, kv, _ = to_device(dsa, bt)
    rng = np.random.default_rng(9)
    stride = 48
    A = np.full((3, 2, stride), -1, np.int32)
    Pp = np.full((3, 2, stride), -1, np.int32)
    ac = np.zeros((3, 2), np.int32)
    pc = np.zeros((3, 2), np.int32)
    modes = ["overlap", "subset", "disjoint", "emptyP", "emptyA", "same"]
    for b in range(3):
        n = oracle.n_pages(lens[b], P)
        for h in range(2):
            mode = modes[(2 * b + h) % len(modes)]
            a = np.sort(rng.choice(n, size=min(n, 30), replace=False))
            if mode == "overlap":
                p = np.sort(np.concatenate([a[:20], rng.choice(np.setdiff1d(np.arange(n), a), size=min(8, n - len(a)), replace=False)]))
            elif mode == "subset":
                p = a[::2]
            elif mode == "disjoint":
                p = np.sort(rng.choice(np.setdiff1d(np.arange(n), a), size=min(10, n - len(a)), replace=False))
            elif mode == "emptyP":
                p = np.zeros(0, int)
            elif mode == "emptyA":
                p, a = a[:10], np.zeros(0, int)
            else:
                p = a.copy()
            A[b, h, :len(a)], ac[b, h] = a, len(a)
            Pp[b, h, :len(p)], pc[b, h] = p, len(p)
    t = lambda x: torch.from_numpy(x).cuda()
    O, l, m = dsa.sparse_decode_attn(q, kv, t(Pp), t(pc))
    dsa.attn_repair(q, kv, t(A), t(ac), t(Pp), t(pc), O, l, m)
    union = [[np.array(sorted(set(A[b, h, :ac[b, h]]) | set(Pp[b, h, :pc[b, h]])), np.int64) for h in range(2)]
             for b in range(3)]
    rO, rl, rm = oracle.sparse_decode(bt, union)
    check_attention("bf16", np_(O), np_(l), np_(m), rO, rl, rm, "repair")



@pytest.mark.parametrize("G,P", [(4, 16), (16, 16), (8, 64)])
def test_repair_compacted(gpu_lib, G, P):
    """Repair given M = A \\ P already compacted (no P argument; the PRR
    step's form, run with short splits): spec over P + repair over M ==
    attention over P u A.  M counts span empty, one page, ragged lengths
    and the whole id row."""
    dsa = gpu_lib
    _banner(f"repair compacted G={G} P={P}")
    lens = [P * 150 + 3, P * 64, P * 10]
    bt = wl.random_batch(73, lens, n_q_heads=2 * G, n_kv_heads=2, head_dim=128, page_size=P)
    q, kv, _ = to_device(dsa, bt)
    rng = np.random.default_rng(11)
    stride = 48
    M = np.full((3, 2, stride), -1, np.int32)
    Pp = np.full((3, 2, stride), -1, np.int32)
    mc = np.zeros((3, 2), np.int32)
    pc = np.zeros((3, 2), np.int32)
    m_sizes = [0, 1, 5, 17, 33, stride]
    for b in range(3):
        n = oracle.n_pages(lens[b], P)
        for h in range(2):
            want = min(m_sizes[(2 * b + h) % len(m_sizes)], n)
            perm = rng.permutation(n)
            m_ = np.sort(perm[:want])
            p_ = np.sort(perm[want:want + min(stride, n - want, 20)])
            M[b, h, :len(m_)], mc[b, h] = m_, len(m_)
            Pp[b, h, :len(p_)], pc[b, h] = p_, len(p_)
    t = lambda x: torch.from_numpy(x).cuda()
    O, l, m = dsa.sparse_decode_attn(q, kv, t(Pp), t(pc))
    dsa.attn_repair(q, kv, t(M), t(mc), None, None, O, l, m)
    union = [[np.array(sorted(set(M[b, h, :mc[b, h]]) | set(Pp[b, h, :pc[b, h]])), np.int64) for h in range(2)]
             for b in range(3)]
    rO, rl, rm = oracle.sparse_decode(bt, union)
    check_attention("bf16", np_(O), np_(l), np_(m), rO, rl, rm, "repair compacted")

# ---------------------------------------------------------------- EMA
@pytest.mark.parametrize("n", [1, 3, 1000, 65539])
def test_ema(gpu_lib, n):
    dsa = gpu_lib
    rng = np.random.default_rng(n)
    a, b_, g = 0.6, 0.3, 0.25
    is0 = rng.standard_normal(n).astype(np.float32) * 10
    lv = torch.empty(n, device="cuda")
    tr = torch.empty(n, device="cuda")
    pr = torch.empty(n, device="cuda")
    dsa.ema_predict_update(torch.from_numpy(is0).cuda(), lv, tr, pr, a, b_, g, init=True)
    rl, rt = is0.astype(np.float64), np.zeros(n)
    assert np.array_equal(np_(pr), is0)
    for step in range(5):
        x = (is0 + rng.standard_normal(n) * 3).astype(np.float32)
        dsa.ema_predict_update(torch.from_numpy(x).cuda(), lv, tr, pr, a, b_, g)
        rl, rt = oracle.ema_update(x, rl, rt, a, b_)
        rp = oracle.ema_predict(rl, rt, g)
        assert np.allclose(np_(lv), rl, rtol=1e-6, atol=1e-5)
        assert np.allclose(np_(tr), rt, rtol=1e-6, atol=1e-5)
        assert np.allclose(np_(pr), rp, rtol=1e-6, atol=1e-5)
    pr2 = torch.empty(n, device="cuda")
    dsa.ema_predict_update(None, lv, tr, pr2, a, b_, g)
    assert np.allclose(np_(pr2), oracle.ema_predict(rl, rt, g), rtol=1e-6, atol=1e-5)


# ---------------------------------------------------------------- HIP graph replay
def test_graph_replay_matches_eager(gpu_lib):
    """The decode step captured in a HIP graph gives the eager result on every
    replay, with eager work and synchronisations between replays."""
    dsa = gpu_lib
    bt = wl.quest_gqa(seed=3, seq_len=16 * 300 + 5, n_q_heads=8, n_kv_heads=2)
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv)
    B, Hkv, N = kv.batch, kv.n_kv_heads, kv.max_pages
    sc = torch.empty((B, Hkv, N), device="cuda")
    ids = torch.empty((B, Hkv, 40), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    O = torch.empty((B, 8, 128), device="cuda")
    l = torch.empty((B, 8), device="cuda")
    m = torch.empty((B, 8), device="cuda")
    ws = torch.zeros(dsa.workspace_bytes(dsa.OP_SPARSE_DECODE_ATTN, kv, 8, 40), dtype=torch.uint8, device="cuda")

    def step():
        dsa.page_score(q, kv, meta, scores=sc)
        dsa.page_select_topk(sc, kv.seq_lens, 16, 40, ids=ids, counts=cnt)
        dsa.sparse_decode_attn(q, kv, ids, cnt, out=(O, l, m), ws=ws)

    step()
    torch.cuda.synchronize()
    ref = [np_(x).copy() for x in (sc, ids, cnt, O, l, m)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for x in (sc, O, l, m):
            x.fill_(float("nan"))
        ids.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        got = [np_(x) for x in (sc, ids, cnt, O, l, m)]
        for a_, b_ in zip(got, ref):
            assert np.array_equal(a_, b_), f"replay {rep} differs"
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()   # eager work between replays
