"""Pins for the oracle: each test ties an oracle function to something other
than itself -- a closed form, an invariant that fixes the result uniquely,
brute-force enumeration, a textbook/library routine, or a hand-built input
whose answer is worked out by hand.  CPU only."""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads as wl
from workloads import Batch


# ---------------------------------------------------------------- helpers
def token_major(batch, pool, b, h):
    """Token-major [L][D] values of (b, h), by direct pool indexing."""
    L, P = int(batch.seq_lens[b]), batch.page_size
    t = np.arange(L)
    slots = batch.page_table[b][t // P]
    vals = pool[slots, h, t % P]
    if batch.dtype == "bf16":
        return wl.from_bf16_bits(vals).astype(np.float64)
    return vals.astype(np.float64)


def textbook(batch, b, hq, mask=None):
    """softmax(scale * K q) V over the (masked) valid tokens, via scipy."""
    h = hq // batch.group
    K = token_major(batch, batch.k, b, h)
    V = token_major(batch, batch.v, b, h)
    if mask is not None:
        K, V = K[mask], V[mask]
    q = (wl.from_bf16_bits(batch.q[b, hq]) if batch.dtype == "bf16" else batch.q[b, hq]).astype(np.float64)
    s = float(batch.scale) * (K @ q)
    return softmax(s) @ V, s


def hand_batch(keys_per_page, q, page_size, values=None, dtype="f32", logical_page=None):
    """One sequence, one head, pages given explicitly (identity page table)."""
    keys_per_page = [np.asarray(k, np.float32) for k in keys_per_page]
    D = len(q)
    N = len(keys_per_page)
    L = sum(len(k) for k in keys_per_page[:-1]) + len(keys_per_page[-1])
    k = np.zeros((N, 1, page_size, D), np.float32)
    v = np.zeros((N, 1, page_size, D), np.float32)
    rng = np.random.default_rng(0)
    for j, kk in enumerate(keys_per_page):
        k[j, 0, :len(kk)] = kk
        v[j, 0, :len(kk)] = rng.standard_normal((len(kk), D)) if values is None else values[j]
    pt = np.arange(N, dtype=np.int32)[None, :]
    return Batch("hand", dtype, 1, 1, 1, D, page_size, logical_page or page_size, N,
                 np.asarray(q, np.float32)[None, None, :], k, v, pt, np.array([L], np.int32))


# ---------------------------------------------------------------- step 1: metadata
@pytest.mark.parametrize("dtype,P,Pl", [("bf16", 16, 16), ("bf16", 64, 16), ("f32", 16, 8)])
def test_meta_is_the_attained_per_channel_box(dtype, P, Pl):
    """kmin <= k_t <= kmax for every valid token, and every bound is attained
    by some valid token: that characterises per-channel min/max uniquely.
    Padding rows of the last page hold 1e3-scale garbage, which would break
    attainment or the bound if it leaked in."""
    bt = wl.random_batch(3, [37, 130, 5], n_q_heads=2, n_kv_heads=2, head_dim=16, page_size=P,
                         logical_page=Pl, dtype=dtype)
    meta, has = oracle.page_meta(bt)
    g = P // Pl
    for b in range(bt.batch):
        L = int(bt.seq_lens[b])
        for h in range(bt.n_kv_heads):
            K = token_major(bt, bt.k, b, h)
            for j in range(oracle.n_pages(L, P)):
                slot = bt.page_table[b][j]
                for s in range(g):
                    lo, hi = j * P + s * Pl, min(j * P + (s + 1) * Pl, L)
                    assert has[slot, h, s] == (hi > lo)
                    if hi <= lo:
                        continue
                    sub = K[lo:hi]
                    kmin, kmax = meta[slot, h, s, 0], meta[slot, h, s, 1]
                    assert np.all(sub >= kmin) and np.all(sub <= kmax)
                    assert np.all((sub == kmin).any(axis=0)) and np.all((sub == kmax).any(axis=0))


# ---------------------------------------------------------------- decode-time append
def free_slots(bt):
    return sorted(set(range(bt.num_slots)) - set(int(x) for x in bt.page_table[bt.page_table >= 0]))


def stored(x, dtype):
    return (wl.from_bf16_bits(x) if dtype == "bf16" else np.asarray(x, np.float32)).astype(np.float64)


@pytest.mark.parametrize("dtype,P,Pl", [("bf16", 16, 16), ("bf16", 64, 16), ("f32", 32, 16)])
def test_append_writes_the_next_token_and_nothing_else(dtype, P, Pl):
    """By direct pool indexing: after one append every sequence reads back
    its old tokens followed by the new row (in both pools), and exactly one
    row per (sequence, KV head) of each pool changed.  Sequence 1's new token
    opens page 1, whose slot the test allocates first."""
    bt = wl.random_batch(11, [5, P, 3 * P - 1], n_q_heads=2, n_kv_heads=2, head_dim=16, page_size=P,
                         logical_page=Pl, dtype=dtype, max_pages=4, spare_slots=4)
    bt.page_table[1][1] = free_slots(bt)[0]
    kn, vn = wl.append_stream(5, 3, 2, 16, 1, dtype)
    nb, done = oracle.append_token(bt, kn[0], vn[0])
    assert done.all() and list(nb.seq_lens) == [6, P + 1, 3 * P]
    for b in range(3):
        for h in range(2):
            for pool0, pool1, new in ((bt.k, nb.k, kn), (bt.v, nb.v, vn)):
                before, after = token_major(bt, pool0, b, h), token_major(nb, pool1, b, h)
                np.testing.assert_array_equal(after[:-1], before)
                np.testing.assert_array_equal(after[-1], stored(new[0, b, h], dtype))
    for pool0, pool1 in ((bt.k, nb.k), (bt.v, nb.v)):
        assert int((pool0 != pool1).any(axis=-1).sum()) == 3 * 2


def test_append_skips_full_and_unallocated_sequences():
    """A sequence at max_pages * P tokens and one whose next page has no slot
    (page-table entry -1) are left exactly as they were."""
    bt = wl.random_batch(12, [64, 32, 7], n_q_heads=2, n_kv_heads=2, head_dim=16, page_size=16,
                         dtype="f32", max_pages=4, spare_slots=2)
    kn, vn = wl.append_stream(6, 3, 2, 16, 1, "f32")
    nb, done = oracle.append_token(bt, kn[0], vn[0])
    assert list(done) == [False, False, True]
    assert list(nb.seq_lens) == [64, 32, 8]
    for b in (0, 1):
        for h in range(2):
            np.testing.assert_array_equal(token_major(nb, nb.k, b, h), token_major(bt, bt.k, b, h))
    assert int((nb.k != bt.k).any(axis=-1).sum()) == 2


@pytest.mark.parametrize("dtype,P,Pl", [("bf16", 64, 16), ("f32", 16, 16)])
def test_append_meta_is_the_running_min_max(dtype, P, Pl):
    """Metadata of the grown cache, by the per-channel identities of min and
    max: in the new token's logical page, a token that opens it gives
    kmin = kmax = token, any other gives kmin' = min(kmin, token) and
    kmax' = max(kmax, token); every other logical page keeps its box.  The
    appends walk across logical-page and page boundaries."""
    bt = wl.random_batch(13, [1, Pl - 1, P - 1], n_q_heads=2, n_kv_heads=2, head_dim=16, page_size=P,
                         logical_page=Pl, dtype=dtype, max_pages=3, spare_slots=6)
    spare = free_slots(bt)
    kn, vn = wl.append_stream(7, 3, 2, 16, Pl + 2, dtype)
    for t in range(Pl + 2):
        for b in range(3):
            L = int(bt.seq_lens[b])
            if L % P == 0 and bt.page_table[b][L // P] < 0:
                bt.page_table[b][L // P] = spare.pop()
        m0, h0 = oracle.page_meta(bt)
        nb, done = oracle.append_token(bt, kn[t], vn[t])
        assert done.all()
        m1, h1 = oracle.page_meta(nb)
        touched = set()
        for b in range(3):
            p = int(bt.seq_lens[b])
            slot, s = int(bt.page_table[b][p // P]), (p % P) // Pl
            touched.add((slot, s))
            for h in range(2):
                x = stored(kn[t, b, h], dtype)
                assert h1[slot, h, s]
                if p % Pl == 0:
                    assert not h0[slot, h, s]
                    np.testing.assert_array_equal(m1[slot, h, s, 0], x)
                    np.testing.assert_array_equal(m1[slot, h, s, 1], x)
                else:
                    np.testing.assert_array_equal(m1[slot, h, s, 0], np.minimum(m0[slot, h, s, 0], x))
                    np.testing.assert_array_equal(m1[slot, h, s, 1], np.maximum(m0[slot, h, s, 1], x))
        for slot in range(bt.num_slots):
            for s in range(P // Pl):
                if (slot, s) not in touched:
                    assert (h0[slot, :, s] == h1[slot, :, s]).all()
                    np.testing.assert_array_equal(m0[slot, :, s][h0[slot, :, s]], m1[slot, :, s][h1[slot, :, s]])
        bt = nb


# ---------------------------------------------------------------- steps 2-4: scores
def test_criticality_is_max_over_box_corners():
    """max_i-separable bound == maximum of q.x over the 2^D corners of the box
    [kmin, kmax] (a linear function peaks at a corner); brute force, D=6."""
    rng = np.random.default_rng(7)
    D = 6
    for _ in range(50):
        q = rng.standard_normal(D)
        a, b2 = rng.standard_normal(D), rng.standard_normal(D)
        kmin, kmax = np.minimum(a, b2), np.maximum(a, b2)
        best = max(sum(q[i] * (kmax[i] if c[i] else kmin[i]) for i in range(D))
                   for c in itertools.product([0, 1], repeat=D))
        assert oracle.criticality(q, kmin, kmax) == pytest.approx(best, rel=1e-12, abs=1e-12)


def test_score_upper_bounds_every_key_and_is_tight_for_constant_pages():
    bt = wl.random_batch(5, [300], n_q_heads=1, n_kv_heads=1, head_dim=32, page_size=16, dtype="f32")
    S = oracle.page_scores(bt)
    K = token_major(bt, bt.k, 0, 0)
    q = bt.q[0, 0].astype(np.float64)
    for j in range(oracle.n_pages(300, 16)):
        dots = K[j * 16:(j + 1) * 16] @ q
        assert S[0, 0, j] >= dots.max() - 1e-12
    # pages of identical keys: the bound is attained exactly
    key = np.random.default_rng(1).standard_normal(8)
    qq = np.random.default_rng(2).standard_normal(8)
    hb = hand_batch([np.tile(key, (16, 1)), np.tile(-key, (16, 1)), key[None, :]], qq, 16)
    S = oracle.page_scores(hb)
    kf = key.astype(np.float32).astype(np.float64)
    qf = qq.astype(np.float32).astype(np.float64)
    assert S[0, 0, :3] == pytest.approx([kf @ qf, -(kf @ qf), kf @ qf], rel=1e-12)


def test_group_query_is_the_mean():
    """Two identical q heads in a group score exactly like one head (a sum
    would double the score); opposite heads cancel to zero."""
    bt = wl.random_batch(9, [64], n_q_heads=1, n_kv_heads=1, head_dim=16, dtype="f32")
    S1 = oracle.page_scores(bt)
    q2 = np.repeat(bt.q, 2, axis=1)
    bt2 = Batch(**{**bt.__dict__, "q": q2, "n_q_heads": 2})
    assert np.array_equal(oracle.page_scores(bt2), S1)
    q3 = np.concatenate([bt.q, -bt.q], axis=1)
    bt3 = Batch(**{**bt.__dict__, "q": q3, "n_q_heads": 2})
    assert np.all(oracle.page_scores(bt3)[0, 0, :4] == 0.0)


def test_physical_score_is_max_of_logical_pages():
    """The same token stream paged as 64/16 (g=4) and as 16/16 (g=1): the
    hierarchical physical score equals the max of the 4 small-page scores."""
    big = wl.random_batch(11, [64 * 9 + 20], n_q_heads=4, n_kv_heads=2, head_dim=16, page_size=64,
                          logical_page=16, dtype="bf16")
    S64 = oracle.page_scores(big)
    L = int(big.seq_lens[0])
    small_k = np.zeros((oracle.n_pages(L, 16), 2, 16, 16), np.uint16)
    for h in range(2):
        for t in range(L):
            small_k[t // 16, h, t % 16] = big.k[big.page_table[0][t // 64], h, t % 64]
    small = Batch(**{**big.__dict__, "k": small_k, "v": small_k, "page_size": 16, "logical_page": 16,
                     "max_pages": small_k.shape[0],
                     "page_table": np.arange(small_k.shape[0], dtype=np.int32)[None, :]})
    S16 = oracle.page_scores(small)
    for h in range(2):
        for j in range(oracle.n_pages(L, 64)):
            assert S64[0, h, j] == S16[0, h, 4 * j:4 * j + 4].max()
    assert np.all(np.isneginf(S64[0, :, oracle.n_pages(L, 64):]))


def test_streaming_heads_score_minus_inf():
    bt = wl.random_batch(2, [100], n_q_heads=4, n_kv_heads=2, head_dim=16, streaming=[1, 0],
                         sink=4, local=8)
    S = oracle.page_scores(bt)
    assert np.all(np.isneginf(S[0, 0]))
    assert np.all(np.isfinite(S[0, 1, :oracle.n_pages(100, 16)]))


# ---------------------------------------------------------------- step 5: top-k
def test_topk_matches_subset_enumeration():
    """Top-k == the k-subset with the largest total score; among equal totals
    (exact ties) the lexicographically smallest index set."""
    rng = np.random.default_rng(3)
    for trial in range(200):
        N = int(rng.integers(1, 10))
        s = rng.integers(0, 4, size=N).astype(float)   # many exact ties
        k = int(rng.integers(1, N + 2))
        kk = min(k, N)
        best = max(itertools.combinations(range(N), kk), key=lambda c: (sum(s[list(c)]), [-i for i in c]))
        assert list(oracle.topk_pages(s, N, k)) == list(best), (s, k)


def test_topk_k_at_least_n_gives_all_and_ranks_ties_by_index():
    s = np.array([1.0, 5.0, 5.0, -2.0, 5.0])
    assert list(oracle.topk_pages(s, 5, 9)) == [0, 1, 2, 3, 4]
    assert list(oracle.rank_pages(s, 5)) == [1, 2, 4, 0, 3]
    assert list(oracle.topk_pages(s, 5, 2)) == [1, 2]
    assert list(oracle.topk_pages(s, 3, 9)) == [0, 1, 2]      # only valid pages


def test_streaming_pages():
    assert list(oracle.streaming_pages(1000, 64, 128, 256)) == [0, 1, 11, 12, 13, 14, 15]
    assert list(oracle.streaming_pages(100, 64, 128, 256)) == [0, 1]
    assert list(oracle.streaming_pages(1024, 64, 0, 64)) == [15]


# ---------------------------------------------------------------- step 7: attention
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_pages_equals_textbook_softmax(dtype):
    """k >= N reaches dense attention; checked against scipy softmax over the
    token-major keys rebuilt by direct pool indexing."""
    bt = wl.random_batch(4, [77, 160], n_q_heads=4, n_kv_heads=2, head_dim=32, dtype=dtype)
    S = oracle.page_scores(bt)
    ids = oracle.select_topk(bt, S, 10_000)
    O, l, m = oracle.sparse_decode(bt, ids)
    for b in range(2):
        for hq in range(4):
            ref, s = textbook(bt, b, hq)
            assert np.allclose(O[b, hq], ref, atol=1e-12)
            assert m[b, hq] == pytest.approx(s.max(), abs=1e-12)
            assert l[b, hq] == pytest.approx(np.exp(s - s.max()).sum(), rel=1e-12)


def test_streaming_head_is_masked_dense_attention():
    bt = wl.random_batch(8, [200], n_q_heads=2, n_kv_heads=2, head_dim=16, streaming=[1, 0],
                         sink=5, local=40)
    ids = oracle.select_topk(bt, oracle.page_scores(bt), 10_000)
    O, l, m = oracle.sparse_decode(bt, ids)
    t = np.arange(200)
    ref, _ = textbook(bt, 0, 0, mask=(t < 5) | (t >= 160))
    assert np.allclose(O[0, 0], ref, atol=1e-12)
    ref1, _ = textbook(bt, 0, 1)
    assert np.allclose(O[0, 1], ref1, atol=1e-12)


def test_psa_streaming_head_is_masked_dense_attention():
    """PSA on a batch with a streaming head: the streaming head visits its
    sink and local pages in ascending order, never stops, and its result is
    softmax attention over the sink and local tokens only (textbook, scipy);
    the dense head still takes the progressive walk."""
    bt = wl.random_batch(9, [300], n_q_heads=2, n_kv_heads=2, head_dim=16, page_size=16, streaming=[1, 0],
                         sink=20, local=70)
    sc = oracle.page_scores(bt)
    ids, n, O, l, m = oracle.psa_unit(bt, 0, 0, sc[0, 0], 0.5)
    assert list(ids) == [0, 1, 14, 15, 16, 17, 18] and n == 7   # tokens [0, 20) and [230, 300)
    t = np.arange(300)
    ref, _ = textbook(bt, 0, 0, mask=(t < 20) | (t >= 230))
    assert np.allclose(O[0], ref, atol=1e-12)
    d = oracle.psa_unit(bt, 0, 1, sc[0, 1], 0.5)
    p = oracle.psa_progressive(bt, 0, 1, sc[0, 1], 0.5)
    assert np.array_equal(d[0], p[0]) and d[1] == p[1] and np.allclose(d[2], p[2])


def test_empty_set_is_merge_identity():
    O, l, m = oracle.attention(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 0.5)
    assert l == 0.0 and m == -math.inf and np.all(O == 0)
    x = (np.arange(4.0), 2.0, 1.5)
    for a, b in ((x, (O, l, m)), ((O, l, m), x)):
        r = oracle.merge(a, b)
        assert np.allclose(r[0], x[0]) and r[1] == pytest.approx(2.0) and r[2] == 1.5


# ---------------------------------------------------------------- merge / repair
def test_merge_of_disjoint_parts_is_attention_of_union_and_commutes():
    rng = np.random.default_rng(12)
    q = rng.standard_normal(16)
    K, V = rng.standard_normal((40, 16)) * 2, rng.standard_normal((40, 16))
    parts = [slice(0, 7), slice(7, 8), slice(8, 30), slice(30, 40)]
    res = [oracle.attention(q, K[p], V[p], 0.25) for p in parts]
    whole = oracle.attention(q, K, V, 0.25)
    left = res[0]
    for r in res[1:]:
        left = oracle.merge(left, r)
    right = res[-1]
    for r in res[-2::-1]:
        right = oracle.merge(r, right)
    tree = oracle.merge(oracle.merge(res[0], res[1]), oracle.merge(res[2], res[3]))
    for x in (left, right, tree, oracle.merge(res[1], oracle.merge(res[3], oracle.merge(res[0], res[2])))):
        assert np.allclose(x[0], whole[0], atol=1e-13)
        assert x[1] == pytest.approx(whole[1], rel=1e-13) and x[2] == whole[2]


def test_missing_set_by_brute_force():
    rng = np.random.default_rng(5)
    for _ in range(100):
        A = np.sort(rng.choice(50, size=int(rng.integers(0, 20)), replace=False))
        P = rng.choice(50, size=int(rng.integers(0, 20)), replace=False)
        M = oracle.missing_pages(A, P)
        assert list(M) == [a for a in A if a not in set(P)]


def test_repair_folds_to_attention_over_union():
    """spec over P then repair over A\\P == attention over P u A; equal to
    attention over A when P is a subset of A."""
    bt = wl.random_batch(21, [16 * 20], n_q_heads=4, n_kv_heads=1, head_dim=16, dtype="bf16")
    for A, P in (([1, 3, 4, 8, 9, 15], [3, 4, 15]), ([1, 3, 4, 8], [0, 3, 19, 8, 2]), ([2, 5], []),
                 ([], [6, 7]), ([4, 5], [4, 5])):
        spec = oracle.attend_pages(bt, 0, 0, sorted(P))
        O, l, m = oracle.repair(bt, 0, 0, spec, A, P)
        ref = oracle.attend_pages(bt, 0, 0, sorted(set(A) | set(P)))
        assert np.allclose(O, ref[0], atol=1e-13) and np.allclose(l, ref[1], rtol=1e-13)
        assert np.array_equal(m, ref[2])
        if set(P) <= set(A):
            refA = oracle.attend_pages(bt, 0, 0, A)
            assert np.allclose(O, refA[0], atol=1e-13)


# ---------------------------------------------------------------- step 6: PSA
def _psa_pages(masses, P=4, D=16):
    """Pages whose keys are all a_b*sqrt(D)*e1 with q = e1, so every logit of
    page b is exactly a_b and the block mass is P*exp(a_b) (D=16: the fp32
    scale 1/4 is exact, and a_b*4 is chosen exactly representable)."""
    a = [math.log(mb / P) for mb in masses]
    a = [round(x * 4 * 2 ** 12) / 2 ** 12 / 4 for x in a]        # exact in fp32 after *4
    e1 = np.zeros(D)
    e1[0] = 1.0
    keys = [np.tile(ab * 4.0 * e1, (P, 1)) for ab in a]
    return hand_batch(keys, e1, P), np.array(a)


def test_psa_hand_built_stop():
    """Masses (100, 50, 25, 1, 1, 1, ...): printed-rule ratios 0.5, 0.75,
    0.875, 176/177 -> stops after 4 pages (threshold 0.95)."""
    bt, a = _psa_pages([100, 50, 25] + [1] * 13)
    S = oracle.page_scores(bt)
    ids, n, O, l, m = oracle.psa_progressive(bt, 0, 0, S[0, 0], 0.95, 0)
    assert n == 4 and list(ids) == [0, 1, 2, 3]
    r = oracle.psa_ratios(bt, 0, 0, S[0, 0], 0)
    exact = np.exp(a) * 4
    acc = np.cumsum(exact)
    mins = np.minimum.accumulate(exact)
    assert np.allclose(r, acc / (acc + mins), rtol=1e-12)
    assert r[:4] == pytest.approx([0.5, 0.75, 0.875, 176 / 177], rel=1e-3)
    # output is attention over the visited pages
    ref = oracle.attend_pages(bt, 0, 0, [0, 1, 2, 3])
    assert np.allclose(O, ref[0], atol=1e-12) and np.allclose(l, ref[1]) and np.allclose(m, ref[2])


def test_psa_rank_follows_scores_not_position():
    bt, a = _psa_pages([1, 1, 25, 100, 1, 50, 1, 1])
    S = oracle.page_scores(bt)
    ids, n, *_ = oracle.psa_progressive(bt, 0, 0, S[0, 0], 0.95, 0)
    assert list(ids) == [3, 5, 2, 0] and n == 4            # ties (mass 1) -> lowest index


def test_psa_printed_rule_bound_and_uniform_masses():
    """AS_acc >= n*AS_min, so the printed rule stops by n = ceil(thr/(1-thr));
    uniform masses reach n/(n+1) >= 0.93 first at n = 14."""
    bt, _ = _psa_pages([3.0] * 40)
    S = oracle.page_scores(bt)
    _, n, *_ = oracle.psa_progressive(bt, 0, 0, S[0, 0], 0.93, 0)
    assert n == 14
    rng = np.random.default_rng(0)
    for _ in range(20):
        bt, _ = _psa_pages(list(np.exp(rng.uniform(0, 4, size=60))))
        S = oracle.page_scores(bt)
        _, n, *_ = oracle.psa_progressive(bt, 0, 0, S[0, 0], 0.95, 0)
        assert n <= 20


def test_psa_remaining_pages_rule():
    """stop_mode 1 multiplies AS_min by the unvisited count: with 5 pages of
    mass 1000 and 95 of mass 1 it needs the remaining tail <= 5% of the
    accumulated mass: after the 5 hot pages ratio = 5000/(5000+95) = 0.981."""
    bt, _ = _psa_pages([1000] * 5 + [1] * 95)
    S = oracle.page_scores(bt)
    _, n1, *_ = oracle.psa_progressive(bt, 0, 0, S[0, 0], 0.95, 1)
    assert n1 == 6      # min drops to 1 only at page 6: 5001/(5001+94) = 0.9816
    _, n0, *_ = oracle.psa_progressive(bt, 0, 0, S[0, 0], 0.95, 0)
    assert n0 == 6      # printed rule: 5000/(5000+1000)=0.833 at 5, 5001/5002 at 6
    # 10 pages of mass 10, 90 of mass 1: printed rule 101/102 at n=11; the
    # remaining-pages rule needs (90+n)/190 >= 0.95, i.e. n = 91
    bt, _ = _psa_pages([10] * 10 + [1] * 90)
    S = oracle.page_scores(bt)
    assert oracle.psa_progressive(bt, 0, 0, S[0, 0], 0.95, 0)[1] == 11
    assert oracle.psa_progressive(bt, 0, 0, S[0, 0], 0.95, 1)[1] == 91


def test_psa_threshold_one_is_dense():
    bt = wl.random_batch(13, [16 * 12 + 3], n_q_heads=1, n_kv_heads=1, head_dim=32, dtype="bf16")
    S = oracle.page_scores(bt)
    ids, n, O, l, m = oracle.psa_progressive(bt, 0, 0, S[0, 0], 1.0, 0)
    assert n == 13
    ref, s = textbook(bt, 0, 0)
    assert np.allclose(O[0], ref, atol=1e-12)
    assert l[0] == pytest.approx(np.exp(s - s.max()).sum(), rel=1e-12)


def test_psa_fusion_equals_merge_with_group():
    """The printed weighted fusion and the (O,l,m) merge are the same algebra:
    with G=2 the fused output equals attention over the visited pages."""
    bt = wl.random_batch(14, [16 * 30], n_q_heads=2, n_kv_heads=1, head_dim=16, dtype="f32")
    S = oracle.page_scores(bt)
    ids, n, O, l, m = oracle.psa_progressive(bt, 0, 0, S[0, 0], 0.8, 0)
    ref = oracle.attend_pages(bt, 0, 0, ids)
    assert np.allclose(O, ref[0], atol=1e-12) and np.allclose(l, ref[1]) and np.allclose(m, ref[2])


def test_blocks_needed_hand_built():
    bt, _ = _psa_pages([100, 50, 25, 1, 1])   # total 177: 0.95*177 = 168.15 -> 3 pages
    assert oracle.blocks_needed(bt, 0, 0, 0.95) == 3


# ---------------------------------------------------------------- step 9: EMA
A, B_, G_ = 0.6, 0.3, 0.25


def _run_ema(series, alpha=A, beta=B_, gamma=G_):
    level, trend = np.array([series[0]], float), np.zeros(1)
    preds = []
    for x in series[1:]:
        preds.append(float(oracle.ema_predict(level, trend, gamma)[0]))
        level, trend = oracle.ema_update(np.array([x]), level, trend, alpha, beta)
    return np.array(preds), level, trend


def test_ema_constant_series_predicts_the_constant():
    preds, level, trend = _run_ema([3.5] * 30)
    assert np.all(preds == 3.5) and level[0] == 3.5 and trend[0] == 0.0


def test_ema_linear_series_closed_form():
    """IS_t = b t: trend -> b/alpha, level lags by (1-alpha) b/alpha, one-step
    error -> b (1-gamma)/alpha = 1.25 b at (0.6, 0.3, 0.25)."""
    b = 2.0
    series = b * np.arange(400)
    preds, level, trend = _run_ema(series)
    assert trend[0] == pytest.approx(b / A, rel=1e-9)
    assert series[-1] - level[0] == pytest.approx((1 - A) * b / A, rel=1e-9)
    err = series[1:] - preds
    assert err[-1] == pytest.approx(b * (1 - G_) / A, rel=1e-9)
    assert err[-1] == pytest.approx(1.25 * b, rel=1e-9)


def test_ema_alpha_one_gamma_zero_is_reuse_last():
    rng = np.random.default_rng(4)
    series = rng.standard_normal(50)
    preds, *_ = _run_ema(series, alpha=1.0, beta=0.3, gamma=0.0)
    assert np.array_equal(preds, series[:-1])


def test_ema_update_reads_previous_level():
    """One hand step: level 2, trend 1, IS 5 -> trend 0.3*(5-2)+0.7*1 = 1.6,
    level 0.6*5+0.4*2 = 3.8, prediction 3.8 + 0.25*1.6 = 4.2."""
    lv, tr = oracle.ema_update([5.0], [2.0], [1.0], A, B_)
    assert lv[0] == pytest.approx(3.8) and tr[0] == pytest.approx(1.6)
    assert oracle.ema_predict(lv, tr, G_)[0] == pytest.approx(4.2)


def test_speculative_set_size():
    pred = np.array([5.0, 1.0, 4.0, 4.0, 0.0, 9.0])
    assert list(oracle.speculative_set(pred, 6, 4, 1.0)) == [0, 2, 3, 5]
    assert list(oracle.speculative_set(pred, 6, 4, 0.5)) == [0, 5]
    assert list(oracle.speculative_set(pred, 6, 3, 0.9)) == [0, 5]   # floor(2.7) = 2


def test_calibration_grid_has_80_candidates():
    """PRR section 3.2 grid: alpha 0.2..0.8 step 0.2, beta 0.1..0.5 step 0.1,
    gamma 0..0.75 step 0.25 -> the page states 80 candidates; the oracle's
    grid is exactly that product, alpha slowest and gamma fastest."""
    alphas = np.arange(0.2, 0.8 + 1e-9, 0.2)
    betas = np.arange(0.1, 0.5 + 1e-9, 0.1)
    gammas = np.arange(0.0, 0.75 + 1e-9, 0.25)
    assert len(alphas) * len(betas) * len(gammas) == 80
    grid = oracle.calibration_grid()
    assert len(grid) == 80 and len(set(grid)) == 80
    for ia, a in enumerate(alphas):
        for ib, b in enumerate(betas):
            for ig, g in enumerate(gammas):
                assert grid[(ia * 5 + ib) * 4 + ig] == pytest.approx((a, b, g), abs=1e-12)


# ---------------------------------------------------------------- calibration (PRR section 3.2)
def test_f32_ema_is_the_ema():
    """The float32 predictor of the calibration agrees with the pinned fp64
    update and prediction to float32 rounding, on random states and on the
    hand step (level 2, trend 1, IS 5 -> 3.8, 1.6, prediction 4.2)."""
    rng = np.random.default_rng(21)
    is_, lv, tr = (rng.standard_normal(1000).astype(np.float32) * 10 for _ in range(3))
    for a, b, g in oracle.calibration_grid()[::7]:
        l32, t32 = oracle.ema_step_f32(is_, lv, tr, a, b)
        l64, t64 = oracle.ema_update(is_, lv, tr, a, b)
        assert np.allclose(l32, l64, rtol=0, atol=1e-5 * 30) and np.allclose(t32, t64, rtol=0, atol=1e-5 * 30)
        p32 = oracle.ema_predict_f32(l32, t32, g)
        assert np.allclose(p32, oracle.ema_predict(l64, t64, g), rtol=0, atol=1e-4)
        assert l32.dtype == np.float32 and p32.dtype == np.float32
    l, t_ = oracle.ema_step_f32([5.0], [2.0], [1.0], 0.6, 0.3)
    assert l[0] == pytest.approx(3.8, rel=1e-6) and t_[0] == pytest.approx(1.6, rel=1e-6)
    assert oracle.ema_predict_f32(l, t_, 0.25)[0] == pytest.approx(4.2, rel=1e-6)


def test_hit_rate_hand_built():
    """IS = [5, 1, 4, 3, 2], k = 2: A = {0, 2}, weight 9.  A prediction that
    ranks pages 0 and 1 highest covers 5 of it; all five pages cover it all;
    no page covers nothing; an empty A has nothing to miss."""
    is_ = np.array([5.0, 1.0, 4.0, 3.0, 2.0])
    pred = np.array([9.0, 8.0, 0.0, 1.0, 2.0])
    assert oracle.hit_rate(pred, is_, 5, 2, 2) == pytest.approx(5 / 9)
    assert oracle.hit_rate(pred, is_, 5, 2, 5) == 1.0
    assert oracle.hit_rate(pred, is_, 5, 2, 0) == 0.0
    assert oracle.hit_rate(pred, is_, 5, 0, 2) == 1.0
    assert oracle.hit_rate(pred, is_, 3, 2, 1) == pytest.approx(5 / 9)   # pages 0..2 valid: A = {0, 2}, P = {0}


def _ramp_trace(T=12, N=40, U=2, seed=22):
    """Pages on straight lines that cross: base ~ U(0, 50), slope ~ U(0, 6)."""
    rng = np.random.default_rng(seed)
    base = rng.uniform(0, 50, (U, N))
    slope = rng.uniform(0, 6, (U, N))
    return np.stack([base + slope * phi for phi in range(T)]).astype(np.float32)


def test_calibrate_bounds_and_degenerate_budgets():
    """0 <= H <= 1; a constant trace is predicted exactly (H = 1 for every
    candidate); P over all valid pages covers A (H = 1); an empty P covers
    nothing (H = 0)."""
    tr = _ramp_trace()
    nv = [40, 33]
    H = oracle.calibrate(tr, nv, 8, 8)
    assert np.all((H >= 0) & (H <= 1)) and not np.all(H == 1)
    const = np.repeat(tr[:1], 6, axis=0)
    assert np.all(oracle.calibrate(const, nv, 8, 8) == 1.0)
    assert np.all(oracle.calibrate(tr[:5], nv, 8, 40) == 1.0)
    assert np.all(oracle.calibrate(tr[:5], nv, 8, 0) == 0.0)


def test_calibrate_prefers_fast_extrapolation_on_ramps():
    """On crossing straight lines the EMA lags each page by about
    slope * (1 - gamma) / alpha (the linear-series closed form), so rising
    pages are under-ranked: the highest alpha and gamma of the grid win, and
    more extrapolation never hurts at fixed (alpha, beta)."""
    tr = _ramp_trace(T=16, N=60, U=1, seed=23)
    H = oracle.calibrate(tr, [60], 10, 10)[0]
    grid = oracle.calibration_grid()
    a, _, g = grid[oracle.best_candidate(H)]
    assert a == 0.8 and g == 0.75
    assert H[0] < H[oracle.best_candidate(H)]
    for c in range(0, 80, 4):   # gamma = 0, 0.25, 0.5, 0.75 at one (alpha, beta)
        assert H[c] <= H[c + 1] <= H[c + 2] <= H[c + 3]


def test_calibrate_matches_a_direct_loop():
    """On a trace whose scores are spaced widely enough that float32 and
    float64 rank alike, H of a few candidates equals a direct loop over the
    fp64 EMA, top-k selections and the weighted hit share."""
    rng = np.random.default_rng(24)
    T, U, N, k, m = 7, 2, 30, 6, 5
    tr = (rng.permutation(np.arange(T * U * N)).reshape(T, U, N) * 8.0 + 64.0).astype(np.float32)
    grid = oracle.calibration_grid()
    cols = [0, 17, 42, 79]
    H = oracle.calibrate(tr, [N, N - 4], k, m, candidates=cols)
    for u, nv in enumerate([N, N - 4]):
        for c in cols:
            a, b, g = grid[c]
            level, trend, total = tr[0, u].astype(float), np.zeros(N), 0.0
            for phi in range(1, T):
                pred = oracle.ema_predict(level, trend, g)
                is_ = tr[phi, u].astype(float)
                A = set(np.argsort(-is_[:nv], kind="stable")[:k].tolist())
                P = set(np.argsort(-pred[:nv], kind="stable")[:m].tolist())
                total += sum(is_[j] for j in A & P) / sum(is_[j] for j in A)
                level, trend = oracle.ema_update(is_, level, trend, a, b)
            assert H[u, c] == pytest.approx(total / (T - 1), rel=1e-12)


# ---------------------------------------------------------------- workload checks
# ---------------------------------------------------------------- block-sparse prefill (LServe sections 2.3, 4.1)
def test_prefill_dense_is_textbook_causal_softmax():
    """Dense heads: query i is softmax(scale * K[:i+1] q_i) V[:i+1], by scipy."""
    L, Hq, Hkv, D = 23, 4, 2, 8
    q, k, v = wl.prefill_inputs(41, L, Hq, Hkv, D, "f32", q_gain=2.0)
    sc = 0.35
    O, l, m = oracle.prefill_attention(q, k, v, "f32", sc)
    for hq in range(Hq):
        h = hq // 2
        for i in range(L):
            s = sc * (k[:i + 1, h].astype(float) @ q[i, hq].astype(float))
            np.testing.assert_allclose(O[i, hq], softmax(s) @ v[:i + 1, h].astype(float), rtol=1e-12, atol=1e-12)
            assert m[i, hq] == pytest.approx(s.max()) and l[i, hq] == pytest.approx(np.exp(s - s.max()).sum())


def test_prefill_streaming_lambda_mask():
    """A streaming head attends to the sink tokens and the last `local`
    tokens up to i (the decode rule at length i + 1); with sink + local
    covering everything it is the dense head; the keys are a subset of the
    causal ones and always include i itself when local >= 1."""
    L, sink, local = 40, 3, 5
    for i in range(L):
        j = oracle.prefill_keys(i, L, True, sink, local)
        expect = [x for x in range(i + 1) if x < sink or x >= i + 1 - local]
        assert list(j) == expect and i in j
        assert list(oracle.prefill_keys(i, L, False, sink, local)) == list(range(i + 1))
    q, k, v = wl.prefill_inputs(42, 17, 2, 1, 8, "bf16")
    a = oracle.prefill_attention(q, k, v, "bf16", 0.3, streaming=[1], sink=4, local=13)
    b = oracle.prefill_attention(q, k, v, "bf16", 0.3)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    c = oracle.prefill_attention(q, k, v, "bf16", 0.3, streaming=[1], sink=2, local=3)
    assert not np.allclose(c[0][10:], b[0][10:])


# ---------------------------------------------------------------- reusable selector (LServe section 4.3)
def test_reuse_chunk_starts():
    """Chunk size 4: steps 0-3 use step 0's selection, 4-7 step 4's, ...;
    chunk size 1 selects at every step."""
    assert [oracle.chunk_start(t, 4) for t in range(10)] == [0, 0, 0, 0, 4, 4, 4, 4, 8, 8]
    assert [oracle.chunk_start(t, 1) for t in range(5)] == [0, 1, 2, 3, 4]


def test_reuse_decode_against_fresh_selection():
    """Chunk 1 is the plain per-step pipeline; with chunk 4 every step uses
    the pages of its chunk's first query and attends with its own query, and
    a query that repeats within a chunk reproduces the fresh step exactly."""
    bt = wl.random_batch(31, [200, 77], n_q_heads=4, n_kv_heads=2, head_dim=16, page_size=16)
    qs = wl.query_drift(32, bt.q, 6, 0.3, bt.dtype)
    ids1, out1 = oracle.reuse_decode(bt, qs, 3, 1)
    ids4, out4 = oracle.reuse_decode(bt, qs, 3, 4)
    for t in range(6):
        _, ref_ids, ref = oracle.quest_step(bt, 3, q=qs[t])
        assert all(np.array_equal(a, b) for ra, rb in zip(ids1[t], ref_ids) for a, b in zip(ra, rb))
        for x, y in zip(out1[t], ref):
            np.testing.assert_array_equal(x, y)
        s = oracle.chunk_start(t, 4)
        _, start_ids, _ = oracle.quest_step(bt, 3, q=qs[s])
        assert all(np.array_equal(a, b) for ra, rb in zip(ids4[t], start_ids) for a, b in zip(ra, rb))
        for x, y in zip(out4[t], oracle.sparse_decode(bt, start_ids, qs[t])):
            np.testing.assert_array_equal(x, y)
    same = np.stack([qs[0]] * 3)
    _, o_same = oracle.reuse_decode(bt, same, 3, 4)
    for x, y in zip(o_same[2], oracle.quest_step(bt, 3, q=qs[0])[2]):
        np.testing.assert_array_equal(x, y)


def test_query_drift_keeps_the_norm_scale():
    """theta = 0 repeats q0; a drifting step is a rotation-like mix whose
    cosine with the previous query is about cos(theta) for wide heads."""
    bt = wl.random_batch(33, [40], n_q_heads=2, n_kv_heads=1, head_dim=128, page_size=16, dtype="f32")
    assert np.array_equal(wl.query_drift(1, bt.q, 3, 0.0, "f32")[2], bt.q)
    qs = wl.query_drift(2, bt.q, 2, 0.3, "f32").astype(np.float64)
    c = (qs[0] * qs[1]).sum(-1) / np.linalg.norm(qs[0], axis=-1) / np.linalg.norm(qs[1], axis=-1)
    assert np.all(np.abs(c - math.cos(0.3)) < 0.1)


def test_quest_bias_pages_have_cosine_0_4_and_rank_high():
    bt = wl.quest_gqa(seq_len=4096, n_kv_heads=2, n_q_heads=8)
    qbar = oracle.group_query(bt)
    S = oracle.page_scores(bt)
    for h in range(2):
        pages = bt.extra["biased_pages"][0, h]
        u = qbar[0, h] / np.linalg.norm(qbar[0, h])
        K = token_major(bt, bt.k, 0, h)
        for p in pages[:3]:
            kk = K[p * 16:(p + 1) * 16]
            cos = (kk @ u) / np.linalg.norm(kk, axis=1)
            assert np.allclose(cos, 0.4, atol=0.01)        # bf16 rounding of the keys
        ranks = np.argsort(np.argsort(-S[0, h, :256]))
        assert np.median(ranks[pages]) < 64


def test_golden_calibration_grid():
    """tests/golden/prr_calibration_grid.txt holds the search space the PRR
    page prints (section 3.2); the oracle's grid is its full product with
    alpha slowest and gamma fastest, and has the printed count."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "prr_calibration_grid.txt")
    spec, count = {}, None
    for line in open(path):
        f = line.split("#")[0].split()
        if not f:
            continue
        if f[0] == "count":
            count = int(f[1])
        else:
            first, last, step = (float(x) for x in f[1:4])
            n = int(round((last - first) / step)) + 1
            spec[f[0]] = [first + i * step for i in range(n)]
    want = [(a, b, g) for a in spec["alpha"] for b in spec["beta"] for g in spec["gamma"]]
    grid = oracle.calibration_grid()
    assert len(want) == count == len(grid)
    for x, y in zip(grid, want):
        assert x == pytest.approx(y, abs=1e-12)
