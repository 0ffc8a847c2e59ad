"""Helpers shared by the GPU parity tests: upload a generated batch, run the
HIP path through the C ABI, and the parity rules that compare it with the
oracle."""
from __future__ import annotations

import numpy as np

import oracle

# Output tolerances (max-abs on O; m absolute; l relative).
TOL = {
    "bf16": dict(O=2e-3, m=1e-4, l=1e-4),
    "f32": dict(O=1e-5, m=1e-6, l=1e-5),
}
SCORE_REL = 1e-5   # selection boundary exemption, relative to the k-th score


def to_device(dsa, batch):
    q = dsa.upload_q(batch.q, batch.dtype)
    kv = dsa.PagedKV.from_numpy(batch.k, batch.v, batch.page_table, batch.seq_lens, batch.dtype)
    st = None
    if batch.streaming is not None:
        st = dsa.Streaming(batch.streaming, batch.sink, batch.local)
    return q, kv, st


def np_(t):
    return t.detach().cpu().numpy()


def check_selection(gpu_ids: np.ndarray, gpu_count: int, oracle_row: np.ndarray, n_valid: int, k: int, what=""):
    """Rule (i): the selected sets match exactly, except pairs in the
    symmetric difference whose oracle scores both lie within SCORE_REL of the
    oracle's k-th score (never pairs of exactly equal oracle scores)."""
    ref = oracle.topk_pages(oracle_row, n_valid, k)
    got = gpu_ids[:gpu_count]
    assert gpu_count == len(ref), f"{what}: count {gpu_count} != {len(ref)}"
    assert np.all(np.diff(got) > 0), f"{what}: ids not strictly ascending"
    assert np.all(gpu_ids[gpu_count:] == -1), f"{what}: padding not -1"
    diff = set(got.tolist()) ^ set(ref.tolist())
    if not diff:
        return 0
    ranked = oracle.rank_pages(oracle_row, n_valid)
    tau = oracle_row[ranked[len(ref) - 1]]
    band = SCORE_REL * abs(tau)
    for x in diff:
        assert abs(oracle_row[x] - tau) <= band, \
            f"{what}: page {x} (score {oracle_row[x]!r}) differs from oracle, k-th score {tau!r}"
    vals = [oracle_row[x] for x in diff]
    assert len(set(vals)) == len(vals), f"{what}: exact ties resolved differently"
    return len(diff) // 2


def check_attention(dtype: str, O, l, m, ref_O, ref_l, ref_m, what=""):
    t = TOL[dtype]
    ref_m = np.asarray(ref_m, float)
    empty = np.isneginf(ref_m)
    assert np.array_equal(np.isneginf(m), empty), f"{what}: empty-set pattern differs"
    assert np.all(l[empty] == 0) and np.all(O[empty] == 0), f"{what}: empty set must give O=0, l=0"
    ok = ~empty
    if ok.any():
        dO = np.abs(O[ok] - ref_O[ok]).max()
        dm = np.abs(m[ok] - ref_m[ok]).max()
        dl = (np.abs(l[ok] - ref_l[ok]) / ref_l[ok]).max()
        assert dO <= t["O"], f"{what}: max|dO| = {dO:.3g} > {t['O']}"
        assert dm <= t["m"] * max(1.0, np.abs(ref_m[ok]).max()), f"{what}: max|dm| = {dm:.3g}"
        assert dl <= t["l"], f"{what}: max rel dl = {dl:.3g}"


def ids_lists(ids: np.ndarray, counts: np.ndarray):
    """[B][H][stride] + counts -> nested python lists of id arrays."""
    B, H = counts.shape
    return [[ids[b, h, :counts[b, h]].astype(np.int64) for h in range(H)] for b in range(B)]


def upload_ids(ref_ids, stride: int):
    """Nested id lists [b][h] -> int32 device tensors (ids [B][H][stride], -1
    padded; counts [B][H])."""
    import torch
    B, H = len(ref_ids), len(ref_ids[0])
    ids = np.full((B, H, stride), -1, np.int32)
    counts = np.zeros((B, H), np.int32)
    for b in range(B):
        for h in range(H):
            r = np.asarray(ref_ids[b][h], np.int64)[:stride]
            ids[b, h, :len(r)] = r
            counts[b, h] = len(r)
    return torch.from_numpy(ids).cuda(), torch.from_numpy(counts).cuda()


def check_selected_attention(dsa, batch, q, kv, st, ids, counts, out, ref_ids, units, what="", **attn_kw):
    """Outputs of an attention over the kernel's own selection, against the
    oracle's attention over the oracle's selection ``ref_ids`` ([b][h] lists;
    the sets were compared by check_selection before).  A unit whose set
    equals the oracle's is compared directly.  Where a unit's set differs by
    an exempted boundary pair, the attention kernel runs again on the
    oracle's ids and that output is compared for the unit, so no value the
    kernels produced becomes an input of the oracle.  Returns the number of
    such units."""
    G = batch.group
    On, ln, mn = (np_(x) for x in out)
    differ = []
    for b, h in units:
        sl = slice(h * G, (h + 1) * G)
        ref = oracle.attend_pages(batch, b, h, np.asarray(ref_ids[b][h], np.int64))
        if np.array_equal(ids[b, h, :counts[b, h]], ref_ids[b][h]):
            check_attention(batch.dtype, On[b, sl], ln[b, sl], mn[b, sl], *ref, f"{what} (b={b}, h={h})")
        else:
            differ.append((b, h, ref))
    if differ:
        it, ct = upload_ids(ref_ids, ids.shape[2])
        O2, l2, m2 = (np_(x) for x in dsa.sparse_decode_attn(q, kv, it, ct, streaming=st, **attn_kw))
        for b, h, ref in differ:
            sl = slice(h * G, (h + 1) * G)
            check_attention(batch.dtype, O2[b, sl], l2[b, sl], m2[b, sl], *ref, f"{what} on oracle ids (b={b}, h={h})")
    return len(differ)


def check_psa(dsa, bt, q, kv, s32: np.ndarray, thr: float, mode: int, what=""):
    """PSA's progressive selection on the score rows `s32` ([B][H][max_pages]
    float32) against the oracle's walk over the same values, unit by unit
    (see check_psa_result).  Returns the counts."""
    import torch
    sc = torch.from_numpy(np.ascontiguousarray(s32, np.float32)).cuda()
    res = [np_(x) for x in dsa.page_select_progressive(q, kv, sc, thr, mode, float(bt.scale))]
    check_psa_result(bt, s32, *res, thr, mode, what)
    return res[1]


def check_psa_result(bt, s32, ids, counts, O, l, m, thr: float, mode: int, what="", units=None):
    """One progressive-selection result against the oracle's walk over the
    same float32 scores: the stop count (a different count only where a
    stop-test ratio sits on the threshold), the visited pages in rank order,
    -1 after them, and the attention over the visited pages."""
    G = bt.group
    if units is None:
        units = [(b, h) for b in range(bt.batch) for h in range(bt.n_kv_heads)]
    for b, h in units:
        nv = oracle.n_pages(bt.seq_lens[b], bt.page_size)
        row = s32[b, h].astype(np.float64)
        rid, rn, *_ = oracle.psa_progressive(bt, b, h, row, thr, mode)
        n = int(counts[b, h])
        if n != rn:
            ratios = oracle.psa_ratios(bt, b, h, row, mode)
            lo, hi = min(n, rn), max(n, rn)
            near = np.abs(ratios[lo - 1:hi] - thr) <= 1e-5 * thr
            assert near.any(), f"{what}: stop {n} != oracle {rn} at (b={b}, h={h})"
        ranked = oracle.rank_pages(row, nv)
        assert np.array_equal(ids[b, h, :n], ranked[:n]), f"{what}: visit order differs at (b={b}, h={h})"
        assert np.all(ids[b, h, n:] == -1), f"{what}: padding not -1 at (b={b}, h={h})"
        ref = oracle.attend_pages(bt, b, h, ids[b, h, :n])
        sl = slice(h * G, (h + 1) * G)
        check_attention(bt.dtype, O[b, sl], l[b, sl], m[b, sl], *ref, f"{what} (b={b}, h={h})")
