"""Oracle for query-aware block-sparse paged decode attention.

TEST INFRASTRUCTURE ONLY.  This is a plain, slow, float64 CPU statement of
what the GPU path computes.  Only the tests, the package smoke check and the
CPU-baseline leg of the benchmark may import it; the product path never does.
It shares no code with the HIP library: it has its own bf16 decoding, its own
page walking and its own arithmetic.

Sources (each function names the passage it follows):

* PSA  = "PSA: Progressive Sparse Attention -- Algorithm and System Co-design
  for Efficient Attention in LLM Serving" (arXiv 2503.00392), blog review.
* LServe = "LServe: Efficient Long-sequence LLM Serving with Unified Sparse
  Attention" (arXiv 2502.14866), blog review.
* PRR  = "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention
  for Long-Context LLM Decoding" (arXiv 2606.30389), blog review.

Readings taken where the pages are silent (listed in the design notes too):
logits are ``scale * q.k`` with the caller's float32 scale; a page's key
metadata is the per-channel min and max over the page's valid tokens; the
GQA representative query is the mean of the group's q heads; ties in any
ranking go to the lower page index; a PSA block weight is the block's
unnormalised softmax mass ``sum_t exp(s_t)``; a logical page with no valid
token takes no part in the physical max; the EMA state starts at
``level = IS, trend = 0``.

Every function here is pinned by the CPU tests (tests/test_oracle_pins.py)
against closed forms, brute force or hand-built inputs.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

NEG_INF = -math.inf


# --------------------------------------------------------------------------
# input decoding (the oracle's own)
# --------------------------------------------------------------------------
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly.  bf16 is the upper half of an IEEE
    binary32 word, so shifting the 16 stored bits up by 16 gives the value."""
    if dtype == "bf16":
        return (np.asarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    raise ValueError(dtype)


def n_pages(seq_len: int, page_size: int) -> int:
    return -(-int(seq_len) // page_size)


def page_tokens(pool: np.ndarray, dtype: str, page_table, b: int, h: int, page: int,
                seq_len: int, page_size: int) -> np.ndarray:
    """The valid key (or value) rows of one page of sequence b, KV head h,
    read through the page table (the paged block pool of PSA section 3.4 and
    LServe section 3.2.1)."""
    n_valid = min(page_size, int(seq_len) - page * page_size)
    if n_valid <= 0:
        return np.zeros((0, pool.shape[-1]))
    slot = int(page_table[b][page])
    return widen(pool[slot, h, :n_valid], dtype)


# --------------------------------------------------------------------------
# step 1: page key metadata  (LServe section 4.2, Figure 7; PSA section 3.1)
# --------------------------------------------------------------------------
def page_meta(batch, units=None) -> tuple[np.ndarray, np.ndarray]:
    """kmin/kmax of every logical page, per channel, over its valid tokens.

    Returns ``meta[num_slots][Hkv][g][2][D]`` (index 0 = kmin, 1 = kmax) and
    ``has[num_slots][Hkv][g]`` (True where the logical page has at least one
    valid token).  Slots no sequence uses stay NaN / False.  ``units``, a
    set of (sequence, KV head) pairs, restricts the work to those."""
    P, Pl, D = batch.page_size, batch.logical_page, batch.head_dim
    g = P // Pl
    meta = np.full((batch.num_slots, batch.n_kv_heads, g, 2, D), np.nan)
    has = np.zeros((batch.num_slots, batch.n_kv_heads, g), bool)
    for b in range(batch.batch):
        L = int(batch.seq_lens[b])
        for j in range(n_pages(L, P)):
            slot = int(batch.page_table[b][j])
            for h in range(batch.n_kv_heads):
                if units is not None and (b, h) not in units:
                    continue
                keys = page_tokens(batch.k, batch.dtype, batch.page_table, b, h, j, L, P)
                for s in range(g):
                    sub = keys[s * Pl:(s + 1) * Pl]
                    if len(sub) == 0:
                        continue
                    meta[slot, h, s, 0] = sub.min(axis=0)
                    meta[slot, h, s, 1] = sub.max(axis=0)
                    has[slot, h, s] = True
    return meta, has


# --------------------------------------------------------------------------
# decode-time append  (PSA section 3.1, system design: the KV cache manager
# writes each new token's K/V into its GPU block, and block metadata stays in
# GPU memory; LServe section 4.2, Figure 7: a physical page's kmin/kmax come
# from the prefill and the earlier decode steps)
# --------------------------------------------------------------------------
def append_token(batch, k_new, v_new):
    """One new token per sequence, at position p = seq_lens[b]: its rows
    k_new[b][h], v_new[b][h] (stored format) go to row p % P of the slot that
    holds page p // P, and the sequence grows by one.  A sequence whose page
    lies past max_pages, or whose page-table entry is no slot, is left as it
    is (the slot of a new page is allocated by the caller beforehand).

    Returns (grown batch, appended flags).  The key metadata of the grown
    cache is, by definition, page_meta() of the returned batch: an
    incremental update must reach exactly that, since min and max are
    exact."""
    P = batch.page_size
    out = dataclasses.replace(batch, k=batch.k.copy(), v=batch.v.copy(),
                              seq_lens=np.array(batch.seq_lens, dtype=np.int32, copy=True))
    done = np.zeros(batch.batch, bool)
    for b in range(batch.batch):
        p = int(batch.seq_lens[b])
        j = p // P
        if p < 0 or j >= batch.max_pages:
            continue
        slot = int(batch.page_table[b][j])
        if not 0 <= slot < batch.num_slots:
            continue
        out.k[slot, :, p % P] = k_new[b]
        out.v[slot, :, p % P] = v_new[b]
        out.seq_lens[b] = p + 1
        done[b] = True
    return out, done


# --------------------------------------------------------------------------
# step 2: representative query  (PRR section 5, Quest GQA extension)
# --------------------------------------------------------------------------
def group_query(batch, q=None) -> np.ndarray:
    """One query per KV head: the mean of the q heads that share it."""
    qf = widen(batch.q if q is None else q, batch.dtype)
    B, Hq, D = qf.shape
    G = Hq // batch.n_kv_heads
    return qf.reshape(B, batch.n_kv_heads, G, D).mean(axis=2)


# --------------------------------------------------------------------------
# step 3+4: logical page criticality and physical max  (LServe section 4.2)
# --------------------------------------------------------------------------
def criticality(qbar: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> float:
    """S = sum over channels of max(q_i * kmax_i, q_i * kmin_i): the largest
    value q.k can take for a key inside the page's per-channel box."""
    return float(np.sum(np.maximum(qbar * kmax, qbar * kmin)))


def page_scores(batch, meta=None, has=None, q=None, with_logical: bool = False, units=None):
    """Physical page scores ``[B][Hkv][max_pages]``.  A physical page's score
    is the max of its logical pages' scores; pages past the sequence end and
    every page of a streaming head score -inf.  ``units`` restricts the work
    to those (sequence, KV head) pairs (the others stay -inf)."""
    if meta is None:
        meta, has = page_meta(batch, units)
    qbar = group_query(batch, q)
    P, Pl = batch.page_size, batch.logical_page
    g = P // Pl
    B, Hkv, N = batch.batch, batch.n_kv_heads, batch.max_pages
    phys = np.full((B, Hkv, N), NEG_INF)
    logical = np.full((B, Hkv, N, g), NEG_INF)
    for b in range(B):
        for h in range(Hkv):
            if batch.streaming is not None and batch.streaming[h]:
                continue
            if units is not None and (b, h) not in units:
                continue
            for j in range(n_pages(batch.seq_lens[b], P)):
                slot = int(batch.page_table[b][j])
                for s in range(g):
                    if has[slot, h, s]:
                        logical[b, h, j, s] = criticality(qbar[b, h], meta[slot, h, s, 0], meta[slot, h, s, 1])
                phys[b, h, j] = logical[b, h, j].max()
    return (phys, logical) if with_logical else phys


# --------------------------------------------------------------------------
# step 5: fixed top-k  (PSA section 2.2; PRR section 2, selection stage)
# --------------------------------------------------------------------------
def rank_pages(scores_row: np.ndarray, n_valid: int) -> np.ndarray:
    """Valid page indices by descending score; equal scores by lower index."""
    idx = np.arange(n_valid)
    return idx[np.lexsort((idx, -scores_row[:n_valid]))]


def topk_pages(scores_row: np.ndarray, n_valid: int, k: int) -> np.ndarray:
    """The min(k, n_valid) best pages, returned in ascending index order."""
    return np.sort(rank_pages(scores_row, n_valid)[:max(0, k)])


def streaming_pages(seq_len: int, page_size: int, sink: int, local: int) -> np.ndarray:
    """Pages holding a sink token ([0, sink)) or a local token
    ([L-local, L)), ascending (LServe section 4.1, the Lambda mask)."""
    L = int(seq_len)
    toks = set(range(min(sink, L))) | set(range(max(0, L - local), L))
    return np.array(sorted({t // page_size for t in toks}), dtype=np.int64)


def select_topk(batch, scores: np.ndarray, k: int) -> list:
    """ids[b][h] for every (sequence, KV head): top-k pages of a dense head,
    the sink/local pages of a streaming head."""
    out = []
    for b in range(batch.batch):
        row = []
        n = n_pages(batch.seq_lens[b], batch.page_size)
        for h in range(batch.n_kv_heads):
            if batch.streaming is not None and batch.streaming[h]:
                row.append(streaming_pages(batch.seq_lens[b], batch.page_size, batch.sink, batch.local))
            else:
                row.append(topk_pages(scores[b, h], n, k))
        out.append(row)
    return out


# --------------------------------------------------------------------------
# step 7: softmax attention over a token set, emitting (O, l, m)
#         (PRR section 3.3, instrumented speculative kernel)
# --------------------------------------------------------------------------
def attention(qh: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Logits s_t = scale * q.k_t; m = max s, l = sum exp(s - m),
    O = sum exp(s - m) v_t / l.  An empty set gives (0, 0, -inf)."""
    if len(keys) == 0:
        return np.zeros(values.shape[-1]), 0.0, NEG_INF
    s = scale * (keys @ qh)
    m = float(s.max())
    p = np.exp(s - m)
    l = float(p.sum())
    return (p @ values) / l, l, m


def gather(batch, b: int, h: int, pages, streaming_mask: bool):
    """Keys and values of the valid tokens of ``pages`` (sequence b, KV head
    h).  With ``streaming_mask`` only sink and local tokens are kept."""
    L, P = int(batch.seq_lens[b]), batch.page_size
    ks, vs = [], []
    for j in pages:
        j = int(j)
        kk = page_tokens(batch.k, batch.dtype, batch.page_table, b, h, j, L, P)
        vv = page_tokens(batch.v, batch.dtype, batch.page_table, b, h, j, L, P)
        if streaming_mask:
            t = j * P + np.arange(len(kk))
            keep = (t < batch.sink) | (t >= L - batch.local)
            kk, vv = kk[keep], vv[keep]
        ks.append(kk)
        vs.append(vv)
    D = batch.head_dim
    if not ks:
        return np.zeros((0, D)), np.zeros((0, D))
    return np.concatenate(ks), np.concatenate(vs)


def attend_pages(batch, b: int, h: int, pages, q=None):
    """(O[G][D], l[G], m[G]) for the G q heads of KV head h over ``pages``."""
    qf = widen(batch.q if q is None else q, batch.dtype)
    G = batch.group
    streaming = batch.streaming is not None and bool(batch.streaming[h])
    keys, values = gather(batch, b, h, pages, streaming)
    scale = float(batch.scale)
    O = np.zeros((G, batch.head_dim))
    l = np.zeros(G)
    m = np.full(G, NEG_INF)
    for g in range(G):
        O[g], l[g], m[g] = attention(qf[b, h * G + g], keys, values, scale)
    return O, l, m


def sparse_decode(batch, ids, q=None):
    """(O[B][Hq][D], l[B][Hq], m[B][Hq]) over the given page lists."""
    G = batch.group
    B, Hq, D = batch.batch, batch.n_q_heads, batch.head_dim
    O, l, m = np.zeros((B, Hq, D)), np.zeros((B, Hq)), np.full((B, Hq), NEG_INF)
    for b in range(B):
        for h in range(batch.n_kv_heads):
            o_, l_, m_ = attend_pages(batch, b, h, ids[b][h], q)
            O[b, h * G:(h + 1) * G], l[b, h * G:(h + 1) * G], m[b, h * G:(h + 1) * G] = o_, l_, m_
    return O, l, m


def dense_attention(batch, q=None):
    """Textbook softmax attention over every valid token (the limit that
    top-k with k >= N, or PSA with threshold 1, must reach)."""
    ids = [[np.arange(n_pages(batch.seq_lens[b], batch.page_size))] * batch.n_kv_heads
           for b in range(batch.batch)]
    return sparse_decode(batch, ids, q)


# --------------------------------------------------------------------------
# the (O, l, m) merge  (PRR section 3.3 recurrence; PSA section 3.2 fusion)
# --------------------------------------------------------------------------
def merge(a, b):
    """Fold two partial results over disjoint token sets: the new max is the
    larger max, each side's denominator is rescaled by exp(m_side - m_new)
    and the outputs are averaged with the rescaled denominators."""
    O1, l1, m1 = a
    O2, l2, m2 = b
    m = max(m1, m2)
    if m == NEG_INF:
        return np.zeros_like(np.asarray(O1, float)), 0.0, NEG_INF
    w1 = math.exp(m1 - m) * l1 if m1 != NEG_INF else 0.0
    w2 = math.exp(m2 - m) * l2 if m2 != NEG_INF else 0.0
    l = w1 + w2
    return (w1 * np.asarray(O1) + w2 * np.asarray(O2)) / l, l, m


# --------------------------------------------------------------------------
# step 6: progressive threshold selection  (PSA section 3.2)
# --------------------------------------------------------------------------
def psa_progressive(batch, b: int, h: int, scores_row: np.ndarray, threshold: float,
                    stop_mode: int = 0, q=None):
    """Rank the pages by criticality, attend to them one at a time from the
    most critical, fold each block into the running output with weight equal
    to its attention mass, and stop as soon as the accumulated mass over
    (accumulated mass + smallest block mass) reaches ``threshold``.

    stop_mode 0 is that printed test.  stop_mode 1 multiplies the smallest
    block mass by the number of blocks not yet visited (the pseudo-code keeps
    that counter but the printed test never reads it).  A threshold >= 1
    never stops early; a test that never passes visits every page.

    Returns (ranked ids visited, n_visited, O[G][D], l[G], m[G]); with G > 1
    the block mass is summed over the group's q heads."""
    qf = widen(batch.q if q is None else q, batch.dtype)
    G, D = batch.group, batch.head_dim
    n_valid = n_pages(batch.seq_lens[b], batch.page_size)
    order = rank_pages(scores_row, n_valid)
    O_acc = np.zeros((G, D))
    lnAS_acc_h = np.full(G, NEG_INF)     # per head, for the fusion weights
    tot = [(np.zeros(D), 0.0, NEG_INF) for _ in range(G)]
    lnAS_acc, lnAS_min = NEG_INF, math.inf
    n_left = n_valid
    visited = []
    scale = float(batch.scale)
    for j in order:
        keys, values = gather(batch, b, h, [j], False)
        lnAS_blk = NEG_INF
        for g in range(G):
            o, l, m = attention(qf[b, h * G + g], keys, values, scale)
            ln_as = m + math.log(l)                   # block mass l * e^m
            # O_acc <- (AS_acc * O_acc + AS * O) / (AS_acc + AS)
            new = np.logaddexp(lnAS_acc_h[g], ln_as)
            w_old = math.exp(lnAS_acc_h[g] - new) if lnAS_acc_h[g] != NEG_INF else 0.0
            O_acc[g] = w_old * O_acc[g] + math.exp(ln_as - new) * o
            lnAS_acc_h[g] = new
            tot[g] = merge(tot[g], (o, l, m))
            lnAS_blk = np.logaddexp(lnAS_blk, ln_as)
        lnAS_acc = float(np.logaddexp(lnAS_acc, lnAS_blk))
        lnAS_min = min(lnAS_min, float(lnAS_blk))
        n_left -= 1
        visited.append(int(j))
        if threshold >= 1.0:
            continue
        mult = 1.0 if stop_mode == 0 else float(n_left)
        ratio = 1.0 / (1.0 + mult * math.exp(lnAS_min - lnAS_acc))
        if ratio >= threshold:
            break
    l = np.array([t[1] for t in tot])
    m = np.array([t[2] for t in tot])
    return np.array(visited, np.int64), len(visited), O_acc, l, m


def psa_unit(batch, b: int, h: int, scores_row: np.ndarray, threshold: float, stop_mode: int = 0, q=None):
    """PSA's result for one (sequence, KV head) of a batch that may hold
    streaming heads: a dense head takes the progressive walk above; a
    streaming head (LServe section 4.1: it attends only to its sink and
    local tokens) is not ranked -- it visits the pages holding such tokens in
    ascending order and attends to those tokens only, with no early stop.
    Returns (ids visited, n_visited, O[G][D], l[G], m[G])."""
    if batch.streaming is not None and batch.streaming[h]:
        pages = streaming_pages(batch.seq_lens[b], batch.page_size, batch.sink, batch.local)
        O, l, m = attend_pages(batch, b, h, pages, q)
        return pages, len(pages), O, l, m
    return psa_progressive(batch, b, h, scores_row, threshold, stop_mode, q)


def psa_ratios(batch, b: int, h: int, scores_row: np.ndarray, stop_mode: int = 0, q=None) -> np.ndarray:
    """The stop-test ratio after each page in rank order (diagnostic used by
    the parity rule for stops that sit on the threshold)."""
    qf = widen(batch.q if q is None else q, batch.dtype)
    G = batch.group
    n_valid = n_pages(batch.seq_lens[b], batch.page_size)
    order = rank_pages(scores_row, n_valid)
    out = []
    lnAS_acc, lnAS_min, n_left = NEG_INF, math.inf, n_valid
    for j in order:
        keys, values = gather(batch, b, h, [j], False)
        lnAS_blk = NEG_INF
        for g in range(G):
            _, l, m = attention(qf[b, h * G + g], keys, values, float(batch.scale))
            lnAS_blk = np.logaddexp(lnAS_blk, m + math.log(l))
        lnAS_acc = float(np.logaddexp(lnAS_acc, lnAS_blk))
        lnAS_min = min(lnAS_min, float(lnAS_blk))
        n_left -= 1
        mult = 1.0 if stop_mode == 0 else float(n_left)
        out.append(1.0 / (1.0 + mult * math.exp(lnAS_min - lnAS_acc)))
    return np.array(out)


def blocks_needed(batch, b: int, h: int, threshold: float, q=None) -> int:
    """Diagnostic, never a GPU output: the fewest pages whose true softmax
    mass reaches ``threshold`` of the total (PSA section 2.2, Observation 1)."""
    qf = widen(batch.q if q is None else q, batch.dtype)
    G = batch.group
    n = n_pages(batch.seq_lens[b], batch.page_size)
    masses = np.zeros(n)
    for j in range(n):
        keys, _ = gather(batch, b, h, [j], False)
        for g in range(G):
            masses[j] += np.exp(float(batch.scale) * (keys @ qf[b, h * G + g])).sum()
    c = np.cumsum(np.sort(masses)[::-1])
    return int(np.searchsorted(c, threshold * c[-1]) + 1)


# --------------------------------------------------------------------------
# step 8: repair  (PRR section 3.3 repair kernel, section 3.4 missing set)
# --------------------------------------------------------------------------
def missing_pages(a_ids, p_ids) -> np.ndarray:
    """M = A \\ P, in A's (ascending) order."""
    p = set(int(x) for x in p_ids)
    return np.array([int(x) for x in a_ids if int(x) not in p], dtype=np.int64)


def repair(batch, b: int, h: int, spec, a_ids, p_ids, q=None):
    """Fold the attention over the missing pages into the speculative
    (O, l, m) of the q heads of KV head h, one missing page at a time."""
    O, l, m = (np.array(spec[0], float), np.array(spec[1], float), np.array(spec[2], float))
    for j in missing_pages(a_ids, p_ids):
        Oj, lj, mj = attend_pages(batch, b, h, [j], q)
        for g in range(batch.group):
            O[g], l[g], m[g] = merge((O[g], l[g], m[g]), (Oj[g], lj[g], mj[g]))
    return O, l, m


# --------------------------------------------------------------------------
# step 9: EMA predictor  (PRR section 3.1)
# --------------------------------------------------------------------------
def ema_predict(level, trend, gamma: float):
    """Predicted score of each block: level + gamma * trend."""
    return np.asarray(level, float) + gamma * np.asarray(trend, float)


def ema_update(is_true, level, trend, alpha: float, beta: float):
    """Both updates read the previous level: trend' = beta*(IS - level) +
    (1-beta)*trend, level' = alpha*IS + (1-alpha)*level."""
    is_true, level, trend = (np.asarray(x, float) for x in (is_true, level, trend))
    new_trend = beta * (is_true - level) + (1.0 - beta) * trend
    new_level = alpha * is_true + (1.0 - alpha) * level
    return new_level, new_trend


# --------------------------------------------------------------------------
# online predictor calibration  (PRR section 3.2 of the page = the paper's
# section 4.2: score-weighted hit rate H(theta; IS) over a prefill score
# trace, maximised over the printed 4 x 5 x 4 grid)
# --------------------------------------------------------------------------
CALIB_ALPHAS = (0.2, 0.4, 0.6, 0.8)
CALIB_BETAS = (0.1, 0.2, 0.3, 0.4, 0.5)
CALIB_GAMMAS = (0.0, 0.25, 0.5, 0.75)


def calibration_grid() -> list:
    """The 80 candidates (alpha, beta, gamma), alpha slowest, gamma fastest."""
    return [(a, b, g) for a in CALIB_ALPHAS for b in CALIB_BETAS for g in CALIB_GAMMAS]


def ema_step_f32(is_true, level, trend, alpha: float, beta: float):
    """ema_update in float32 with every product and sum rounded on its own,
    in the order trend' = beta*(IS - level) + (1-beta)*trend, level' =
    alpha*IS + (1-alpha)*level.  The calibration ranks pages by the
    prediction, so the reference takes that decision in the precision and
    rounding of the kernel (float32, no fused multiply-add)."""
    f = np.float32
    is_true, level, trend = (np.asarray(x, f) for x in (is_true, level, trend))
    a, b = f(alpha), f(beta)
    new_trend = b * (is_true - level) + (f(1) - b) * trend
    new_level = a * is_true + (f(1) - a) * level
    return new_level, new_trend


def ema_predict_f32(level, trend, gamma: float):
    """ema_predict in float32: level + (gamma * trend), each rounded."""
    f = np.float32
    return np.asarray(level, f) + f(gamma) * np.asarray(trend, f)


def hit_rate(pred_row, is_row, n_valid: int, k: int, m: int) -> float:
    """One term of H: the IS-weighted share of A = top-k(IS) covered by
    P = top-m(prediction), over the n_valid valid pages.  An empty A (or one
    of zero total weight) leaves nothing to miss: 1."""
    A = topk_pages(np.asarray(is_row, float), n_valid, k)
    P = topk_pages(np.asarray(pred_row, float), n_valid, m)
    w = np.asarray(is_row, float)
    den = float(w[A].sum())
    if len(A) == 0 or den == 0.0:
        return 1.0
    return float(w[np.intersect1d(P, A)].sum()) / den


def calibrate(trace, n_valid, k: int, m: int, candidates=None) -> np.ndarray:
    """H[u][c] for trace[T][units][N] (float32 scores of T consecutive steps).

    Per unit and candidate the EMA starts at level = IS_0, trend = 0; every
    later step phi is first predicted from the state so far, scored as
    hit_rate(pred_phi, IS_phi), then absorbed into the state.  H is the mean
    over the T - 1 predicted steps.  `candidates` (indices into
    calibration_grid()) restricts the columns computed; the rest are NaN."""
    trace = np.asarray(trace, np.float32)
    T, U, N = trace.shape
    grid = calibration_grid()
    cols = range(len(grid)) if candidates is None else candidates
    H = np.full((U, len(grid)), np.nan)
    for u in range(U):
        nv = int(n_valid[u])
        for c in cols:
            alpha, beta, gamma = grid[c]
            level, trend = trace[0, u].copy(), np.zeros(N, np.float32)
            acc = 0.0
            for phi in range(1, T):
                acc += hit_rate(ema_predict_f32(level, trend, gamma), trace[phi, u], nv, k, m)
                level, trend = ema_step_f32(trace[phi, u], level, trend, alpha, beta)
            H[u, c] = acc / (T - 1)
    return H


def best_candidate(H_row) -> int:
    """argmax over the candidates, the lowest index among equal maxima."""
    return int(np.argmax(np.asarray(H_row, float)))


def speculative_set(pred_row: np.ndarray, n_valid: int, a_size: int, delta: float) -> np.ndarray:
    """P = the floor(delta*|A|) pages with the highest prediction, ascending
    (PRR section 3.4: |P| is bounded by delta*|A|)."""
    return topk_pages(pred_row, n_valid, int(math.floor(delta * a_size)))


# --------------------------------------------------------------------------
# the composed decode steps (used for end-to-end checks and the CPU baseline)
# --------------------------------------------------------------------------
def quest_step(batch, k: int, q=None):
    """Score -> top-k -> sparse attention for one decode step."""
    scores = page_scores(batch, q=q)
    ids = select_topk(batch, scores, k)
    return scores, ids, sparse_decode(batch, ids, q)


# --------------------------------------------------------------------------
# block-sparse prefill  (LServe section 2.3: every T_Q x T_K tile is either
# skipped or computed as causal attention; section 3.3 / Figure 5: dense and
# streaming heads in one kernel; section 4.1: a streaming head keeps the
# Lambda mask of sink and local tokens)
# --------------------------------------------------------------------------
def prefill_keys(i: int, L: int, streaming: bool, sink: int, local: int) -> np.ndarray:
    """Keys query i attends to: j <= i (causal), and for a streaming head
    only the sink tokens j < sink and the local ones j > i - local (the
    decode rule with the sequence ending at i)."""
    j = np.arange(min(i + 1, L))
    if streaming:
        j = j[(j < sink) | (j > i - local)]
    return j


def prefill_attention(q, k, v, dtype: str, scale: float, streaming=None, sink: int = 0, local: int = 0):
    """(O[L][Hq][D], l[L][Hq], m[L][Hq]) of one sequence: q [L][Hq][D],
    k, v [L][Hkv][D] (stored format); q head hq reads KV head hq // G."""
    qf, kf, vf = (widen(x, dtype) for x in (q, k, v))
    L, Hq, D = qf.shape
    Hkv = kf.shape[1]
    G = Hq // Hkv
    O, l, m = np.zeros((L, Hq, D)), np.zeros((L, Hq)), np.full((L, Hq), NEG_INF)
    for hq in range(Hq):
        h = hq // G
        st = streaming is not None and bool(streaming[h])
        for i in range(L):
            j = prefill_keys(i, L, st, sink, local)
            O[i, hq], l[i, hq], m[i, hq] = attention(qf[i, hq], kf[j, h], vf[j, h], scale)
    return O, l, m


# --------------------------------------------------------------------------
# reusable page selector  (LServe section 4.3: the selector runs only at the
# start of each chunk of C consecutive decode tokens -- 4 by default -- and
# the chunk's later tokens reuse the first token's pages)
# --------------------------------------------------------------------------
def chunk_start(t: int, chunk: int) -> int:
    """The decode step whose selection step t uses."""
    return (t // chunk) * chunk


def reuse_decode(batch, q_trace, k: int, chunk: int):
    """For each step t of q_trace [T][B][Hq][D] (stored format): the pages
    selected for the query of step chunk_start(t), and the attention of step
    t's own query over them.  Returns ([ids per step], [(O, l, m) per step])."""
    ids_of, out_ids, outs = {}, [], []
    for t in range(len(q_trace)):
        s = chunk_start(t, chunk)
        if s not in ids_of:
            ids_of[s] = select_topk(batch, page_scores(batch, q=q_trace[s]), k)
        out_ids.append(ids_of[s])
        outs.append(sparse_decode(batch, ids_of[s], q_trace[t]))
    return out_ids, outs
