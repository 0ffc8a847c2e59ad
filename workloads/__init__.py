"""Seeded synthetic decode batches: the only code that both the oracle side and
the HIP side consume.

This module draws random numbers and lays them out in the paged KV format.
It computes nothing of the method itself: no page metadata, no scores, no
selection and no attention.  Every array is produced from a numpy
``SeedSequence``, so a batch is a pure function of its recipe and seed.

Storage conventions shared by both sides (they are the input format):

* ``k``/``v`` pool: ``[num_slots][n_kv_heads][page_size][head_dim]``, one
  slot per physical page, as in the single block pool of PSA's unified
  memory management (Progressive Sparse Attention, section 3.4) and the
  paged layout of LServe (section 3.2.1).
* ``page_table``: int32 ``[batch][max_pages]``; entry ``j`` is the slot that
  holds tokens ``[j*page_size, (j+1)*page_size)`` of that sequence, ``-1``
  past the last page that holds a token.
* ``q``: ``[batch][n_q_heads][head_dim]``; q head ``h`` belongs to KV head
  ``h // (n_q_heads // n_kv_heads)``.
* bf16 values are stored as their uint16 bit patterns, rounded from float32
  by round-to-nearest-even; fp32 values as float32.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Batch", "to_bf16_bits", "from_bf16_bits",
    "tiny_heavy", "quest_gqa", "lserve_hier", "psa_mha", "prr_trace",
    "random_batch", "append_stream", "score_trace", "query_drift", "prefill_inputs", "PREFILL_16K", "WORKLOADS", "make",
]


# --------------------------------------------------------------------------
# storage helpers (format conversion only)
# --------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _stored_as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    return (from_bf16_bits(x) if dtype == "bf16" else x).astype(np.float64)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclass
class Batch:
    """One decode step's inputs in the paged layout described above."""
    name: str
    dtype: str                 # "bf16" | "f32"
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int             # physical page (tokens per slot)
    logical_page: int          # selection granularity (divides page_size)
    max_pages: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    page_table: np.ndarray
    seq_lens: np.ndarray
    streaming: np.ndarray | None = None   # uint8 [n_kv_heads], 1 = streaming head
    sink: int = 0
    local: int = 0
    topk: int | None = None
    threshold: float | None = None
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def num_slots(self) -> int:
        return self.k.shape[0]

    @property
    def scale(self) -> np.float32:
        """Logit scale 1/sqrt(head_dim), rounded once to float32."""
        return np.float32(1.0 / math.sqrt(self.head_dim))

    def n_pages(self, b: int) -> int:
        return -(-int(self.seq_lens[b]) // self.page_size)


def _page_table(rng: np.random.Generator, seq_lens, page_size: int, max_pages: int,
                spare_slots: int = 0):
    """Random slot permutation; -1 past each sequence's last page."""
    B = len(seq_lens)
    used = [-(-int(L) // page_size) for L in seq_lens]
    n_slots = sum(used) + spare_slots
    perm = rng.permutation(n_slots).astype(np.int32)
    pt = np.full((B, max_pages), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        pt[b, :used[b]] = perm[o:o + used[b]]
        o += used[b]
    return pt, n_slots


def _scatter_unit(pool: np.ndarray, pt_row: np.ndarray, h: int, tokens: np.ndarray, page_size: int):
    """Write a unit's token-major [L][D] values into its slots."""
    L, D = tokens.shape
    full, rem = divmod(L, page_size)
    if full:
        pool[pt_row[:full], h] = tokens[:full * page_size].reshape(full, page_size, D)
    if rem:   # rows past the sequence end keep whatever the pool held
        pool[pt_row[full], h, :rem] = tokens[full * page_size:]


def _alloc_pool(n_slots, Hkv, P, D, dtype):
    return np.zeros((n_slots, Hkv, P, D), dtype=np.uint16 if dtype == "bf16" else np.float32)


def _unit_direction(qf64: np.ndarray, b: int, h: int, G: int) -> np.ndarray:
    """Unit vector along the sum of KV head h's q heads (a data direction)."""
    s = qf64[b, h * G:(h + 1) * G].sum(axis=0)
    return s / np.linalg.norm(s)


# --------------------------------------------------------------------------
# workload recipes
# --------------------------------------------------------------------------
def tiny_heavy(seed: int = 101, seq_len: int = 2048, page_size: int = 16, head_dim: int = 64,
               n_heavy: int = 6, topk: int = 8, threshold: float = 0.95) -> Batch:
    """Single query, single head, fp32: q, K, V ~ N(0,1); the keys of
    ``n_heavy`` pages (drawn without replacement) are ``0.5*q + N(0, 0.3^2)``."""
    rs, rq, rk, rv = (np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(4))
    N = -(-seq_len // page_size)
    pt, n_slots = _page_table(rs, [seq_len], page_size, N)
    q = rq.standard_normal((1, 1, head_dim), dtype=np.float32)
    K = rk.standard_normal((seq_len, head_dim), dtype=np.float32)
    V = rv.standard_normal((seq_len, head_dim), dtype=np.float32)
    heavy = np.sort(rs.choice(N, size=min(n_heavy, N), replace=False))
    for p in heavy:
        lo, hi = p * page_size, min((p + 1) * page_size, seq_len)
        K[lo:hi] = 0.5 * q[0, 0] + 0.3 * rs.standard_normal((hi - lo, head_dim), dtype=np.float32)
    k = _alloc_pool(n_slots, 1, page_size, head_dim, "f32")
    v = _alloc_pool(n_slots, 1, page_size, head_dim, "f32")
    _scatter_unit(k, pt[0], 0, K, page_size)
    _scatter_unit(v, pt[0], 0, V, page_size)
    return Batch("tiny_f32", "f32", 1, 1, 1, head_dim, page_size, page_size, N, q, k, v, pt,
                 np.array([seq_len], np.int32), topk=topk, threshold=threshold,
                 extra={"heavy_pages": heavy})


def quest_gqa(seed: int = 102, batch: int = 1, n_q_heads: int = 32, n_kv_heads: int = 8,
              head_dim: int = 128, seq_len: int = 32768, page_size: int = 16,
              budget_tokens: int = 4096, bias_frac: float = 0.02, cos: float = 0.4) -> Batch:
    """Quest-style GQA decode, bf16.  q, K, V ~ N(0,1).  In every (sequence,
    KV head), ``round(bias_frac*N)`` pages get keys
    ``|g| * (cos*u + sqrt(1-cos^2) * e_perp(g))`` with g ~ N(0, I), u the unit
    vector along the group's summed q heads and e_perp(g) the unit part of g
    orthogonal to u, so every such key has cosine ``cos`` with u."""
    G = n_q_heads // n_kv_heads
    N = -(-seq_len // page_size)
    ss = np.random.SeedSequence(seed).spawn(2 + batch * n_kv_heads)
    rs, rq = np.random.default_rng(ss[0]), np.random.default_rng(ss[1])
    pt, n_slots = _page_table(rs, [seq_len] * batch, page_size, N)
    q = to_bf16_bits(rq.standard_normal((batch, n_q_heads, head_dim), dtype=np.float32))
    qf = _stored_as_f64(q, "bf16")
    k = _alloc_pool(n_slots, n_kv_heads, page_size, head_dim, "bf16")
    v = _alloc_pool(n_slots, n_kv_heads, page_size, head_dim, "bf16")
    n_bias = int(round(bias_frac * N))
    biased = np.zeros((batch, n_kv_heads, n_bias), np.int64)

    def unit(u):
        b, h = divmod(u, n_kv_heads)
        r = np.random.default_rng(ss[2 + u])
        K = r.standard_normal((seq_len, head_dim), dtype=np.float32)
        V = r.standard_normal((seq_len, head_dim), dtype=np.float32)
        pages = np.sort(r.choice(N, size=n_bias, replace=False))
        uvec = _unit_direction(qf, b, h, G)
        for p in pages:
            lo, hi = p * page_size, min((p + 1) * page_size, seq_len)
            g = K[lo:hi].astype(np.float64)
            par = g @ uvec
            perp = g - par[:, None] * uvec[None, :]
            perp /= np.linalg.norm(perp, axis=1, keepdims=True)
            K[lo:hi] = (np.linalg.norm(g, axis=1, keepdims=True)
                        * (cos * uvec[None, :] + math.sqrt(1 - cos * cos) * perp)).astype(np.float32)
        _scatter_unit(k, pt[b], h, to_bf16_bits(K).reshape(seq_len, head_dim), page_size)
        _scatter_unit(v, pt[b], h, to_bf16_bits(V).reshape(seq_len, head_dim), page_size)
        biased[b, h] = pages

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(unit, range(batch * n_kv_heads)))
    return Batch("quest_gqa", "bf16", batch, n_q_heads, n_kv_heads, head_dim, page_size, page_size,
                 N, q, k, v, pt, np.full(batch, seq_len, np.int32),
                 topk=budget_tokens // page_size, extra={"biased_pages": biased})


def lserve_hier(seed: int = 103, batch: int = 4, n_q_heads: int = 32, n_kv_heads: int = 8,
                head_dim: int = 128, seq_len: int = 131072, page_size: int = 64,
                logical_page: int = 16, budget_tokens: int = 4096, n_streaming: int | None = None,
                sink: int = 128, local: int = 256, zipf: float = 1.1, shift: float = 8.0) -> Batch:
    """LServe hierarchical paging, bf16.  Half of the KV heads (a seeded
    choice shared by every sequence) are streaming heads.  For dense heads the
    logical pages get a random rank permutation r_j and relevance
    ``w_j = r_j**-zipf``; every key of logical page j is ``z + shift*w_j*u``
    with z ~ N(0, I) and u the unit vector along the group's summed q heads.
    Streaming-head keys and all values are N(0, 1)."""
    G = n_q_heads // n_kv_heads
    N = -(-seq_len // page_size)
    ss = np.random.SeedSequence(seed).spawn(2 + batch * n_kv_heads)
    rs, rq = np.random.default_rng(ss[0]), np.random.default_rng(ss[1])
    pt, n_slots = _page_table(rs, [seq_len] * batch, page_size, N)
    if n_streaming is None:
        n_streaming = n_kv_heads // 2
    streaming = np.zeros(n_kv_heads, np.uint8)
    streaming[rs.choice(n_kv_heads, size=n_streaming, replace=False)] = 1
    q = to_bf16_bits(rq.standard_normal((batch, n_q_heads, head_dim), dtype=np.float32))
    qf = _stored_as_f64(q, "bf16")
    k = _alloc_pool(n_slots, n_kv_heads, page_size, head_dim, "bf16")
    v = _alloc_pool(n_slots, n_kv_heads, page_size, head_dim, "bf16")
    Nl = -(-seq_len // logical_page)

    def unit(u):
        b, h = divmod(u, n_kv_heads)
        r = np.random.default_rng(ss[2 + u])
        K = r.standard_normal((seq_len, head_dim), dtype=np.float32)
        V = r.standard_normal((seq_len, head_dim), dtype=np.float32)
        if not streaming[h]:
            ranks = r.permutation(Nl).astype(np.float64) + 1.0
            w = ranks ** (-zipf)
            uvec = _unit_direction(qf, b, h, G)
            tok_w = np.repeat(w, logical_page)[:seq_len]
            K += (shift * tok_w[:, None] * uvec[None, :]).astype(np.float32)
        _scatter_unit(k, pt[b], h, to_bf16_bits(K).reshape(seq_len, head_dim), page_size)
        _scatter_unit(v, pt[b], h, to_bf16_bits(V).reshape(seq_len, head_dim), page_size)

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(unit, range(batch * n_kv_heads)))
    return Batch("lserve_hier", "bf16", batch, n_q_heads, n_kv_heads, head_dim, page_size, logical_page,
                 N, q, k, v, pt, np.full(batch, seq_len, np.int32), streaming=streaming,
                 sink=sink, local=local, topk=budget_tokens // page_size)


def psa_mha(seed: int = 104, batch: int = 8, n_heads: int = 32, head_dim: int = 128,
            seq_len: int = 65536, page_size: int = 16, threshold: float = 0.95,
            hot_range=(20, 300), hot_mass: float = 0.97) -> Batch:
    """PSA progressive selection, MHA, bf16.  Per (sequence, head):
    ``n_h = round(exp(U[ln lo, ln hi]))`` hot pages; every key of a hot page is
    ``z + (mu_h*sqrt(d)/|q|) * q/|q|`` with ``mu_h = ln(hot_mass*(N-n_h) /
    ((1-hot_mass)*n_h))``, which shifts its logit by mu_h so the hot pages hold
    about ``hot_mass`` of the softmax mass.  Other keys and all values N(0,1)."""
    N = -(-seq_len // page_size)
    ss = np.random.SeedSequence(seed).spawn(2 + batch * n_heads)
    rs, rq = np.random.default_rng(ss[0]), np.random.default_rng(ss[1])
    pt, n_slots = _page_table(rs, [seq_len] * batch, page_size, N)
    q = to_bf16_bits(rq.standard_normal((batch, n_heads, head_dim), dtype=np.float32))
    qf = _stored_as_f64(q, "bf16")
    k = _alloc_pool(n_slots, n_heads, page_size, head_dim, "bf16")
    v = _alloc_pool(n_slots, n_heads, page_size, head_dim, "bf16")
    n_hot = np.zeros((batch, n_heads), np.int64)
    lo_h, hi_h = hot_range

    def unit(u):
        b, h = divmod(u, n_heads)
        r = np.random.default_rng(ss[2 + u])
        K = r.standard_normal((seq_len, head_dim), dtype=np.float32)
        V = r.standard_normal((seq_len, head_dim), dtype=np.float32)
        nh = int(round(math.exp(r.uniform(math.log(lo_h), math.log(hi_h)))))
        nh = max(1, min(nh, N - 1))
        hot = r.choice(N, size=nh, replace=False)
        mu = math.log(hot_mass * (N - nh) / ((1 - hot_mass) * nh))
        qv = qf[b, h]
        qn = np.linalg.norm(qv)
        shift = (mu * math.sqrt(head_dim) / qn) * (qv / qn)
        for p in hot:
            lo, hi = p * page_size, min((p + 1) * page_size, seq_len)
            K[lo:hi] += shift.astype(np.float32)[None, :]
        _scatter_unit(k, pt[b], h, to_bf16_bits(K).reshape(seq_len, head_dim), page_size)
        _scatter_unit(v, pt[b], h, to_bf16_bits(V).reshape(seq_len, head_dim), page_size)
        n_hot[b, h] = nh

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(unit, range(batch * n_heads)))
    return Batch("psa_mha", "bf16", batch, n_heads, n_heads, head_dim, page_size, page_size, N,
                 q, k, v, pt, np.full(batch, seq_len, np.int32), threshold=threshold,
                 extra={"n_hot": n_hot})


def prr_trace(seed: int = 105, batch: int = 1, n_q_heads: int = 32, n_kv_heads: int = 2,
              head_dim: int = 128, seq_len: int = 524288, page_size: int = 16, topk: int = 2048,
              steps: int = 64, theta=(0.05, 0.35), ema=(0.6, 0.3, 0.25), delta: float = 1.0) -> Batch:
    """PRR speculate+repair trace, bf16.  K, V ~ N(0,1).  The query drifts over
    ``steps`` decode steps: ``q_t = cos(th_t) q_{t-1} + sin(th_t) xi_t`` with
    xi_t ~ N(0, I) per head and th_t ramped linearly over ``theta``; the
    recursion runs in float64 and each step's query is stored rounded to bf16.
    ``extra['q_trace']`` is ``[steps][batch][n_q_heads][head_dim]``; ``q`` is
    step 0."""
    N = -(-seq_len // page_size)
    ss = np.random.SeedSequence(seed).spawn(2 + batch * n_kv_heads)
    rs, rq = np.random.default_rng(ss[0]), np.random.default_rng(ss[1])
    pt, n_slots = _page_table(rs, [seq_len] * batch, page_size, N)
    qcur = rq.standard_normal((batch, n_q_heads, head_dim))
    trace = [to_bf16_bits(qcur.astype(np.float32))]
    for t in range(1, steps):
        th = theta[0] + (theta[1] - theta[0]) * (t - 1) / max(1, steps - 2)
        xi = rq.standard_normal((batch, n_q_heads, head_dim))
        qcur = math.cos(th) * qcur + math.sin(th) * xi
        trace.append(to_bf16_bits(qcur.astype(np.float32)))
    q_trace = np.stack(trace)
    k = _alloc_pool(n_slots, n_kv_heads, page_size, head_dim, "bf16")
    v = _alloc_pool(n_slots, n_kv_heads, page_size, head_dim, "bf16")

    def unit(u):
        b, h = divmod(u, n_kv_heads)
        r = np.random.default_rng(ss[2 + u])
        K = r.standard_normal((seq_len, head_dim), dtype=np.float32)
        V = r.standard_normal((seq_len, head_dim), dtype=np.float32)
        _scatter_unit(k, pt[b], h, to_bf16_bits(K).reshape(seq_len, head_dim), page_size)
        _scatter_unit(v, pt[b], h, to_bf16_bits(V).reshape(seq_len, head_dim), page_size)

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(unit, range(batch * n_kv_heads)))
    return Batch("prr_trace", "bf16", batch, n_q_heads, n_kv_heads, head_dim, page_size, page_size, N,
                 q_trace[0], k, v, pt, np.full(batch, seq_len, np.int32), topk=topk,
                 extra={"q_trace": q_trace, "ema": ema, "delta": delta, "steps": steps})


def random_batch(seed: int, seq_lens, n_q_heads: int = 4, n_kv_heads: int = 2, head_dim: int = 128,
                 page_size: int = 16, logical_page: int | None = None, dtype: str = "bf16",
                 max_pages: int | None = None, spare_slots: int = 3, streaming=None,
                 sink: int = 0, local: int = 0, dup_pages: int = 0) -> Batch:
    """Plain N(0,1) batch with ragged sequence lengths for edge-case tests.
    ``dup_pages`` > 0 copies the keys of page 0 into that many other pages of
    every (sequence, KV head), which creates exact score ties."""
    seq_lens = np.asarray(seq_lens, np.int32)
    B = len(seq_lens)
    if max_pages is None:
        max_pages = max(1, max(-(-int(L) // page_size) for L in seq_lens))
    ss = np.random.SeedSequence(seed).spawn(2 + B * n_kv_heads)
    rs, rq = np.random.default_rng(ss[0]), np.random.default_rng(ss[1])
    pt, n_slots = _page_table(rs, seq_lens, page_size, max_pages, spare_slots)
    q = _store(rq.standard_normal((B, n_q_heads, head_dim), dtype=np.float32), dtype)
    k = _alloc_pool(n_slots, n_kv_heads, page_size, head_dim, dtype)
    v = _alloc_pool(n_slots, n_kv_heads, page_size, head_dim, dtype)
    # spare slots hold garbage that must never be read
    k[:] = _store(rs.standard_normal(k.shape, dtype=np.float32) * 1e3, dtype)
    v[:] = _store(rs.standard_normal(v.shape, dtype=np.float32) * 1e3, dtype)
    for u in range(B * n_kv_heads):
        b, h = divmod(u, n_kv_heads)
        L = int(seq_lens[b])
        r = np.random.default_rng(ss[2 + u])
        K = r.standard_normal((L, head_dim), dtype=np.float32)
        V = r.standard_normal((L, head_dim), dtype=np.float32)
        n = -(-L // page_size)
        if dup_pages and n > 1:
            for p in r.choice(np.arange(1, n), size=min(dup_pages, n - 1), replace=False):
                lo, hi = p * page_size, min((p + 1) * page_size, L)
                K[lo:hi] = K[0:hi - lo]
        _scatter_unit(k, pt[b], h, _store(K, dtype).reshape(L, head_dim), page_size)
        _scatter_unit(v, pt[b], h, _store(V, dtype).reshape(L, head_dim), page_size)
    st = None if streaming is None else np.asarray(streaming, np.uint8)
    return Batch("random", dtype, B, n_q_heads, n_kv_heads, head_dim, page_size,
                 logical_page or page_size, max_pages, q, k, v, pt, seq_lens, streaming=st,
                 sink=sink, local=local)


def append_stream(seed: int, batch: int, n_kv_heads: int, head_dim: int, steps: int, dtype: str = "bf16"):
    """K and V rows of `steps` newly generated tokens per sequence, N(0,1),
    stored format: two arrays [steps][batch][n_kv_heads][head_dim]."""
    rk, rv = (np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(2))
    shape = (steps, batch, n_kv_heads, head_dim)
    return (_store(rk.standard_normal(shape, dtype=np.float32), dtype),
            _store(rv.standard_normal(shape, dtype=np.float32), dtype))


def score_trace(seed: int, steps: int, units: int, n: int, mean: float = 100.0, spread: float = 3.0,
                drift: float = 0.5, noise: float = 0.3, ties: bool = False) -> np.ndarray:
    """Page-score trace [steps][units][n] (float32) standing in for the
    scores of consecutive prefill steps: every page has a base level
    N(mean, spread), a constant drift N(0, drift) per step and fresh N(0,
    noise) noise at every step.  ``ties`` rounds the scores to integers,
    which makes equal scores common."""
    rb, rd, rn = (np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3))
    base = rb.normal(mean, spread, (units, n))
    vel = rd.normal(0.0, drift, (units, n))
    phi = np.arange(steps, dtype=np.float64)[:, None, None]
    tr = base[None] + vel[None] * phi + rn.normal(0.0, noise, (steps, units, n))
    if ties:
        tr = np.round(tr)
    return tr.astype(np.float32)


def query_drift(seed: int, q0: np.ndarray, steps: int, theta: float, dtype: str = "bf16") -> np.ndarray:
    """Queries of `steps` consecutive decode tokens starting from q0 (stored
    format [B][Hq][D]): q_t = cos(theta) q_{t-1} + sin(theta) xi_t with xi_t
    ~ N(0, I), the recursion in float64, each step stored rounded.  Returns
    [steps][B][Hq][D]; step 0 is q0 itself."""
    rng = np.random.default_rng(seed)
    cur = _stored_as_f64(q0, dtype)
    out = [np.array(q0, copy=True)]
    for _ in range(1, steps):
        cur = math.cos(theta) * cur + math.sin(theta) * rng.standard_normal(cur.shape)
        out.append(_store(cur.astype(np.float32), dtype))
    return np.stack(out)


def prefill_inputs(seed: int, L: int, n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: str = "bf16",
                   q_gain: float = 1.0):
    """q [L][n_q_heads][D], k, v [L][n_kv_heads][D] of one prompt (stored
    format), N(0, 1); q is multiplied by q_gain (larger gains give peakier
    attention)."""
    rq, rk, rv = (np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3))
    q = rq.standard_normal((L, n_q_heads, head_dim), dtype=np.float32) * np.float32(q_gain)
    k = rk.standard_normal((L, n_kv_heads, head_dim), dtype=np.float32)
    v = rv.standard_normal((L, n_kv_heads, head_dim), dtype=np.float32)
    return _store(q, dtype), _store(k, dtype), _store(v, dtype)


# The block-sparse prefill workload: one 16K-token prompt, 32 q / 8 KV heads,
# head_dim 128, bf16, every other KV head streaming (sink 128, local 256
# tokens): the LServe shape of the decode workload, at prefill.
PREFILL_16K = {"seed": 106, "L": 16384, "n_q_heads": 32, "n_kv_heads": 8, "head_dim": 128,
               "streaming": np.array([0, 1, 0, 1, 0, 1, 0, 1], np.uint8), "sink": 128, "local": 256}


# Full-size workloads, by what they are.
WORKLOADS = {
    "tiny_f32": tiny_heavy,          # 1 query, 1 head, d=64, 2048 tokens, top-8 and PSA 0.95
    "quest_gqa_32k": quest_gqa,      # B=1, 32q/8kv, d=128, 32K tokens, top-256 pages
    "lserve_hier_128k": lserve_hier,  # B=4, 32q/8kv, 128K tokens, 64/16 paging, streaming heads
    "psa_mha_64k": psa_mha,          # B=8, 32 heads MHA, 64K tokens, PSA threshold 0.95
    "prr_512k": prr_trace,           # B=1, 32q/2kv, 512K tokens, top-2048, 64-step trace
}


def make(name: str, **overrides) -> Batch:
    return WORKLOADS[name](**overrides)
