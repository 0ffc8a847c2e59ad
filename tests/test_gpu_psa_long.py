"""GPU parity of PSA's progressive selection (PSA, section 3.2) on rows of
up to 65536 pages and on score rows built to drive every branch of the
per-round pick: the linear first pass, key-shift passes, equal keys resolved
by index, candidate sets taken whole, many rounds.  Each case runs the
selection on the given float32 score rows and the oracle walks the same
values (stop count, rank order, attention over the visited pages)."""
import functools

import numpy as np
import pytest

import workloads as wl
from parity_util import check_psa, to_device

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[case] {msg}", flush=True)


@functools.lru_cache(maxsize=2)
def _batch(seq_lens, G, D, seed):
    return wl.random_batch(seed, list(seq_lens), n_q_heads=G, n_kv_heads=1, head_dim=D, page_size=16)


# ---------------------------------------------------------------- long rows
@pytest.mark.parametrize("n_pages,G,second", [(65536, 1, 20001), (65536, 2, 0), (32768, 1, 0)])
def test_psa_long_rows(gpu_lib, n_pages, G, second):
    """Rows at the capacity (65536 pages) and half of it, with a ragged last
    page; the printed rule stops within the first round, the remaining-pages
    rule and threshold 1 walk tens of thousands of pages over hundreds of
    rounds.  The optional second sequence is shorter than the page table."""
    dsa = gpu_lib
    lens = (16 * n_pages - 5,) + ((16 * second + 7,) if second else ())
    _banner(f"psa long rows pages={n_pages} G={G} lens={lens}")
    bt = _batch(lens, G, 64, 401 + G)
    q, kv, _ = to_device(dsa, bt)
    import oracle
    s32 = oracle.page_scores(bt).astype(np.float32)
    for thr, mode in ((0.95, 0), (0.95, 1), (1.0, 0)):
        _banner(f"  thr={thr} mode={mode}")
        cnt = check_psa(dsa, bt, q, kv, s32, thr, mode, f"long {n_pages} G={G} thr={thr} mode={mode}")
        print(f"    visited {cnt.ravel().tolist()}", flush=True)


# ---------------------------------------------------------------- score patterns
def _pattern(name, n, rng):
    if name == "normal":
        return rng.standard_normal(n)
    if name == "const":          # one key: the index decides every rank
        return np.full(n, 2.5)
    if name == "two":            # two keys
        return rng.integers(0, 2, n).astype(np.float64)
    if name == "int":            # many ties
        return np.round(rng.standard_normal(n) * 3.0)
    if name == "outliers":       # the linear map puts nearly every page in one bucket
        x = rng.standard_normal(n)
        x[rng.choice(n, 5, replace=False)] = 1e30
        x[rng.choice(n, 3, replace=False)] = -1e30
        return x
    if name == "neginf":
        x = rng.standard_normal(n)
        x[rng.random(n) < 0.3] = -np.inf
        return x
    if name == "ulp":            # keys less than 2048 apart: exact buckets at once
        bits = np.int64(np.float32(1.0).view(np.int32)) + rng.integers(0, 1000, n)
        return bits.astype(np.int32).view(np.float32).astype(np.float64)
    if name == "span":           # value span overflows float: shift map from the start
        return rng.uniform(-3e38, 3e38, n)
    if name == "desc":           # rank order = index order
        return np.linspace(10.0, -10.0, n)
    if name == "zeros":          # -0 and +0 are equal keys
        x = np.where(rng.random(n) < 0.5, -0.0, 0.0)
        x[rng.choice(n, 7, replace=False)] = 1.0
        return x
    raise ValueError(name)


PATTERNS = ["normal", "const", "two", "int", "outliers", "neginf", "ulp", "span", "desc", "zeros"]


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("n_pages,G", [(3000, 1), (12000, 1), (12000, 2)])
def test_psa_score_patterns(gpu_lib, n_pages, G, pattern):
    dsa = gpu_lib
    _banner(f"psa pattern={pattern} pages={n_pages} G={G}")
    lens = (16 * n_pages - 9, 16 * (n_pages // 3) + 1)
    bt = _batch(lens, G, 64, 411 + G)
    q, kv, _ = to_device(dsa, bt)
    rng = np.random.default_rng(1000 * PATTERNS.index(pattern) + n_pages + G)
    s = np.stack([_pattern(pattern, bt.max_pages, rng) for _ in range(bt.batch)])[:, None, :]
    s32 = s.astype(np.float32)
    cases = [(0.95, 0), (0.6, 1)]
    if n_pages <= 3000 or pattern in ("const", "int"):
        cases.append((1.0, 0))
    for thr, mode in cases:
        check_psa(dsa, bt, q, kv, s32, thr, mode, f"pattern {pattern} pages={n_pages} G={G} thr={thr} mode={mode}")
