"""The pins must be able to fail: each case plants one plausible mistake in a
temporary copy of the oracle (a dropped term, a wrong index or operand, an
off-by-one) and checks that the pin suite rejects it.  CPU only; the real
oracle is never modified."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("np.maximum(qbar * kmax, qbar * kmin)", "np.maximum(qbar * kmax, qbar * kmax)"),
    ("mean(axis=2)", "sum(axis=2)"),
    ("phys[b, h, j] = logical[b, h, j].max()", "phys[b, h, j] = logical[b, h, j].mean()"),
    ("idx[np.lexsort((idx, -scores_row[:n_valid]))]", "idx[np.lexsort((-idx, -scores_row[:n_valid]))]"),
    ("new_trend = beta * (is_true - level)", "new_trend = beta * (is_true - level) * 1.01"),
    ("mult = 1.0 if stop_mode == 0 else float(n_left)", "mult = 1.0 if stop_mode == 0 else float(n_left + 1)"),
    ("w1 = math.exp(m1 - m) * l1", "w1 = math.exp(m1 - m)"),
    ("sub.min(axis=0)", "sub[1:].min(axis=0) if len(sub) > 1 else sub.min(axis=0)"),
    ("keep = (t < batch.sink) | (t >= L - batch.local)", "keep = (t < batch.sink) | (t > L - batch.local)"),
    ("s = scale * (keys @ qh)", "s = (keys @ qh)"),
    ("[:max(0, k)])", "[:max(0, k - 1)])"),
    ("lnAS_min = min(lnAS_min, float(lnAS_blk))\n        n_left -= 1\n        visited",
     "lnAS_min = min(lnAS_min, float(lnAS_acc))\n        n_left -= 1\n        visited"),
    ("new_level = alpha * is_true + (1.0 - alpha) * level",
     "new_level = alpha * is_true + (1.0 - alpha) * new_trend"),
    ("return np.asarray(level, float) + gamma * np.asarray(trend, float)",
     "return np.asarray(level, float) + np.asarray(trend, float)"),
    ("set(range(max(0, L - local), L))", "set(range(max(0, L - local + page_size), L))"),
    ("int(math.floor(delta * a_size))", "int(math.ceil(delta * a_size))"),
    ("out.k[slot, :, p % P] = k_new[b]", "out.k[slot, :, (p + 1) % P] = k_new[b]"),
    ("out.v[slot, :, p % P] = v_new[b]", "out.v[slot, :, p % P] = k_new[b]"),
    ("if p < 0 or j >= batch.max_pages:", "if p < 0 or j > batch.max_pages:"),
    ("out.seq_lens[b] = p + 1", "out.seq_lens[b] = p + 1 if p % P else p"),
    ("H[u, c] = acc / (T - 1)", "H[u, c] = acc / T"),
    ("j = np.arange(min(i + 1, L))", "j = np.arange(min(i, L))"),
    ("j = j[(j < sink) | (j > i - local)]", "j = j[(j < sink) | (j >= i - local)]"),
    ("return (t // chunk) * chunk", "return t - t % chunk + (1 if t % chunk else 0)"),
    ("outs.append(sparse_decode(batch, ids_of[s], q_trace[t]))", "outs.append(sparse_decode(batch, ids_of[s], q_trace[s]))"),
    ("for phi in range(1, T):\n                acc", "for phi in range(2, T):\n                acc"),
    ("return float(w[np.intersect1d(P, A)].sum()) / den", "return float(w[np.union1d(P, A)].sum()) / den"),
    ("new_trend = b * (is_true - level) + (f(1) - b) * trend", "new_trend = b * (is_true - level) + (f(1) - a) * trend"),
    ("return np.asarray(level, f) + f(gamma) * np.asarray(trend, f)", "return np.asarray(level, f) + np.asarray(trend, f)"),
    ("A = topk_pages(np.asarray(is_row, float), n_valid, k)\n    P = topk_pages(np.asarray(pred_row, float), n_valid, m)",
     "A = topk_pages(np.asarray(is_row, float), n_valid, k)\n    P = topk_pages(np.asarray(pred_row, float), n_valid, k)"),
]


@pytest.fixture(scope="module")
def sandbox(tmp_path_factory):
    d = tmp_path_factory.mktemp("mut")
    for sub in ("tests", "workloads"):
        shutil.copytree(os.path.join(ROOT, sub), d / sub,
                        ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py"))
    (d / "oracle").mkdir()
    return d


@pytest.mark.parametrize("before,after", MUTATIONS, ids=[f"m{i}" for i in range(len(MUTATIONS))])
def test_planted_mistake_is_caught(sandbox, before, after):
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert src.count(before) >= 1, before
    (sandbox / "oracle" / "__init__.py").write_text(src.replace(before, after))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=sandbox, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0, f"pins accepted a planted mistake: {after!r}"
