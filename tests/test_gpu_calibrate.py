"""GPU parity of dsa_prr_calibrate against the oracle's calibration.

Both sides compute the EMA prediction in float32 with the same rounding
steps, so the speculative sets P and the exact sets A are identical and
only the weighted sums differ by rounding: H agrees to 1e-5 (absolute, H is
a share in [0, 1]) for every candidate, and the chosen candidate is one the
oracle scores within that tolerance of its best (exactly the oracle's
argmax when that maximum is clear by more).  Cases cover every register
layout of the kernel (state in registers; state in the workspace), ragged
and empty valid ranges, budgets above the valid count and zero, integer
traces with many equal scores, and the 32768-page PRR shape with sampled
candidates."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import np_

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _check(H_gpu, best_gpu, H_ref, cols):
    for u in range(H_ref.shape[0]):
        d = np.abs(H_gpu[u, cols] - H_ref[u, cols]).max()
        assert d <= TOL, f"unit {u}: max |dH| = {d:.3g}"
        assert np.all((H_gpu[u] >= 0) & (H_gpu[u] <= 1 + 1e-6))
        b = int(best_gpu[u])
        assert H_gpu[u, b] == H_gpu[u].max() and np.all(H_gpu[u, :b] < H_gpu[u, b]), f"unit {u}: best not the first max"
        ref = H_ref[u, cols]
        if b in cols:
            assert H_ref[u, b] >= ref.max() - TOL, f"unit {u}: candidate {b} is not a best one"
        top = np.sort(ref)[::-1]
        if len(top) > 1 and top[0] - top[1] > 4 * TOL and len(cols) == 80:
            assert b == int(np.argmax(ref)), f"unit {u}: clear best {int(np.argmax(ref))}, got {b}"


@pytest.mark.parametrize("T,units,N,n_valid,k,m,ties", [
    (10, 3, 700, [700, 500, 0], 64, 64, False),      # 4 per thread, state in registers
    (10, 3, 700, [700, 451, 30], 64, 48, True),       # integer scores, P smaller than A, n_valid < k
    (8, 2, 5000, [5000, 4097], 300, 300, False),      # 8 per thread, 16 waves
    (6, 2, 12000, [12000, 9000], 800, 1000, False),   # 16 per thread: state in the workspace
    (5, 2, 20000, [20000, 19999], 1000, 0, False),     # 32 per thread; empty P
    (5, 1, 300, [300], 0, 20, False),                  # empty A: every step counts 1
])
def test_calibrate_matches_oracle(gpu_lib, T, units, N, n_valid, k, m, ties):
    dsa = gpu_lib
    _banner(f"prr_calibrate T={T} units={units} N={N} n_valid={n_valid} k={k} m={m} ties={ties}")
    tr = wl.score_trace(71 + N, T, units, N, ties=ties)
    nv = np.asarray(n_valid, np.int32)
    H, best = dsa.prr_calibrate(torch.from_numpy(tr).cuda(), torch.from_numpy(nv).cuda(), k, m)
    torch.cuda.synchronize()
    H, best = np_(H), np_(best)
    ref = oracle.calibrate(tr, nv, k, m)
    _check(H, best, ref, list(range(80)))
    if m == 0:
        assert np.all(H[np.asarray(n_valid) > 0] == 0.0)
    if k == 0:
        assert np.all(H == 1.0)


def test_calibrate_prr_shape_sampled(gpu_lib):
    """32768 pages, 2 KV heads, 32 steps, |A| = |P| = 2048: every candidate
    in [0, 1]; the oracle recomputes 6 spread-out candidates and the one the
    kernel chose."""
    dsa = gpu_lib
    _banner("prr_calibrate 32768 pages x 2 units x 32 steps")
    T, U, N, k = 32, 2, 32768, 2048
    tr = wl.score_trace(75, T, U, N)
    nv = np.full(U, N, np.int32)
    H, best = dsa.prr_calibrate(torch.from_numpy(tr).cuda(), torch.from_numpy(nv).cuda(), k, k)
    torch.cuda.synchronize()
    H, best = np_(H), np_(best)
    cols = sorted({0, 19, 38, 57, 76, 79, *[int(b) for b in best]})
    ref = oracle.calibrate(tr, nv, k, k, candidates=cols)
    _check(H, best, ref, cols)
