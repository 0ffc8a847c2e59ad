"""GPU runs of the host policies over the kernels: PRR's offline profile of
the speculation budget (section 3.4) and PSA's zero-copy notification of
the host (section 3.3)."""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from parity_util import np_, to_device

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def test_delta_profile_gives_a_table_the_decoder_uses(gpu_lib):
    dsa = gpu_lib
    from dynamic_sparse_attention_page_amd.prr import DELTA_GRID, PRRDecoder, profile_delta_table
    _banner("PRR delta profile, 4K and 8K contexts")
    table, report = profile_delta_table(contexts=(4096, 8192), reps=3)
    assert [c for c, _ in table.entries] == [4096, 8192]
    for c, d in table.entries:
        assert d in DELTA_GRID
        r = report[c]
        assert r["select_us"] > 0 and all(v > 0 for v in r["spec_us"].values())
        fits = [float(x) for x, v in r["spec_us"].items() if v <= r["select_us"]]
        assert d == (max(fits) if fits else min(DELTA_GRID))
    bt = wl.random_batch(91, [8192], n_q_heads=8, n_kv_heads=2, head_dim=128, page_size=16)
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, 16)
    dec = PRRDecoder(kv, meta, 8, 32, 0.6, 0.3, 0.25, delta_table=table, context_tokens=8192)
    assert dec.k_spec == max(1, int(math.floor(table.lookup(8192) * 32)))


def test_signal_host_delivers_psa_counts_without_sync(gpu_lib):
    dsa = gpu_lib
    _banner("PSA counts through the pinned host signal")
    bt = wl.random_batch(92, [900, 300, 2000], n_q_heads=4, n_kv_heads=2, head_dim=128, page_size=16)
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, 16)
    sc = dsa.page_score(q, kv, meta, 16)
    host = torch.zeros(bt.batch * bt.n_kv_heads, dtype=torch.int32, pin_memory=True)
    flag = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    for seq, thr in ((5, 0.9), (6, 0.99)):
        ids, cnt, O, l, m = dsa.page_select_progressive(q, kv, sc, thr, 0)
        dsa.signal_host(cnt.view(-1), host, flag, seq)
        assert dsa.wait_host_flag(flag, seq, timeout_s=20.0), "flag never arrived"
        seen = host.numpy().copy()
        torch.cuda.synchronize()
        assert np.array_equal(seen, np_(cnt).reshape(-1)), f"seq {seq}: host values differ from the counts"
        assert np.all(seen >= 1)
