"""dsa_psa_decode (page criticality, LServe section 4.2, then PSA's
progressive selection, section 3.2, in one call) against the two separate
calls on the same inputs.  With at least as many (sequence, KV head) rows as
the GPU has CUs and rows of up to 8192 pages the call runs one fused launch
whose scores are computed operation for operation like page_score's, so its
scores, visited pages, counts and (O, l, m) must equal the two calls' bit
for bit; sampled rows are also checked against the oracle.  With fewer rows
it runs the two calls itself."""
import numpy as np
import pytest
import torch

import workloads as wl
from parity_util import check_psa_result, np_, to_device

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _compare(dsa, bt, q, kv, meta, thr, mode, what, st=None):
    scale = float(bt.scale)
    s_ref = dsa.page_score(q, kv, meta, streaming=st)
    ref = dsa.page_select_progressive(q, kv, s_ref, thr, mode, scale, streaming=st)
    got = dsa.psa_decode(q, kv, meta, thr, mode, scale, streaming=st)
    torch.cuda.synchronize()
    assert torch.equal(got[0], s_ref), f"{what}: scores differ"
    for name, a, b in zip(("ids", "counts", "O", "l", "m"), got[1:], ref):
        assert torch.equal(a, b), f"{what}: {name} differ"
    return got


CASES = [  # G, D, dtype, P, max_pages (None: the longest sequence's)
    (1, 128, "bf16", 16, None),
    (1, 128, "bf16", 16, 6000),    # rows held 8 per thread
    (2, 64, "bf16", 16, None),
    (4, 128, "bf16", 64, None),
    (2, 64, "bf16", 16, 7000),     # 8-wave rows streamed from LDS
    (1, 64, "f32", 16, None),
]


@pytest.mark.parametrize("G,D,dtype,P,max_pages", CASES)
def test_psa_decode_fused_matches_two_calls(gpu_lib, G, D, dtype, P, max_pages):
    dsa = gpu_lib
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    Hkv = 32
    B = max(8, -(-n_cu // Hkv))            # enough rows for the fused launch
    _banner(f"psa_decode fused G={G} D={D} {dtype} P={P} max_pages={max_pages} rows={B * Hkv}")
    rng = np.random.default_rng(5 + G + D)
    lens = [0, 5, P * 3 + 1] + [int(x) for x in rng.integers(P * 40, P * 90, size=B - 3)]
    bt = wl.random_batch(800 + G, lens, n_q_heads=Hkv * G, n_kv_heads=Hkv, head_dim=D, page_size=P, dtype=dtype,
                         max_pages=max_pages, dup_pages=2)
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv)
    for thr, mode in ((0.95, 0), (0.6, 1), (1.0, 0), (0.0, 0)):
        got = _compare(dsa, bt, q, kv, meta, thr, mode, f"G={G} thr={thr} mode={mode}")
    # a few rows against the oracle, on the call's own scores
    s32, ids, counts, O, l, m = (np_(x) for x in dsa.psa_decode(q, kv, meta, 0.9, 0, float(bt.scale)))
    units = [(b, h) for b in (0, 1, 2, 3, B - 1) for h in (0, Hkv - 1)]
    check_psa_result(bt, s32, ids, counts, O, l, m, 0.9, 0, f"psa_decode oracle G={G}", units)


def test_psa_decode_few_rows_runs_the_two_calls(gpu_lib):
    dsa = gpu_lib
    _banner("psa_decode two-call path")
    bt = wl.random_batch(811, [16 * 70 + 3, 16 * 20], n_q_heads=8, n_kv_heads=4, head_dim=128, page_size=16)
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv)
    for thr, mode in ((0.95, 0), (0.7, 1)):
        _compare(dsa, bt, q, kv, meta, thr, mode, f"few rows thr={thr}")


@pytest.mark.parametrize("G,P", [(1, 16), (4, 64)])
def test_psa_decode_streaming_heads(gpu_lib, G, P):
    """Streaming heads (LServe section 4.1) in the fused launch: their rows
    score -inf and their workgroups attend to the sink and local pages; the
    result equals the two calls' bit for bit and the oracle's unit by unit."""
    import oracle
    dsa = gpu_lib
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    Hkv = 32
    B = max(8, -(-n_cu // Hkv))
    _banner(f"psa_decode streaming G={G} P={P} rows={B * Hkv}")
    rng = np.random.default_rng(17 + G)
    lens = [0, 5, P * 3 + 1] + [int(x) for x in rng.integers(P * 40, P * 90, size=B - 3)]
    flags = np.zeros(Hkv, np.uint8)
    flags[::3] = 1
    bt = wl.random_batch(820 + G, lens, n_q_heads=Hkv * G, n_kv_heads=Hkv, head_dim=128, page_size=P,
                         streaming=flags, sink=3 * P // 2, local=4 * P + 5)
    q, kv, st = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv)
    for thr, mode in ((0.95, 0), (0.6, 1)):
        _compare(dsa, bt, q, kv, meta, thr, mode, f"streaming G={G} thr={thr}", st)
    s32, ids, counts, O, l, m = (np_(x) for x in dsa.psa_decode(q, kv, meta, 0.9, 0, float(bt.scale), streaming=st))
    units = [(b, h) for b in (0, 1, 2, 3, B - 1) for h in (0, 1, 3, Hkv - 1)]
    dense = [(b, h) for b, h in units if not flags[h]]
    check_psa_result(bt, s32, ids, counts, O, l, m, 0.9, 0, f"psa_decode streaming oracle G={G}", dense)
    from parity_util import check_attention
    for b, h in units:
        if not flags[h]:
            continue
        assert np.all(np.isneginf(s32[b, h])), f"streaming row scores (b={b}, h={h})"
        rid, rn, rO, rl, rm = oracle.psa_unit(bt, b, h, s32[b, h].astype(np.float64), 0.9, 0)
        n = int(counts[b, h])
        assert n == rn and np.array_equal(ids[b, h, :n], rid), f"streaming pages (b={b}, h={h})"
        assert np.all(ids[b, h, n:] == -1)
        sl = slice(h * G, (h + 1) * G)
        check_attention("bf16", O[b, sl], l[b, sl], m[b, sl], rO, rl, rm, f"streaming (b={b}, h={h})")
