"""GPU parity of dsa_kv_append against the oracle's decode-time append.

Each case appends a stream of new tokens to a seeded batch, one token per
sequence per step, with a host stand-in for the cache manager that gives a
sequence's next page a free slot when its new token opens one.  After every
step: K/V pools bit-exact, lengths and per-sequence status exact, and the
key metadata equal (as values) to the oracle's page_meta of the grown cache
in every logical page that holds a token; logical pages that hold none keep
what they held.  At the end, page scores over the appended metadata match
the oracle's scores of the grown cache.  The streams cross logical-page and
page boundaries, start from empty sequences, and include a sequence at
max_pages and one whose next page is never allocated (both must be skipped).
Lengths are advanced in place in some cases and into a separate buffer in
others."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import np_, to_device

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _widen(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return wl.from_bf16_bits(x.view(np.uint16)).astype(np.float64)
    return x.astype(np.float64)


def _host_bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    a = np_(t.view(torch.int16) if dtype == "bf16" else t)
    return a.view(np.uint16) if dtype == "bf16" else a


# dtype, head_dim, page, logical page, n_kv_heads, lengths, max_pages, steps, in place,
# index of the sequence whose pages are never allocated
CASES = [
    ("bf16", 128, 16, 16, 2, [0, 15, 47, 64, 30], 4, 36, True, 4),
    ("bf16", 128, 64, 16, 4, [1, 63, 100, 192, 128], 3, 40, True, 4),
    ("bf16", 64, 32, 16, 2, [31, 0, 33, 96], 3, 35, False, 3),
    ("f32", 128, 16, 16, 2, [5, 16, 0, 64], 4, 34, False, 1),
    ("f32", 64, 64, 32, 8, [0, 70, 129, 192], 3, 66, True, 1),
]


@pytest.mark.parametrize("dtype,D,P,Pl,Hkv,lens,max_pages,steps,inplace,no_alloc", CASES)
def test_append_matches_oracle(gpu_lib, dtype, D, P, Pl, Hkv, lens, max_pages, steps, inplace, no_alloc):
    dsa = gpu_lib
    _banner(f"kv_append {dtype} D={D} P={P} Pl={Pl} Hkv={Hkv} lens={lens} steps={steps} inplace={inplace}")
    B = len(lens)
    bt = wl.random_batch(61, lens, n_q_heads=2 * Hkv, n_kv_heads=Hkv, head_dim=D, page_size=P, logical_page=Pl,
                         dtype=dtype, max_pages=max_pages, spare_slots=B * max_pages)
    spare = sorted(set(range(bt.num_slots)) - set(int(x) for x in bt.page_table[bt.page_table >= 0]))
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, Pl)
    meta0 = _widen(_host_bits(meta, dtype), dtype)
    kn, vn = wl.append_stream(62, B, Hkv, D, steps, dtype)
    status = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    side = torch.empty((B,), dtype=torch.int32, device="cuda")
    skipped = 0
    for t in range(steps):
        for b in range(B):   # cache-manager stand-in: a new page gets a free slot
            L = int(bt.seq_lens[b])
            if b != no_alloc and L % P == 0 and L // P < max_pages and bt.page_table[b][L // P] < 0:
                slot = spare.pop()
                bt.page_table[b][L // P] = slot
                kv.page_table[b, L // P] = slot
        before = np_(kv.seq_lens).copy()
        bt, done = oracle.append_token(bt, kn[t], vn[t])
        out = kv.seq_lens if inplace else side
        dsa.kv_append(kv, dsa.upload_q(kn[t], dtype), dsa.upload_q(vn[t], dtype), meta, Pl, new_seq_lens=out,
                      status=status)
        torch.cuda.synchronize()
        skipped += int((~done).sum())
        assert np.array_equal(np_(status), done.astype(np.int32)), f"step {t}: status"
        assert np.array_equal(np_(out), bt.seq_lens), f"step {t}: lengths"
        if not inplace:
            assert np.array_equal(np_(kv.seq_lens), before), f"step {t}: lengths changed in place"
            kv.seq_lens.copy_(side)
        assert np.array_equal(_host_bits(kv.k, dtype), bt.k), f"step {t}: K pool"
        assert np.array_equal(_host_bits(kv.v, dtype), bt.v), f"step {t}: V pool"
        ref, has = oracle.page_meta(bt)
        got = _widen(_host_bits(meta, dtype), dtype)
        assert np.array_equal(got[has], ref[has]), f"step {t}: metadata of filled logical pages"
        assert np.array_equal(got[~has], meta0[~has]), f"step {t}: metadata of empty logical pages changed"
    assert skipped >= steps, "the full and the unallocated sequence were not exercised"
    assert bt.seq_lens[no_alloc] == min(-(-lens[no_alloc] // P) * P, max_pages * P)
    sc = np_(dsa.page_score(q, kv, meta, Pl))
    ref = oracle.page_scores(bt)
    assert np.array_equal(np.isneginf(sc), np.isneginf(ref))
    fin = np.isfinite(ref)
    err = np.abs(sc[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))
    assert err.max() <= 2e-6, err.max()


def test_append_idempotent_rewrite_of_last_token(gpu_lib):
    """Appending a sequence's own last token at its last position (lengths
    one short, result into a side buffer) leaves pools and metadata
    unchanged: the call the benchmark times is a no-op on the cache."""
    dsa = gpu_lib
    _banner("kv_append rewrite of the last token")
    bt = wl.random_batch(63, [47, 200, 129], n_q_heads=8, n_kv_heads=4, head_dim=128, page_size=64,
                         logical_page=16, dtype="bf16", max_pages=4)
    q, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, 16)
    k0, v0, m0 = kv.k.clone(), kv.v.clone(), meta.clone()
    short = dsa.PagedKV(kv.k, kv.v, kv.page_table, (kv.seq_lens - 1).contiguous())
    last = [(int(bt.page_table[b][(L - 1) // 64]), (L - 1) % 64) for b, L in enumerate(bt.seq_lens)]
    kn = torch.stack([kv.k[s, :, o] for s, o in last]).contiguous()
    vn = torch.stack([kv.v[s, :, o] for s, o in last]).contiguous()
    out = torch.empty(3, dtype=torch.int32, device="cuda")
    for _ in range(3):
        dsa.kv_append(short, kn, vn, meta, 16, new_seq_lens=out)
    torch.cuda.synchronize()
    assert torch.equal(out, kv.seq_lens)
    assert torch.equal(kv.k.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(kv.v.view(torch.int16), v0.view(torch.int16))
    assert torch.equal(meta.view(torch.int16), m0.view(torch.int16))
