"""GPU parity of the reusable page selector (LServe section 4.3) against the
oracle: over a drifting query trace, the decoder selects at the first step
of every chunk of 4 -- ids checked against the oracle's selection for that
query with the boundary rule -- and every step attends with its own query
over the kept pages, within the attention tolerance of the oracle over
those pages.  Streaming heads keep their sink/local pages.  Chunk 1 is the
per-step pipeline, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from dynamic_sparse_attention_page_amd.reuse import ChunkedReuseDecoder
from parity_util import check_selected_attention, check_selection, np_, to_device

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("dtype,P,Pl,streaming", [("bf16", 64, 16, [0, 1, 0, 1]), ("f32", 16, 16, None)])
def test_chunked_reuse_matches_oracle(gpu_lib, dtype, P, Pl, streaming):
    dsa = gpu_lib
    _banner(f"chunked reuse {dtype} P={P} Pl={Pl} streaming={streaming}")
    bt = wl.random_batch(81, [700, P * 9, 1000], n_q_heads=8, n_kv_heads=4, head_dim=128, page_size=P,
                         logical_page=Pl, dtype=dtype, streaming=streaming, sink=64, local=128)
    k = 6
    q0, kv, st = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, Pl)
    qs = wl.query_drift(82, bt.q, 9, 0.3, dtype)
    dec = ChunkedReuseDecoder(kv, meta, bt.n_q_heads, k, chunk=4, logical_page=Pl, streaming=st)
    for t in range(len(qs)):
        opens = dec.selects_now
        assert opens == (t % 4 == 0)
        qd = dsa.upload_q(qs[t], dtype)
        O, l, m = dec.step(qd)
        torch.cuda.synchronize()
        ids, cnt = np_(dec.ids), np_(dec.counts)
        s = oracle.chunk_start(t, 4)
        if opens:
            ref_sc = oracle.page_scores(bt, q=qs[s])
            for b in range(bt.batch):
                for h in range(bt.n_kv_heads):
                    n = oracle.n_pages(bt.seq_lens[b], P)
                    if streaming is not None and streaming[h]:
                        ref = oracle.streaming_pages(bt.seq_lens[b], P, bt.sink, bt.local)
                        assert np.array_equal(ids[b, h, :cnt[b, h]], ref)
                    else:
                        check_selection(ids[b, h], int(cnt[b, h]), ref_sc[b, h], n, k, f"t={t} b={b} h={h}")
            kept = (ids.copy(), cnt.copy())
            ref_ids = oracle.select_topk(bt, ref_sc, k)   # the oracle's own chunk selection
        else:
            assert np.array_equal(ids, kept[0]) and np.array_equal(cnt, kept[1]), f"t={t}: kept pages changed"
        bq = wl.Batch(**{**bt.__dict__, "q": qs[t]})
        units = [(b, h) for b in range(bt.batch) for h in range(bt.n_kv_heads)]
        check_selected_attention(dsa, bq, qd, kv, st, ids, cnt, (O, l, m), ref_ids, units, f"step {t}")


def test_chunk_one_is_the_per_step_pipeline(gpu_lib):
    dsa = gpu_lib
    _banner("chunked reuse with chunk 1")
    bt = wl.random_batch(83, [1500, 333], n_q_heads=8, n_kv_heads=2, head_dim=128, page_size=16)
    q0, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, 16)
    qs = wl.query_drift(84, bt.q, 3, 0.3, "bf16")
    dec = ChunkedReuseDecoder(kv, meta, bt.n_q_heads, 8, chunk=1)
    for t in range(3):
        q = dsa.upload_q(qs[t], "bf16")
        O, l, m = (x.clone() for x in dec.step(q))
        sc = dsa.page_score(q, kv, meta, 16)
        ids, cnt, O2, l2, m2 = dsa.sparse_decode_attn_topk(q, kv, sc, 8)
        torch.cuda.synchronize()
        assert torch.equal(dec.ids, ids) and torch.equal(dec.counts, cnt)
        assert torch.equal(O, O2) and torch.equal(l, l2) and torch.equal(m, m2)
