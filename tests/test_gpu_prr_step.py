"""The one-call PRR speculative step (dsa_prr_decode_step: the independent
parts of the step share launches on one stream) against the two-stream
decoder that chains the separate calls ("Predict, Reuse, and Repair",
sections 2-3): same scores, EMA state, A^t, M^t, P^{t+1} and (O, l, m), bit
for bit, step after step on a drifting query.  The separate calls are
themselves checked against the oracle (test_gpu_parity, test_gpu_prr_select,
and the full PRR trace in test_gpu_fullsize, which runs this one-call step)."""
import numpy as np
import pytest
import torch

import workloads as wl
from parity_util import np_, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # (G, page_size, logical_page, seq_lens, k, head_dim)
    (16, 16, 16, [16 * 3000 + 5, 16 * 1200], 256, 128),
    (8, 16, 16, [16 * 5000 + 11], 512, 128),
    (16, 64, 64, [64 * 700 + 40, 64 * 300], 64, 128),
    (8, 32, 32, [32 * 90 + 7, 32 * 2], 200, 128),   # k above a row's pages
    (16, 16, 16, [16 * 900 + 1, 16 * 2500, 16 * 40 + 9], 128, 64),
    # VALU partials (4 and 2 q heads per KV head), one with more speculative splits than CUs
    (4, 16, 16, [16 * 4000 + 3, 16 * 900], 512, 128),
    (4, 16, 16, [16 * 8000] * 4, 1024, 128),
    (2, 32, 32, [32 * 600 + 17, 32 * 5], 100, 64),
    (1, 16, 16, [16 * 2000 + 7, 16 * 30], 128, 128),   # one q head per KV head
    # an empty sequence and one of a single partial page beside a long one
    (16, 16, 16, [0, 16 * 300 + 1, 5], 64, 128),
    (4, 16, 16, [5, 0, 16 * 700], 128, 128),
]


def _same(x: torch.Tensor, y: torch.Tensor) -> bool:
    """Bit for bit (NaNs of pages past a sequence's end included)."""
    if x.dtype == torch.float32:
        return torch.equal(x.view(torch.int32), y.view(torch.int32))
    return torch.equal(x, y)


def _drift(q: torch.Tensor, t: int, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu").manual_seed(seed + t)
    xi = torch.randn(q.shape, generator=g).to(q.device)
    th = 0.05 + 0.05 * t
    return (q.float() * np.cos(th) + xi * np.sin(th)).to(q.dtype)


@pytest.mark.parametrize("G,P,Pl,lens,k,D", CASES)
def test_one_call_step_equals_two_streams(gpu_lib, G, P, Pl, lens, k, D):
    dsa = gpu_lib
    from dynamic_sparse_attention_page_amd.prr import PRRDecoder
    print(f"[case] prr one-call step G={G} P={P} Pl={Pl} lens={lens} k={k} D={D}", flush=True)
    bt = wl.random_batch(401 + G + P, lens, n_q_heads=2 * G, n_kv_heads=2, head_dim=D, page_size=P,
                         logical_page=Pl)
    q0, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv, Pl)
    decs = [PRRDecoder(kv, meta, 2 * G, k, 0.6, 0.3, 0.25, 1.0, logical_page=Pl, one_stream=one)
            for one in (True, False)]
    assert decs[0].one_stream and not decs[1].one_stream
    q = q0
    for t in range(6):
        outs = [d.step(q) for d in decs]
        for d in decs:
            d.join()
        torch.cuda.synchronize()
        a, b = decs
        for name in ("scores", "level", "trend", "pred", "a_ids", "a_counts", "m_ids", "m_counts"):
            assert _same(getattr(a, name), getattr(b, name)), f"step {t}: {name}"
        assert _same(a.p_ids, b.p_ids) and _same(a.p_counts, b.p_counts), f"step {t}: P^(t+1)"
        for x, y, nm in zip(outs[0], outs[1], "Olm"):
            assert _same(x, y), f"step {t}: {nm} differs by {np.nanmax(np.abs(np_(x) - np_(y)))}"
        if t > 0:   # the speculative steps: M^t is A^t minus P^t
            mc = np_(a.m_counts)
            assert (mc <= np_(a.a_counts)).all()
        q = _drift(q0, t, 7)


def test_one_call_step_graph_replays(gpu_lib):
    """The one-call step captured in a HIP graph gives the eager result on
    every replay (its state restored before each, eager work and
    synchronisations between replays): nothing in the step depends on a
    memory clear that a replay would not repeat."""
    dsa = gpu_lib
    from dynamic_sparse_attention_page_amd.prr import PRRDecoder
    print("[case] prr one-call step graph replay", flush=True)
    bt = wl.random_batch(431, [16 * 2500 + 9, 16 * 800], n_q_heads=32, n_kv_heads=2, head_dim=128, page_size=16)
    q0, kv, _ = to_device(dsa, bt)
    meta = dsa.page_meta_build(kv)
    dec = PRRDecoder(kv, meta, 32, 256, 0.6, 0.3, 0.25, 1.0, one_stream=True)
    dec.step(q0)                       # the plain first step
    q1 = _drift(q0, 0, 3)
    state = ("level", "trend", "pred")
    saved = {n: getattr(dec, n).clone() for n in state}
    saved_p = [x.clone() for x in dec._p[dec._cur]]
    cur = dec._cur

    def restore():
        for n in state:
            getattr(dec, n).copy_(saved[n])
        for dst, src in zip(dec._p[cur], saved_p):
            dst.copy_(src)
        dec._cur = cur
        dec.t = 1

    restore()
    dec.step(q1)
    torch.cuda.synchronize()
    outs = ("scores", "level", "trend", "pred", "a_ids", "a_counts", "m_ids", "m_counts", "O", "l", "m")
    ref = {n: getattr(dec, n).clone() for n in outs}
    ref_p = [x.clone() for x in dec._p[1 - cur]]
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            dec.step(q1)
    torch.cuda.synchronize()
    for rep in range(4):
        restore()
        for n in ("scores", "O", "l", "m"):
            getattr(dec, n).fill_(float("nan"))
        for n in ("a_ids", "m_ids"):
            getattr(dec, n).fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in outs:
            assert _same(getattr(dec, n), ref[n]), f"replay {rep}: {n}"
        assert all(_same(x, y) for x, y in zip(dec._p[1 - cur], ref_p)), f"replay {rep}: P^(t+1)"
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()   # eager work between replays
