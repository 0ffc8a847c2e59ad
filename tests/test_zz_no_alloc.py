"""dsa_sparse_decode_attn_noalloc, for callers that cannot allocate: called
through the C ABI, its outputs must equal those of dsa_sparse_decode_attn
(with a caller workspace) on the same inputs -- bit for bit, since the same
kernels run -- on two calls in a row, the second with a smaller input, so
the fixed scratch is reused with stale content from the first call."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from parity_util import np_, to_device

pytestmark = pytest.mark.gpu


def _ids(seed, bt, k):
    """k random distinct valid pages per (sequence, KV head), ragged counts
    (one unit empty when there are several)."""
    rng = np.random.default_rng(seed)
    B, H = bt.batch, bt.n_kv_heads
    ids = np.full((B, H, k), -1, np.int32)
    cnt = np.zeros((B, H), np.int32)
    for b in range(B):
        n = -(-int(bt.seq_lens[b]) // bt.page_size)
        for h in range(H):
            c = 0 if (B * H > 1 and b == B - 1 and h == H - 1) else min(n, int(rng.integers(1, k + 1)))
            ids[b, h, :c] = np.sort(rng.choice(n, size=c, replace=False))
            cnt[b, h] = c
    return torch.from_numpy(ids).cuda(), torch.from_numpy(cnt).cuda()


def _both(dsa, seed, seq_lens, n_q_heads, n_kv_heads, k, dtype):
    bt = wl.random_batch(seed, seq_lens, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, dtype=dtype)
    q, kv, _ = to_device(dsa, bt)
    ids, cnt = _ids(seed + 1, bt, k)
    B, Hq, D = bt.batch, n_q_heads, bt.head_dim
    scale = float(np.float32(1.0 / np.sqrt(D)))
    ws = torch.zeros(dsa.workspace_bytes(dsa.OP_SPARSE_DECODE_ATTN, kv, Hq, k), dtype=torch.uint8, device="cuda")
    ref = dsa.sparse_decode_attn(q, kv, ids, cnt, scale=scale, ws=ws)
    O = torch.full((B, Hq, D), float("nan"), device="cuda")
    l = torch.full((B, Hq), float("nan"), device="cuda")
    m = torch.full((B, Hq), float("nan"), device="cuda")
    rc = dsa.lib.dsa_sparse_decode_attn_noalloc(
        ctypes.c_void_p(q.data_ptr()), Hq, ctypes.byref(kv.c()), ctypes.c_void_p(ids.data_ptr()),
        ctypes.c_void_p(cnt.data_ptr()), k, None, scale, ctypes.c_void_p(O.data_ptr()),
        ctypes.c_void_p(l.data_ptr()), ctypes.c_void_p(m.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, dsa.lib.dsa_status_str(rc)
    torch.cuda.synchronize()
    for name, a, b in (("O", O, ref[0]), ("l", l, ref[1]), ("m", m, ref[2])):
        a, b = np_(a), np_(b)
        assert np.array_equal(a, b), f"{name}: no-alloc differs from the workspace call (max |d| " \
                                     f"{np.nanmax(np.abs(a - b))})"
    return np_(cnt)


@pytest.mark.parametrize("dtype,n_q_heads,n_kv_heads", [("bf16", 8, 2), ("bf16", 32, 2), ("f32", 4, 4)])
def test_noalloc_matches_workspace_call(gpu_lib, dtype, n_q_heads, n_kv_heads):
    dsa = gpu_lib
    print(f"noalloc {dtype} Hq={n_q_heads} Hkv={n_kv_heads}: large call", flush=True)
    c1 = _both(dsa, 11, [16 * 300 + 5, 16 * 97], n_q_heads, n_kv_heads, 128, dtype)
    print(f"noalloc {dtype} Hq={n_q_heads} Hkv={n_kv_heads}: smaller call", flush=True)
    c2 = _both(dsa, 12, [16 * 40 + 3], n_q_heads, n_kv_heads, 24, dtype)
    assert c1.sum() > c2.sum() > 0


def test_noalloc_rejects_calls_beyond_its_scratch(gpu_lib):
    """A shape whose partials exceed the fixed scratch is refused before
    anything is enqueued."""
    dsa = gpu_lib
    bt = wl.random_batch(13, [16 * 64], n_q_heads=32, n_kv_heads=2, dtype="bf16", max_pages=8192)
    q, kv, _ = to_device(dsa, bt)
    k = 8192
    assert dsa.workspace_bytes(dsa.OP_SPARSE_DECODE_ATTN, kv, 32, k) > dsa.NOALLOC_SCRATCH_BYTES
    ids = torch.full((1, 2, k), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    out = [torch.empty(s, device="cuda") for s in ((1, 32, 128), (1, 32), (1, 32))]
    with pytest.raises(dsa.DsaError, match="no-allocation scratch"):
        dsa.sparse_decode_attn_noalloc(q, kv, ids, cnt, *out)
