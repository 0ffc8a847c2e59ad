"""GPU parity of dsa_block_sparse_prefill against the oracle's prefill
attention (causal, with the Lambda mask on streaming heads): (O, l, m) of
every (token, q head) within the bf16 attention tolerance.  Cases cover
ragged lengths (partial last tiles), head_dim 64 and 128, GQA groups of 1 to
8, peaky logits, sink/local windows on and off tile boundaries, a streaming
head with an empty mask, a one-token prompt, and the 16K-token workload the
benchmark times (sampled queries)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import check_attention, np_

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _bf16(dsa, x):
    return dsa.upload_q(x, "bf16")


@pytest.mark.parametrize("L,Hq,Hkv,D,streaming,sink,local,gain", [
    (200, 4, 2, 128, None, 0, 0, 1.0),
    (257, 8, 2, 64, [0, 1], 20, 70, 2.0),
    (130, 4, 4, 128, [1, 1, 0, 0], 64, 64, 3.0),
    (64, 2, 1, 128, [1], 0, 0, 1.0),
    (1, 2, 1, 128, None, 0, 0, 1.0),
    (500, 16, 2, 128, [0, 1], 128, 256, 1.0),
])
def test_prefill_matches_oracle(gpu_lib, L, Hq, Hkv, D, streaming, sink, local, gain):
    dsa = gpu_lib
    _banner(f"prefill L={L} Hq={Hq} Hkv={Hkv} D={D} streaming={streaming} sink={sink} local={local}")
    q, k, v = wl.prefill_inputs(101 + L, L, Hq, Hkv, D, "bf16", q_gain=gain)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    st = None if streaming is None else dsa.Streaming(np.asarray(streaming, np.uint8), sink, local)
    O, l, m = dsa.block_sparse_prefill(_bf16(dsa, q), _bf16(dsa, k), _bf16(dsa, v), streaming=st, scale=scale)
    torch.cuda.synchronize()
    rO, rl, rm = oracle.prefill_attention(q, k, v, "bf16", scale, streaming=streaming, sink=sink, local=local)
    check_attention("bf16", np_(O).reshape(L * Hq, D), np_(l).reshape(-1), np_(m).reshape(-1),
                    rO.reshape(L * Hq, D), rl.reshape(-1), rm.reshape(-1), "prefill")


def test_prefill_16k_sampled(gpu_lib):
    """The benchmark's 16K-token prompt (32 q / 8 KV heads, half of them
    streaming): 48 sampled (token, head) pairs, including tile edges and the
    last token, against the oracle's attention over the same keys."""
    dsa = gpu_lib
    _banner("prefill 16K sampled")
    cfg = wl.PREFILL_16K
    L, Hq, Hkv, D = cfg["L"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    q, k, v = wl.prefill_inputs(cfg["seed"], L, Hq, Hkv, D, "bf16")
    st = dsa.Streaming(cfg["streaming"], cfg["sink"], cfg["local"])
    scale = float(np.float32(1.0 / np.sqrt(D)))
    O, l, m = dsa.block_sparse_prefill(_bf16(dsa, q), _bf16(dsa, k), _bf16(dsa, v), streaming=st, scale=scale)
    torch.cuda.synchronize()
    O, l, m = np_(O), np_(l), np_(m)
    rng = np.random.default_rng(7)
    toks = sorted({0, 63, 64, 127, 4095, 4096, L - 65, L - 64, L - 1, *rng.integers(0, L, 15).tolist()})
    heads = rng.integers(0, Hq, len(toks))
    qf, kf, vf = (oracle.widen(x, "bf16") for x in (q, k, v))
    G = Hq // Hkv
    for i, hq in zip(toks, heads):
        for h2 in (int(hq), (int(hq) + G) % Hq):   # one head of a dense group, one of a streaming group
            hk = h2 // G
            j = oracle.prefill_keys(i, L, bool(cfg["streaming"][hk]), cfg["sink"], cfg["local"])
            rO, rl, rm = oracle.attention(qf[i, h2], kf[j, hk], vf[j, hk], scale)
            check_attention("bf16", O[i, h2][None], np.array([l[i, h2]]), np.array([m[i, h2]]), rO[None],
                            np.array([rl]), np.array([rm]), f"token {i} head {h2}")
