"""PRR decode step orchestration: selection overlapped with speculative
attention on two HIP streams, then repair and the EMA predictor.

"Predict, Reuse, and Repair", sections 1-3: in a plain dynamic-sparse step
the page selection must finish before attention starts.  PRR predicts the
selection (EMA over past page scores, section 3.1), runs attention over the
predicted set P while the real selection A is computed, then repairs the
result with the pages of A that P missed (section 3.3), and feeds the new
scores back into the predictor.

This module only sequences calls of the C ABI (through the binding) on two
streams joined by an event; every step of the arithmetic runs in the HIP
library.  Stream priorities stay at the default.
"""
from __future__ import annotations

import math

import torch

from . import (OP_ATTN_REPAIR, PagedKV, attn_repair, ema_predict_update, page_score, page_select_topk,
               sparse_decode_attn, workspace_bytes)


class PRRDecoder:
    """Per-layer PRR state for one batch of sequences: EMA level/trend per
    (sequence, KV head, page), the speculative set for the next step, and
    the buffers of one step.  `step(q)` enqueues one decode step on the
    current stream (plus a side stream for the selection) and returns
    (O, l, m); nothing is synchronised with the host."""

    def __init__(self, kv: PagedKV, meta: torch.Tensor, n_q_heads: int, k: int, alpha: float, beta: float,
                 gamma: float, delta: float = 1.0, logical_page: int | None = None, scale: float | None = None):
        self.kv, self.meta, self.k = kv, meta, k
        self.alpha, self.beta, self.gamma, self.delta = alpha, beta, gamma, delta
        self.lp = logical_page or kv.page_size
        self.scale = scale
        self.k_spec = max(1, int(math.floor(delta * k)))
        self.stride = max(k, self.k_spec)
        B, H, N, D = kv.batch, kv.n_kv_heads, kv.max_pages, kv.head_dim
        dev = kv.k.device
        f32, i32 = torch.float32, torch.int32
        self.scores = torch.empty((B, H, N), dtype=f32, device=dev)
        self.a_ids = torch.full((B, H, self.stride), -1, dtype=i32, device=dev)
        self.a_counts = torch.zeros((B, H), dtype=i32, device=dev)
        self.p_ids = torch.full((B, H, self.stride), -1, dtype=i32, device=dev)
        self.p_counts = torch.zeros((B, H), dtype=i32, device=dev)
        self.level = torch.zeros(B * H * N, dtype=f32, device=dev)
        self.trend = torch.zeros(B * H * N, dtype=f32, device=dev)
        self.pred = torch.zeros((B, H, N), dtype=f32, device=dev)
        self.O = torch.empty((B, n_q_heads, D), dtype=f32, device=dev)
        self.l = torch.empty((B, n_q_heads), dtype=f32, device=dev)
        self.m = torch.empty((B, n_q_heads), dtype=f32, device=dev)
        self.ws = torch.zeros(workspace_bytes(OP_ATTN_REPAIR, kv, n_q_heads, self.stride), dtype=torch.uint8,
                              device=dev)
        self.side = torch.cuda.Stream(device=dev)      # default priority
        self.t = 0

    def _select(self, q):
        """IS^t = page scores; A^t = top-k of IS^t (written into a_ids)."""
        page_score(q, self.kv, self.meta, self.lp, scores=self.scores)
        if self.stride == self.k:
            page_select_topk(self.scores, self.kv.seq_lens, self.kv.page_size, self.k, ids=self.a_ids,
                             counts=self.a_counts)
        else:
            ids, counts = page_select_topk(self.scores, self.kv.seq_lens, self.kv.page_size, self.k)
            self.a_ids.fill_(-1)
            self.a_ids[..., :self.k].copy_(ids)
            self.a_counts.copy_(counts)

    def _predict_next(self, init: bool):
        """EMA update with IS^t (or initialisation) and P^{t+1} = top of the prediction."""
        ema_predict_update(self.scores, self.level, self.trend, self.pred, self.alpha, self.beta, self.gamma,
                           init=init)
        if self.stride == self.k_spec:
            page_select_topk(self.pred, self.kv.seq_lens, self.kv.page_size, self.k_spec, ids=self.p_ids,
                             counts=self.p_counts)
        else:
            ids, counts = page_select_topk(self.pred, self.kv.seq_lens, self.kv.page_size, self.k_spec)
            self.p_ids.fill_(-1)
            self.p_ids[..., :self.k_spec].copy_(ids)
            self.p_counts.copy_(counts)

    def step(self, q: torch.Tensor):
        out = (self.O, self.l, self.m)
        if self.t == 0:
            # no prediction yet: a plain selection-then-attention step
            self._select(q)
            sparse_decode_attn(q, self.kv, self.a_ids, self.a_counts, scale=self.scale, out=out, ws=self.ws)
            self._predict_next(init=True)
        else:
            main = torch.cuda.current_stream()
            fork = torch.cuda.Event()
            fork.record(main)
            with torch.cuda.stream(self.side):
                self.side.wait_event(fork)
                self._select(q)                       # selection ...
                joined = torch.cuda.Event()
                joined.record(self.side)
            # ... overlapped with speculative attention over P^t
            sparse_decode_attn(q, self.kv, self.p_ids, self.p_counts, scale=self.scale, out=out, ws=self.ws)
            main.wait_event(joined)
            attn_repair(q, self.kv, self.a_ids, self.a_counts, self.p_ids, self.p_counts, *out, scale=self.scale,
                        ws=self.ws)
            self._predict_next(init=False)
        self.t += 1
        return out
