"""PRR decode step orchestration: the exact selection and the predictor run
on a side stream while the speculative attention runs on the caller's
stream; the repair joins them.

"Predict, Reuse, and Repair", sections 1-3: in a plain dynamic-sparse step
the page selection must finish before attention starts.  PRR predicts the
selection (EMA over past page scores, section 3.1), runs attention over the
predicted set P while the real selection A is computed, then repairs the
result with the pages of A that P missed (section 3.3), and feeds the new
scores back into the predictor.

The predictor update and the next step's speculative set P^{t+1} depend
only on this step's scores IS^t, not on attention or on A^t, so one launch
(dsa_prr_select) selects A^t and, in other workgroups of the same grid,
updates the EMA and selects P^{t+1}; the caller's stream waits for P^{t+1}
only at the next step's speculative attention.  P is
double-buffered: the side stream writes P^{t+1} while the caller's stream
still reads P^t.

This module only sequences calls of the C ABI (through the binding) on two
streams joined by events; every step of the arithmetic runs in the HIP
library.  Stream priorities stay at the default.
"""
from __future__ import annotations

import math

import torch

from . import (OP_ATTN_REPAIR, PagedKV, attn_repair, ema_predict_update, page_score, page_select_topk,
               prr_select, sparse_decode_attn, workspace_bytes)


class PRRDecoder:
    """Per-layer PRR state for one batch of sequences: EMA level/trend per
    (sequence, KV head, page), the speculative sets, and the buffers of one
    step.  `step(q)` enqueues one decode step on the current stream (plus a
    side stream for the selection and the predictor) and returns (O, l, m);
    nothing is synchronised with the host.  After a step, `a_ids` holds A^t
    and `p_ids` the prediction P^{t+1} for the next step."""

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
        self._p = [(torch.full((B, H, self.stride), -1, dtype=i32, device=dev),
                    torch.zeros((B, H), dtype=i32, device=dev)) for _ in range(2)]
        self._cur = 0                      # buffer holding P^t of the coming step
        self.level = torch.zeros(B * H * N, dtype=f32, device=dev)
        self.trend = torch.zeros(B * H * N, dtype=f32, device=dev)
        self.pred = torch.zeros((B, H, N), dtype=f32, device=dev)
        self.O = torch.empty((B, n_q_heads, D), dtype=f32, device=dev)
        self.l = torch.empty((B, n_q_heads), dtype=f32, device=dev)
        self.m = torch.empty((B, n_q_heads), dtype=f32, device=dev)
        self.ws = torch.zeros(workspace_bytes(OP_ATTN_REPAIR, kv, n_q_heads, self.stride), dtype=torch.uint8,
                              device=dev)
        self.side = torch.cuda.Stream(device=dev)      # default priority
        self._p_ready = None               # event: P^t written (side stream of the previous step)
        self.t = 0

    def join(self):
        """Make the current stream wait for the side stream's last work (the
        predictor update of the last step); needed before graph capture ends
        and before timing the caller's stream."""
        if self._p_ready is not None:
            torch.cuda.current_stream().wait_event(self._p_ready)
            self._p_ready = None

    @property
    def p_ids(self):
        """The latest prediction (P^{t+1} after step t)."""
        return self._p[self._cur][0]

    @property
    def p_counts(self):
        return self._p[self._cur][1]

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

    def _predict_next(self, init: bool, buf: int):
        """EMA update with IS^t (or initialisation) and P^{t+1} = top of the prediction, into buffer buf."""
        ema_predict_update(self.scores, self.level, self.trend, self.pred, self.alpha, self.beta, self.gamma,
                           init=init)
        p_ids, p_counts = self._p[buf]
        if self.stride == self.k_spec:
            page_select_topk(self.pred, self.kv.seq_lens, self.kv.page_size, self.k_spec, ids=p_ids,
                             counts=p_counts)
        else:
            ids, counts = page_select_topk(self.pred, self.kv.seq_lens, self.kv.page_size, self.k_spec)
            p_ids.fill_(-1)
            p_ids[..., :self.k_spec].copy_(ids)
            p_counts.copy_(counts)

    def _select_and_predict(self, q, init: bool, buf: int):
        """IS^t, A^t, the EMA update and P^{t+1} (into buffer buf): one
        score launch and one launch that runs both selections side by side
        when |A| = |P|, else the separate calls."""
        if self.k == self.k_spec:
            page_score(q, self.kv, self.meta, self.lp, scores=self.scores)
            p_ids, p_counts = self._p[buf]
            prr_select(self.scores, self.kv.seq_lens, self.kv.page_size, self.k, self.level, self.trend,
                       self.pred.view(-1), self.alpha, self.beta, self.gamma, init, self.k_spec, self.a_ids,
                       self.a_counts, p_ids, p_counts)
        else:
            self._select(q)
            self._predict_next(init=init, buf=buf)

    def step(self, q: torch.Tensor):
        out = (self.O, self.l, self.m)
        main = torch.cuda.current_stream()
        cur, nxt = self._cur, 1 - self._cur
        if self.t == 0:
            # no prediction yet: a plain selection-then-attention step
            self._select_and_predict(q, init=True, buf=nxt)
            sparse_decode_attn(q, self.kv, self.a_ids, self.a_counts, scale=self.scale, out=out, ws=self.ws)
        else:
            # the side stream starts once everything enqueued so far on the
            # caller's stream (the previous step, which read a_ids and P^{t-1})
            # is done
            fork = torch.cuda.Event()
            fork.record(main)
            with torch.cuda.stream(self.side):
                self.side.wait_event(fork)
                if self.k == self.k_spec:
                    self._select_and_predict(q, init=False, buf=nxt)   # IS^t, A^t, EMA, P^{t+1}
                    a_ready = torch.cuda.Event()
                    a_ready.record(self.side)
                    p_ready = a_ready
                else:
                    self._select(q)                              # IS^t, A^t ...
                    a_ready = torch.cuda.Event()
                    a_ready.record(self.side)
                    self._predict_next(init=False, buf=nxt)      # ... then EMA and P^{t+1}
                    p_ready = torch.cuda.Event()
                    p_ready.record(self.side)
            # speculative attention over P^t, overlapped with the selection
            self.join()
            p_ids, p_counts = self._p[cur]
            sparse_decode_attn(q, self.kv, p_ids, p_counts, scale=self.scale, out=out, ws=self.ws)
            main.wait_event(a_ready)
            attn_repair(q, self.kv, self.a_ids, self.a_counts, p_ids, p_counts, *out, scale=self.scale, ws=self.ws)
            self._p_ready = p_ready
        self._cur = nxt
        self.t += 1
        return out
