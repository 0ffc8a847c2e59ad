"""LServe's reusable page selector ("LServe: Efficient Long-sequence LLM
Serving with Unified Sparse Attention", section 4.3, Figure 8).

Consecutive decode queries attend to similar pages, so the page selector
(criticality scores and top-k) runs only for the first token of each chunk
of C consecutive decode steps -- C = 4 by default -- and the chunk's later
tokens reuse that token's pages: the selector's cost drops by a factor of C.

This module only sequences calls of the C ABI (through the binding): the
first step of a chunk is page_score followed by sparse_decode_attn_topk
(selection and attention in one call, the chosen ids kept); the other steps
are sparse_decode_attn over the kept ids.  Nothing is synchronised with the
host.
"""
from __future__ import annotations

import torch

from . import (OP_SPARSE_DECODE_ATTN, PagedKV, Streaming, page_score, sparse_decode_attn, sparse_decode_attn_topk,
               workspace_bytes)


class ChunkedReuseDecoder:
    """Per-layer decode state for one batch: the pages kept from the last
    chunk start and the buffers of one step.  `step(q)` enqueues one decode
    step on the current stream and returns (O, l, m); `ids`/`counts` hold
    the pages in use."""

    def __init__(self, kv: PagedKV, meta: torch.Tensor, n_q_heads: int, k: int, chunk: int = 4,
                 logical_page: int | None = None, streaming: Streaming | None = None, scale: float | None = None):
        if chunk < 1:
            raise ValueError("chunk must be >= 1")
        self.kv, self.meta, self.k, self.chunk = kv, meta, k, chunk
        self.lp = logical_page or kv.page_size
        self.streaming, self.scale = streaming, scale
        B, H, N, D = kv.batch, kv.n_kv_heads, kv.max_pages, kv.head_dim
        dev = kv.k.device
        self.scores = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        self.ids = torch.full((B, H, k), -1, dtype=torch.int32, device=dev)
        self.counts = torch.zeros((B, H), dtype=torch.int32, device=dev)
        self.O = torch.empty((B, n_q_heads, D), dtype=torch.float32, device=dev)
        self.l = torch.empty((B, n_q_heads), dtype=torch.float32, device=dev)
        self.m = torch.empty((B, n_q_heads), dtype=torch.float32, device=dev)
        self.ws = torch.zeros(workspace_bytes(OP_SPARSE_DECODE_ATTN, kv, n_q_heads, k), dtype=torch.uint8,
                              device=dev)
        self.t = 0

    @property
    def selects_now(self) -> bool:
        """Whether the next step runs the selector (it opens a chunk)."""
        return self.t % self.chunk == 0

    def step(self, q: torch.Tensor):
        out = (self.O, self.l, self.m)
        if self.selects_now:
            page_score(q, self.kv, self.meta, self.lp, streaming=self.streaming, scores=self.scores)
            sparse_decode_attn_topk(q, self.kv, self.scores, self.k, streaming=self.streaming, scale=self.scale,
                                    out=out, ids=self.ids, counts=self.counts, ws=self.ws)
        else:
            sparse_decode_attn(q, self.kv, self.ids, self.counts, streaming=self.streaming, scale=self.scale,
                               out=out, ws=self.ws)
        self.t += 1
        return out
