"""PRR decode step orchestration: the exact selection and the predictor run
beside the speculative attention; the repair joins them.

"Predict, Reuse, and Repair", sections 1-3: in a plain dynamic-sparse step
the page selection must finish before attention starts.  PRR predicts the
selection (EMA over past page scores, section 3.1), runs attention over the
predicted set P while the real selection A is computed, then repairs the
result with the pages of A that P missed (section 3.3), and feeds the new
scores back into the predictor.

The predictor update and the next step's speculative set P^{t+1} depend
only on this step's scores IS^t, not on attention or on A^t, so one call
(dsa_prr_select) selects A^t and, in other workgroups of the same grid,
updates the EMA and selects P^{t+1}; the caller's stream waits for P^{t+1}
only at the next step's speculative attention.  The call gets no
workspace, so each row's selections take one workgroup each: the split-row
selection would be faster on its own, but it spreads over many CUs, and
beside the speculative attention the step is faster with the selection
kept to a few CUs.  P is
double-buffered: the side stream writes P^{t+1} while the caller's stream
still reads P^t.

The speculation budget |P| = floor(delta * |A|) comes from an offline
profile indexed by context length (section 3.4): the largest delta whose
speculative attention still fits in the selection window
(profile_delta_table, DeltaTable).

Where the library has it (bf16 KV, one score per page, |A| = |P|) a
speculative step is one call, dsa_prr_decode_step, on the caller's stream:
the independent parts share launches (scores beside the speculative
partials, the speculative combine beside the repair's partials) instead of
streams, because each dependency between the hardware queues of a HIP
graph costs several microseconds on this GPU.  Otherwise the selection runs
on a side stream joined by events.

This module only sequences calls of the C ABI (through the binding); every
step of the arithmetic runs in the HIP library.  Stream priorities stay at
the default.
"""
from __future__ import annotations

import bisect
import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import (OP_ATTN_REPAIR, OP_PRR_DECODE_STEP, PagedKV, attn_repair, ema_predict_update, page_score,
               page_score_ema, page_select_topk, prr_decode_step, prr_select, prr_select_workspace_bytes,
               sparse_decode_attn, workspace_bytes)


class PRRDecoder:
    """Per-layer PRR state for one batch of sequences: EMA level/trend per
    (sequence, KV head, page), the speculative sets, and the buffers of one
    step.  `step(q)` enqueues one decode step on the current stream (in one
    call where the library supports the shape, else with a side stream for
    the selection and the predictor) and returns (O, l, m); nothing is
    synchronised with the host.  After a step, `a_ids` holds A^t and
    `p_ids` the prediction P^{t+1} for the next step.  one_stream=False
    forces the two-stream form (one_stream=None: the one-call step where
    supported)."""

    def __init__(self, kv: PagedKV, meta: torch.Tensor, n_q_heads: int, k: int, alpha: float, beta: float,
                 gamma: float, delta: float = 1.0, logical_page: int | None = None, scale: float | None = None,
                 delta_table: "DeltaTable | None" = None, context_tokens: int | None = None,
                 one_stream: bool | None = None):
        if delta_table is not None:   # section 3.4: delta by context length
            delta = delta_table.lookup(context_tokens or kv.max_pages * kv.page_size)
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
        # M^t = A^t \ P^t, written by the selection launch when |A| = |P|
        self.m_ids = torch.full((B, H, self.stride), -1, dtype=i32, device=dev)
        self.m_counts = torch.zeros((B, H), dtype=i32, device=dev)
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
        self.sel_ws = None                 # a split-row selection workspace (see split_selection)
        can = (self.k == self.k_spec and kv.k.dtype == torch.bfloat16 and self.lp == kv.page_size
               and N <= 65536)
        if one_stream and not can:
            raise ValueError("the one-call PRR step needs bf16 KV, logical page = page and |A| = |P|")
        self.one_stream = can if one_stream is None else bool(one_stream)
        self.step_ws = (torch.zeros(workspace_bytes(OP_PRR_DECODE_STEP, kv, n_q_heads, self.k), dtype=torch.uint8,
                                    device=dev) if self.one_stream else None)
        self.side = torch.cuda.Stream(device=dev)      # default priority
        self._p_ready = None               # event: P^t written (side stream of the previous step)
        self.t = 0

    def split_selection(self, on: bool = True):
        """Give dsa_prr_select a workspace, so that long rows take the
        split-row selection (many CUs) instead of one workgroup each."""
        B, H, N = self.scores.shape
        nb = prr_select_workspace_bytes(B, H, N) if on else 0
        self.sel_ws = torch.empty(nb, dtype=torch.uint8, device=self.scores.device) if nb else None
        if self.sel_ws is not None:
            self.one_stream = False        # the one-call step takes no selection workspace

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

    def _select_and_predict(self, q, init: bool, buf: int, cur: int | None = None):
        """IS^t, A^t, the EMA update and P^{t+1} (into buffer buf): when
        |A| = |P|, one launch for the scores and the EMA update and one that
        runs both selections side by side -- which also writes M^t =
        A^t \\ P^t when P^t is in buffer cur -- else the separate calls."""
        if self.k == self.k_spec:
            page_score_ema(q, self.kv, self.meta, self.level, self.trend, self.pred, self.alpha, self.beta,
                           self.gamma, init=init, logical_page=self.lp, scores=self.scores)
            p_ids, p_counts = self._p[buf]
            with_m = cur is not None
            prr_select(self.scores, self.kv.seq_lens, self.kv.page_size, self.k, None, None,
                       self.pred.view(-1), self.alpha, self.beta, self.gamma, init, self.k_spec, self.a_ids,
                       self.a_counts, p_ids, p_counts, p_cur=self._p[cur] if with_m else None,
                       m_out=(self.m_ids, self.m_counts) if with_m else None, ws=self.sel_ws,
                       split=self.sel_ws is not None)
        else:
            self._select(q)
            self._predict_next(init=init, buf=buf)

    def step(self, q: torch.Tensor):
        out = (self.O, self.l, self.m)
        main = torch.cuda.current_stream()
        cur, nxt = self._cur, 1 - self._cur
        if self.t > 0 and self.one_stream:
            # the whole speculative step in one call on this stream
            self.join()
            prr_decode_step(q, self.kv, self.meta, self.scores, self.level, self.trend, self.pred, self.alpha,
                            self.beta, self.gamma, self.k, self._p[cur], (self.a_ids, self.a_counts),
                            (self.m_ids, self.m_counts), self._p[nxt], *out, logical_page=self.lp, scale=self.scale,
                            ws=self.step_ws)
        elif self.t == 0:
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
                    self._select_and_predict(q, init=False, buf=nxt, cur=cur)   # IS^t, A^t, M^t, EMA, P^{t+1}
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
            if self.k == self.k_spec:   # M^t came with A^t
                attn_repair(q, self.kv, self.m_ids, self.m_counts, None, None, *out, scale=self.scale, ws=self.ws)
            else:
                attn_repair(q, self.kv, self.a_ids, self.a_counts, p_ids, p_counts, *out, scale=self.scale,
                            ws=self.ws)
            self._p_ready = p_ready
        self._cur = nxt
        self.t += 1
        return out


# --------------------------------------------------------------------------
# dynamic speculation budget (section 3.4): min |A \ P| subject to
# |P| <= delta |A|, with delta the largest value whose speculative attention
# fits in the selection window, profiled offline per context length
# --------------------------------------------------------------------------
DELTA_GRID = (0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 2.0)
PROFILE_CONTEXTS = (4096, 8192, 16384, 32768, 65536)


def choose_delta(t_select_us: float, t_spec_us: dict) -> float:
    """The largest delta whose speculative attention takes no longer than
    the selection it overlaps; the smallest profiled delta when none fits."""
    fit = [d for d, t in t_spec_us.items() if t <= t_select_us]
    return max(fit) if fit else min(t_spec_us)


@dataclass
class DeltaTable:
    """(context tokens, delta) pairs, ascending in context, and optionally
    the profiled timings behind them: {context: (select_us, {delta:
    spec_us})}.  Inside the profiled range the pairs are looked up; past the
    longest profiled context the timings are extrapolated (section 3.4 of
    the page profiles 4K-64K and extends the table to longer contexts by
    polynomial regression)."""
    entries: list = field(default_factory=list)
    timings: dict = field(default_factory=dict)

    def lookup(self, context_tokens: int) -> float:
        """delta of the longest profiled context not above context_tokens
        (of the shortest one for shorter contexts); beyond the longest
        profiled context, the delta chosen on extrapolated timings when the
        table holds them."""
        if not self.entries:
            raise ValueError("empty delta table")
        ctx = [c for c, _ in self.entries]
        if int(context_tokens) > ctx[-1] and len(self.timings) >= 2:
            return self.extrapolate(int(context_tokens))
        i = bisect.bisect_right(ctx, int(context_tokens)) - 1
        return self.entries[max(i, 0)][1]

    def extrapolate(self, context_tokens: int, degree: int = 2) -> float:
        """Least-squares polynomials in the context length (degree 2, or
        lower when fewer contexts were profiled) through the selection
        window and through each delta's speculative-attention time, taken at
        context_tokens, then the same choice as inside the table."""
        ctx = sorted(self.timings)
        deg = min(degree, len(ctx) - 1)
        x = np.asarray(ctx, dtype=np.float64)

        def at(values):
            return float(np.polyval(np.polyfit(x, np.asarray(values, dtype=np.float64), deg), context_tokens))
        t_sel = at([self.timings[c][0] for c in ctx])
        deltas = sorted(self.timings[ctx[0]][1])
        t_spec = {d: at([self.timings[c][1][d] for c in ctx]) for d in deltas}
        return choose_delta(t_sel, t_spec)


def _time_us(fn, reps: int, trials: int = 7) -> float:
    """Duration of fn() from a HIP graph of `reps` calls: the median over
    `trials` replays of the per-call average."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / reps)
    return sorted(out)[len(out) // 2]


def profile_delta_table(n_q_heads: int = 32, n_kv_heads: int = 2, head_dim: int = 128, page_size: int = 16,
                        contexts=PROFILE_CONTEXTS, deltas=DELTA_GRID, sparsity: int = 16, reps: int = 20,
                        seed: int = 0):
    """Offline profile of section 3.4 on a seeded bf16 pool (batch 1): per
    context length, the selection window (page scores, then dsa_prr_select:
    the exact selection, the EMA and the next speculative selection) and the
    speculative attention over floor(delta * k) pages for every delta, with
    k = pages / sparsity.  Returns (DeltaTable, {context: timings})."""
    from . import PagedKV as _KV, page_meta_build
    dev = torch.device("cuda", torch.cuda.current_device())
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    entries, report, timings = [], {}, {}
    for L in sorted(contexts):
        N = -(-L // page_size)
        k = max(1, N // sparsity)
        pool = (N, n_kv_heads, page_size, head_dim)
        kv = _KV(torch.randn(pool, generator=gen, device=dev).to(torch.bfloat16),
                 torch.randn(pool, generator=gen, device=dev).to(torch.bfloat16),
                 torch.arange(N, dtype=torch.int32, device=dev)[None, :].contiguous(),
                 torch.full((1,), L, dtype=torch.int32, device=dev))
        meta = page_meta_build(kv)
        q = torch.randn((1, n_q_heads, head_dim), generator=gen, device=dev).to(torch.bfloat16)
        dec = PRRDecoder(kv, meta, n_q_heads, k, 0.6, 0.3, 0.25)
        dec._select_and_predict(q, init=True, buf=0)
        t_sel = _time_us(lambda: dec._select_and_predict(q, init=False, buf=1), reps)
        t_spec = {}
        for d in deltas:
            kd = max(1, min(N, int(math.floor(d * k))))
            ids = torch.arange(kd, dtype=torch.int32, device=dev).view(1, 1, kd).expand(1, n_kv_heads, kd).contiguous()
            cnt = torch.full((1, n_kv_heads), kd, dtype=torch.int32, device=dev)
            ws = torch.zeros(workspace_bytes(OP_ATTN_REPAIR, kv, n_q_heads, kd), dtype=torch.uint8, device=dev)
            out = (dec.O, dec.l, dec.m)
            t_spec[d] = _time_us(lambda: sparse_decode_attn(q, kv, ids, cnt, out=out, ws=ws), reps)
        delta = choose_delta(t_sel, t_spec)
        entries.append((L, delta))
        timings[L] = (t_sel, dict(t_spec))
        report[L] = {"pages": N, "k": k, "select_us": round(t_sel, 3),
                     "spec_us": {str(d): round(v, 3) for d, v in t_spec.items()}, "delta": delta}
    return DeltaTable(entries, timings), report
