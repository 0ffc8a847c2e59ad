"""Query-aware block-sparse paged decode attention for MI355X (gfx950).

Thin ctypes binding of ``libdsa.so`` (declared in ``include/dsa.h``): each
function below marshals torch tensors into the C ABI call of the same name
and launches on the current HIP stream.  Every step of the computation runs
in the library's HIP kernels; torch only provides device memory and streams.
Importing this module fails loudly if the library has not been built
(``python dynamic_sparse_attention_page_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

__all__ = [
    "DsaError", "PagedKV", "Streaming", "lib", "LIB_PATH",
    "page_meta_build", "kv_append", "page_score", "page_score_ema", "page_select_topk", "page_select_progressive",
    "psa_decode", "sparse_decode_attn", "sparse_decode_attn_noalloc", "sparse_decode_attn_topk", "attn_repair", "prr_decode_step", "ema_predict_update", "prr_select", "prr_calibrate", "signal_host", "block_sparse_prefill",
    "workspace_bytes",
    "OP_SPARSE_DECODE_ATTN", "OP_ATTN_REPAIR", "OP_PRR_DECODE_STEP", "EXPORTED", "prr_select_workspace_bytes", "NOALLOC_SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_F32, DSA_BF16 = 0, 1
OP_SPARSE_DECODE_ATTN, OP_ATTN_REPAIR, OP_PRR_DECODE_STEP = 1, 2, 3
EXPORTED = (
    "dsa_status_str", "dsa_version", "dsa_page_meta_build", "dsa_kv_append", "dsa_page_score", "dsa_page_score_ema",
    "dsa_page_select_topk",
    "dsa_page_select_progressive", "dsa_psa_decode", "dsa_sparse_decode_attn", "dsa_sparse_decode_attn_noalloc",
    "dsa_sparse_decode_attn_topk", "dsa_attn_repair", "dsa_prr_decode_step",
    "dsa_ema_predict_update", "dsa_prr_select", "dsa_prr_select_workspace_bytes", "dsa_prr_calibrate",
    "dsa_prr_calibrate_workspace_bytes",
    "dsa_signal_host", "dsa_block_sparse_prefill",
    "dsa_workspace_bytes",
)


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib.dsa_status_str(status).decode()} (status {status})")


class _KV(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32),
        ("num_slots", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
    ]


class _Stream(ctypes.Structure):
    _fields_ = [("kv_head_streaming", ctypes.c_void_p), ("sink", ctypes.c_int32), ("local", ctypes.c_int32)]


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python dynamic_sparse_attention_page_amd/build.py` (hipcc, gfx950)")
    L = ctypes.CDLL(path)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    KV, ST = ctypes.POINTER(_KV), ctypes.POINTER(_Stream)
    sig = {
        "dsa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "dsa_version": (ctypes.c_int, []),
        "dsa_page_meta_build": (ctypes.c_int, [KV, I32, P, I32, I32, P]),
        "dsa_kv_append": (ctypes.c_int, [KV, I32, P, P, P, P, P, P]),
        "dsa_page_score": (ctypes.c_int, [P, I32, KV, P, I32, ST, P, P]),
        "dsa_page_score_ema": (ctypes.c_int, [P, I32, KV, P, I32, ST, P, P, P, P, F32, F32, F32, I32, P]),
        "dsa_page_select_topk": (ctypes.c_int, [P, I32, I32, I32, P, I32, I32, ST, P, P, P]),
        "dsa_page_select_progressive": (ctypes.c_int, [P, I32, KV, P, F32, I32, ST, F32, P, P, P, P, P, P]),
        "dsa_psa_decode": (ctypes.c_int, [P, I32, KV, P, F32, I32, ST, F32, P, P, P, P, P, P, P]),
        "dsa_sparse_decode_attn": (ctypes.c_int, [P, I32, KV, P, P, I32, ST, F32, P, P, P, P, SZ, P]),
        "dsa_sparse_decode_attn_noalloc": (ctypes.c_int, [P, I32, KV, P, P, I32, ST, F32, P, P, P, P]),
        "dsa_sparse_decode_attn_topk": (ctypes.c_int, [P, I32, KV, P, I32, ST, F32, P, P, P, P, P, P, SZ, P]),
        "dsa_attn_repair": (ctypes.c_int, [P, I32, KV, P, P, P, P, I32, ST, F32, P, P, P, P, SZ, P]),
        "dsa_prr_decode_step": (ctypes.c_int, [P, I32, KV, P, I32, P, P, P, P, F32, F32, F32, I32, P, P, P, P, P, P,
                                               P, P, F32, P, P, P, P, SZ, P]),
        "dsa_ema_predict_update": (ctypes.c_int, [P, P, P, P, I64, F32, F32, F32, I32, P]),
        "dsa_prr_select": (ctypes.c_int, [P, I32, I32, I32, P, I32, I32, P, P, P, P, P, F32, F32, F32, I32, I32, P, P,
                                          P, P, P, P, P, SZ, P]),
        "dsa_prr_select_workspace_bytes": (SZ, [I32, I32, I32]),
        "dsa_prr_calibrate": (ctypes.c_int, [P, I32, I32, I32, P, I32, I32, P, P, P, SZ, P]),
        "dsa_prr_calibrate_workspace_bytes": (SZ, [I32, I32, I32]),
        "dsa_signal_host": (ctypes.c_int, [P, I32, P, P, I32, P]),
        "dsa_block_sparse_prefill": (ctypes.c_int, [P, P, P, I32, I32, I32, I32, ST, F32, P, P, P, P]),
        "dsa_workspace_bytes": (SZ, [I32, KV, I32, I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    return L


lib = _load()


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise DsaError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float32:
        return DSA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


@dataclass
class PagedKV:
    """Device-resident paged KV pool: k/v [num_slots][n_kv_heads][page_size][head_dim]
    (bf16 or fp32), page_table int32 [batch][max_pages], seq_lens int32 [batch]."""
    k: torch.Tensor
    v: torch.Tensor
    page_table: torch.Tensor
    seq_lens: torch.Tensor

    def __post_init__(self):
        for name in ("k", "v", "page_table", "seq_lens"):
            if not getattr(self, name).is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        if self.k.shape != self.v.shape or self.k.dtype != self.v.dtype or self.k.dim() != 4:
            raise ValueError("k and v must be equal-shaped [slots][heads][page][dim] tensors")
        if self.page_table.dtype != torch.int32 or self.seq_lens.dtype != torch.int32:
            raise TypeError("page_table and seq_lens must be int32")

    @property
    def num_slots(self): return self.k.shape[0]

    @property
    def n_kv_heads(self): return self.k.shape[1]

    @property
    def page_size(self): return self.k.shape[2]

    @property
    def head_dim(self): return self.k.shape[3]

    @property
    def batch(self): return self.page_table.shape[0]

    @property
    def max_pages(self): return self.page_table.shape[1]

    def c(self) -> _KV:
        return _KV(self.k.data_ptr(), self.v.data_ptr(), _dtype_code(self.k), self.num_slots, self.n_kv_heads,
                   self.page_size, self.head_dim, self.batch, self.max_pages, self.page_table.data_ptr(),
                   self.seq_lens.data_ptr())

    @staticmethod
    def from_numpy(k, v, page_table, seq_lens, dtype: str, device="cuda") -> "PagedKV":
        """Upload host arrays (bf16 as uint16 bit patterns, or float32)."""
        def up(x):
            if dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
            return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)
        return PagedKV(up(k), up(v), torch.from_numpy(np.ascontiguousarray(page_table, np.int32)).to(device),
                       torch.from_numpy(np.ascontiguousarray(seq_lens, np.int32)).to(device))


@dataclass
class Streaming:
    """Streaming (Lambda-mask) KV heads: flags[n_kv_heads], sink and local token counts."""
    flags: np.ndarray
    sink: int
    local: int

    def c(self):
        self._buf = np.ascontiguousarray(self.flags, dtype=np.uint8)
        return _Stream(self._buf.ctypes.data, int(self.sink), int(self.local))


def _stream_arg(streaming: Streaming | None):
    return None if streaming is None else ctypes.byref(streaming.c())


def upload_q(q: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(q).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(device)


_ws_cache: dict = {}


def _workspace(nbytes: int, device) -> torch.Tensor:
    """Scratch for calls given no `ws`: one buffer per (device, stream), so
    calls on different streams never share one.  Calls enqueued on one
    stream run in order, so they may share it.  A buffer that grows is
    replaced; the old one is marked as used by its stream, so the caching
    allocator does not hand its memory out before the work queued there has
    finished.  Kernels never need the content initialised."""
    dev = torch.device(device)
    stream = torch.cuda.current_stream(dev)
    key = (str(dev), stream.cuda_stream)
    t = _ws_cache.get(key)
    if t is None or t.numel() < nbytes:
        if t is not None:
            t.record_stream(stream)
        t = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _ws_cache[key] = t
    return t


def _default_scale(head_dim: int) -> float:
    return float(np.float32(1.0 / np.sqrt(head_dim)))


# --------------------------------------------------------------------------
# the C ABI, one function each
# --------------------------------------------------------------------------
def workspace_bytes(op: int, kv: PagedKV, n_q_heads: int, ids_stride: int) -> int:
    return int(lib.dsa_workspace_bytes(op, ctypes.byref(kv.c()), n_q_heads, ids_stride))


def page_meta_build(kv: PagedKV, logical_page: int | None = None, meta: torch.Tensor | None = None,
                    first_page: int = 0, n_pages: int = -1) -> torch.Tensor:
    """kmin/kmax per logical page: meta [num_slots][n_kv_heads][g][2][head_dim]."""
    lp = logical_page or kv.page_size
    g = kv.page_size // lp
    if meta is None:
        meta = torch.zeros((kv.num_slots, kv.n_kv_heads, g, 2, kv.head_dim), dtype=kv.k.dtype, device=kv.k.device)
    _check("dsa_page_meta_build", lib.dsa_page_meta_build(ctypes.byref(kv.c()), lp, _ptr(meta), first_page,
                                                          n_pages, _stream()))
    return meta


def kv_append(kv: PagedKV, k_new: torch.Tensor, v_new: torch.Tensor, meta: torch.Tensor,
              logical_page: int | None = None, new_seq_lens: torch.Tensor | None = None,
              status: torch.Tensor | None = None) -> torch.Tensor:
    """One token per sequence: k_new/v_new [batch][n_kv_heads][head_dim] go to
    position seq_lens[b], the page's kmin/kmax follow.  Returns the new
    lengths (by default written over kv.seq_lens, in place)."""
    lp = logical_page or kv.page_size
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dtype != kv.k.dtype or tuple(t.shape) != (kv.batch, kv.n_kv_heads, kv.head_dim) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [batch][n_kv_heads][head_dim] tensor of the pool dtype")
    if new_seq_lens is None:
        new_seq_lens = kv.seq_lens
    _check("dsa_kv_append", lib.dsa_kv_append(ctypes.byref(kv.c()), lp, _ptr(k_new), _ptr(v_new), _ptr(meta),
                                              _ptr(new_seq_lens), _ptr(status),
                                              _stream()))
    return new_seq_lens


def page_score(q: torch.Tensor, kv: PagedKV, meta: torch.Tensor, logical_page: int | None = None,
               streaming: Streaming | None = None, scores: torch.Tensor | None = None) -> torch.Tensor:
    """Page criticality scores [batch][n_kv_heads][max_pages] (float32)."""
    lp = logical_page or kv.page_size
    if scores is None:
        scores = torch.empty((kv.batch, kv.n_kv_heads, kv.max_pages), dtype=torch.float32, device=kv.k.device)
    _check("dsa_page_score", lib.dsa_page_score(_ptr(q), q.shape[1], ctypes.byref(kv.c()), _ptr(meta), lp,
                                                _stream_arg(streaming), _ptr(scores), _stream()))
    return scores


def page_score_ema(q: torch.Tensor, kv: PagedKV, meta: torch.Tensor, level: torch.Tensor, trend: torch.Tensor,
                   pred: torch.Tensor, alpha: float, beta: float, gamma: float, init: bool = False,
                   logical_page: int | None = None, streaming: Streaming | None = None,
                   scores: torch.Tensor | None = None) -> torch.Tensor:
    """page_score with PRR's EMA update of level/trend/pred in the same launch."""
    lp = logical_page or kv.page_size
    if scores is None:
        scores = torch.empty((kv.batch, kv.n_kv_heads, kv.max_pages), dtype=torch.float32, device=kv.k.device)
    _check("dsa_page_score_ema", lib.dsa_page_score_ema(
        _ptr(q), q.shape[1], ctypes.byref(kv.c()), _ptr(meta), lp, _stream_arg(streaming), _ptr(scores), _ptr(level),
        _ptr(trend), _ptr(pred), float(alpha), float(beta), float(gamma), 1 if init else 0, _stream()))
    return scores


def page_select_topk(scores: torch.Tensor, seq_lens: torch.Tensor, page_size: int, k: int,
                     streaming: Streaming | None = None, ids: torch.Tensor | None = None,
                     counts: torch.Tensor | None = None):
    """Top-k page ids [batch][n_kv_heads][k] (ascending, -1 padded) and counts."""
    B, H, N = scores.shape
    if ids is None:
        ids = torch.empty((B, H, k), dtype=torch.int32, device=scores.device)
    if counts is None:
        counts = torch.empty((B, H), dtype=torch.int32, device=scores.device)
    _check("dsa_page_select_topk", lib.dsa_page_select_topk(_ptr(scores), B, H, N, _ptr(seq_lens), page_size, k,
                                                            _stream_arg(streaming), _ptr(ids), _ptr(counts),
                                                            _stream()))
    return ids, counts


def page_select_progressive(q: torch.Tensor, kv: PagedKV, scores: torch.Tensor, threshold: float,
                            stop_mode: int = 0, scale: float | None = None, out=None,
                            streaming: Streaming | None = None):
    """PSA progressive selection + attention: (ids, counts, O, l, m); a
    streaming head visits its sink and local pages."""
    B, Hq = q.shape[0], q.shape[1]
    dev = kv.k.device
    if out is None:
        out = (torch.empty((kv.batch, kv.n_kv_heads, kv.max_pages), dtype=torch.int32, device=dev),
               torch.empty((kv.batch, kv.n_kv_heads), dtype=torch.int32, device=dev),
               torch.empty((B, Hq, kv.head_dim), dtype=torch.float32, device=dev),
               torch.empty((B, Hq), dtype=torch.float32, device=dev),
               torch.empty((B, Hq), dtype=torch.float32, device=dev))
    ids, counts, O, l, m = out
    sc = _default_scale(kv.head_dim) if scale is None else scale
    _check("dsa_page_select_progressive", lib.dsa_page_select_progressive(
        _ptr(q), Hq, ctypes.byref(kv.c()), _ptr(scores), float(threshold), stop_mode, _stream_arg(streaming), sc,
        _ptr(ids), _ptr(counts), _ptr(O), _ptr(l), _ptr(m), _stream()))
    return ids, counts, O, l, m


def psa_decode(q: torch.Tensor, kv: PagedKV, meta: torch.Tensor, threshold: float, stop_mode: int = 0,
               scale: float | None = None, out=None, streaming: Streaming | None = None):
    """page_score + page_select_progressive in one call (one launch when the
    rows cover the GPU's CUs): (scores, ids, counts, O, l, m)."""
    B, Hq = q.shape[0], q.shape[1]
    dev = kv.k.device
    if out is None:
        out = (torch.empty((kv.batch, kv.n_kv_heads, kv.max_pages), dtype=torch.float32, device=dev),
               torch.empty((kv.batch, kv.n_kv_heads, kv.max_pages), dtype=torch.int32, device=dev),
               torch.empty((kv.batch, kv.n_kv_heads), dtype=torch.int32, device=dev),
               torch.empty((B, Hq, kv.head_dim), dtype=torch.float32, device=dev),
               torch.empty((B, Hq), dtype=torch.float32, device=dev),
               torch.empty((B, Hq), dtype=torch.float32, device=dev))
    scores, ids, counts, O, l, m = out
    sc = _default_scale(kv.head_dim) if scale is None else scale
    _check("dsa_psa_decode", lib.dsa_psa_decode(
        _ptr(q), Hq, ctypes.byref(kv.c()), _ptr(meta), float(threshold), stop_mode, _stream_arg(streaming), sc,
        _ptr(scores), _ptr(ids), _ptr(counts), _ptr(O), _ptr(l), _ptr(m), _stream()))
    return scores, ids, counts, O, l, m


def sparse_decode_attn(q: torch.Tensor, kv: PagedKV, ids: torch.Tensor, counts: torch.Tensor,
                       streaming: Streaming | None = None, scale: float | None = None, out=None,
                       ws: torch.Tensor | None = None):
    """Attention over the selected pages: (O [B][Hq][D], l [B][Hq], m [B][Hq])."""
    B, Hq = q.shape[0], q.shape[1]
    stride = ids.shape[-1]
    dev = kv.k.device
    if out is None:
        out = (torch.empty((B, Hq, kv.head_dim), dtype=torch.float32, device=dev),
               torch.empty((B, Hq), dtype=torch.float32, device=dev),
               torch.empty((B, Hq), dtype=torch.float32, device=dev))
    O, l, m = out
    need = workspace_bytes(OP_SPARSE_DECODE_ATTN, kv, Hq, stride)
    if ws is None:
        ws = _workspace(need, dev)
    sc = _default_scale(kv.head_dim) if scale is None else scale
    _check("dsa_sparse_decode_attn", lib.dsa_sparse_decode_attn(
        _ptr(q), Hq, ctypes.byref(kv.c()), _ptr(ids), _ptr(counts), stride, _stream_arg(streaming), sc,
        _ptr(O), _ptr(l), _ptr(m), _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return O, l, m


NOALLOC_SCRATCH_BYTES = 8 << 20   # DSA_NOALLOC_SCRATCH_BYTES of include/dsa.h


def sparse_decode_attn_noalloc(q: torch.Tensor, kv: PagedKV, ids: torch.Tensor, counts: torch.Tensor,
                               O: torch.Tensor, l: torch.Tensor, m: torch.Tensor, streaming: Streaming | None = None,
                               scale: float | None = None):
    """sparse_decode_attn into caller-given outputs with no workspace: the
    library's fixed per-GPU scratch holds the partials (calls on one GPU must
    not overlap in time)."""
    sc = _default_scale(kv.head_dim) if scale is None else scale
    _check("dsa_sparse_decode_attn_noalloc", lib.dsa_sparse_decode_attn_noalloc(
        _ptr(q), q.shape[1], ctypes.byref(kv.c()), _ptr(ids), _ptr(counts), ids.shape[-1], _stream_arg(streaming),
        sc, _ptr(O), _ptr(l), _ptr(m), _stream()))
    return O, l, m


def sparse_decode_attn_topk(q: torch.Tensor, kv: PagedKV, scores: torch.Tensor, k: int,
                            streaming: Streaming | None = None, scale: float | None = None, out=None, ids=None,
                            counts=None, ws: torch.Tensor | None = None):
    """Top-k selection from `scores` and attention over the selected pages in
    one call: (ids [B][Hkv][k], counts [B][Hkv], O, l, m)."""
    B, Hq = q.shape[0], q.shape[1]
    dev = kv.k.device
    if out is None:
        out = (torch.empty((B, Hq, kv.head_dim), dtype=torch.float32, device=dev),
               torch.empty((B, Hq), dtype=torch.float32, device=dev),
               torch.empty((B, Hq), dtype=torch.float32, device=dev))
    if ids is None:
        ids = torch.empty((kv.batch, kv.n_kv_heads, k), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((kv.batch, kv.n_kv_heads), dtype=torch.int32, device=dev)
    O, l, m = out
    need = workspace_bytes(OP_SPARSE_DECODE_ATTN, kv, Hq, k)
    if ws is None:
        ws = _workspace(need, dev)
    sc = _default_scale(kv.head_dim) if scale is None else scale
    _check("dsa_sparse_decode_attn_topk", lib.dsa_sparse_decode_attn_topk(
        _ptr(q), Hq, ctypes.byref(kv.c()), _ptr(scores), k, _stream_arg(streaming), sc, _ptr(ids), _ptr(counts),
        _ptr(O), _ptr(l), _ptr(m), _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return ids, counts, O, l, m


def attn_repair(q: torch.Tensor, kv: PagedKV, a_ids, a_counts, p_ids, p_counts, O, l, m,
                scale: float | None = None, ws: torch.Tensor | None = None, streaming: Streaming | None = None):
    """Fold attention over A \\ P into the speculative (O, l, m) in place;
    with p_ids = p_counts = None, a_ids is the missing set itself."""
    Hq = q.shape[1]
    stride = a_ids.shape[-1]
    if (p_ids is None) != (p_counts is None):
        raise ValueError("give both p_ids and p_counts, or neither")
    if p_ids is not None and p_ids.shape[-1] != stride:
        raise ValueError("a_ids and p_ids must share the same stride")
    need = workspace_bytes(OP_ATTN_REPAIR, kv, Hq, stride)
    if ws is None:
        ws = _workspace(need, kv.k.device)
    sc = _default_scale(kv.head_dim) if scale is None else scale
    _check("dsa_attn_repair", lib.dsa_attn_repair(
        _ptr(q), Hq, ctypes.byref(kv.c()), _ptr(a_ids), _ptr(a_counts), _ptr(p_ids), _ptr(p_counts), stride,
        _stream_arg(streaming), sc, _ptr(O), _ptr(l), _ptr(m), _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return O, l, m


def prr_decode_step(q: torch.Tensor, kv: PagedKV, meta: torch.Tensor, scores: torch.Tensor, level: torch.Tensor,
                    trend: torch.Tensor, pred: torch.Tensor, alpha: float, beta: float, gamma: float, k: int,
                    p_cur: tuple, a_out: tuple, m_out: tuple, p_out: tuple, O, l, m,
                    logical_page: int | None = None, scale: float | None = None, ws: torch.Tensor | None = None):
    """One speculative PRR step in one call on the current stream (see
    dsa_prr_decode_step): scores + EMA, attention over P^t = p_cur, A^t into
    a_out, M^t into m_out, P^{t+1} into p_out, (O, l, m) over P^t u A^t.
    Every id tuple is (ids [batch][n_kv_heads][k], counts [batch][n_kv_heads])."""
    lp = logical_page or kv.page_size
    Hq = q.shape[1]
    need = workspace_bytes(OP_PRR_DECODE_STEP, kv, Hq, k)
    if ws is None:
        ws = _workspace(need, kv.k.device)
    sc = _default_scale(kv.head_dim) if scale is None else scale
    _check("dsa_prr_decode_step", lib.dsa_prr_decode_step(
        _ptr(q), Hq, ctypes.byref(kv.c()), _ptr(meta), lp, _ptr(scores), _ptr(level), _ptr(trend), _ptr(pred),
        float(alpha), float(beta), float(gamma), k, _ptr(p_cur[0]), _ptr(p_cur[1]), _ptr(a_out[0]), _ptr(a_out[1]),
        _ptr(m_out[0]), _ptr(m_out[1]), _ptr(p_out[0]), _ptr(p_out[1]), sc, _ptr(O), _ptr(l), _ptr(m), _ptr(ws),
        ws.numel() * ws.element_size(), _stream()))
    return O, l, m


def ema_predict_update(is_true, level: torch.Tensor, trend: torch.Tensor, pred: torch.Tensor,
                       alpha: float, beta: float, gamma: float, init: bool = False):
    """EMA predictor step over flat float32 arrays (is_true None = predict only)."""
    n = level.numel()
    _check("dsa_ema_predict_update", lib.dsa_ema_predict_update(
        _ptr(is_true), _ptr(level), _ptr(trend), _ptr(pred), n, float(alpha), float(beta), float(gamma),
        int(bool(init)), _stream()))
    return pred


def prr_select(scores: torch.Tensor, seq_lens: torch.Tensor, page_size: int, k: int, level: torch.Tensor | None,
               trend: torch.Tensor | None, pred: torch.Tensor, alpha: float, beta: float, gamma: float, init: bool,
               k_spec: int, a_ids: torch.Tensor, a_counts: torch.Tensor, p_ids: torch.Tensor,
               p_counts: torch.Tensor, p_cur: tuple | None = None, m_out: tuple | None = None,
               ws: torch.Tensor | None = None, split: bool = True):
    """A = top-k of scores; EMA update with scores; P = top-k_spec of the new
    prediction (see dsa_prr_select).  With p_cur = (ids, counts) of this
    step's speculative set and m_out = (ids, counts), also the missing set
    M = A \\ P_cur.  level = trend = None: pred already holds the updated
    prediction (page_score_ema).  Long rows use the split-row selection with `ws` (a
    shared scratch tensor when None); split=False passes no workspace, so
    each row takes one workgroup."""
    B, H, N = scores.shape
    pc_i, pc_c = p_cur if p_cur is not None else (None, None)
    m_i, m_c = m_out if m_out is not None else (None, None)
    nb = prr_select_workspace_bytes(B, H, N) if split else 0
    if nb and ws is None:
        ws = _workspace(nb, scores.device)
    if not nb:
        ws = None
    _check("dsa_prr_select", lib.dsa_prr_select(
        _ptr(scores), B, H, N, _ptr(seq_lens), page_size, k, _ptr(a_ids), _ptr(a_counts), _ptr(level), _ptr(trend),
        _ptr(pred), float(alpha), float(beta), float(gamma), 1 if init else 0, k_spec, _ptr(p_ids), _ptr(p_counts),
        _ptr(pc_i), _ptr(pc_c), _ptr(m_i), _ptr(m_c), _ptr(ws), ws.numel() if ws is not None else 0, _stream()))
    return a_ids, a_counts, p_ids, p_counts


def prr_select_workspace_bytes(batch: int, n_kv_heads: int, max_pages: int) -> int:
    return int(lib.dsa_prr_select_workspace_bytes(batch, n_kv_heads, max_pages))


CALIB_CANDIDATES = 80


def prr_calibrate(trace: torch.Tensor, n_valid: torch.Tensor, k: int, m: int, H: torch.Tensor | None = None,
                  best: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """PRR's EMA calibration over a score trace [steps][units][n] (float32):
    (H [units][80], best [units]); candidate c = (ia*5 + ib)*4 + ig."""
    if trace.dtype != torch.float32 or trace.dim() != 3 or not trace.is_contiguous():
        raise ValueError("trace must be a contiguous float32 [steps][units][n] tensor")
    T, U, N = trace.shape
    dev = trace.device
    if H is None:
        H = torch.empty((U, CALIB_CANDIDATES), dtype=torch.float32, device=dev)
    if best is None:
        best = torch.empty((U,), dtype=torch.int32, device=dev)
    need = int(lib.dsa_prr_calibrate_workspace_bytes(T, U, N))
    if ws is None:
        ws = _workspace(need, dev)
    _check("dsa_prr_calibrate", lib.dsa_prr_calibrate(_ptr(trace), T, U, N, _ptr(n_valid), k, m, _ptr(H), _ptr(best),
                                                      _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return H, best


def signal_host(src: torch.Tensor, host_dst: torch.Tensor, host_flag: torch.Tensor, seq: int):
    """Enqueue the zero-copy notification: src (device int32) into host_dst,
    then seq into host_flag[0]; both host tensors pinned int32."""
    for name, t in (("host_dst", host_dst), ("host_flag", host_flag)):
        if t.device.type != "cpu" or not t.is_pinned() or t.dtype != torch.int32:
            raise ValueError(f"{name} must be a pinned int32 host tensor")
    if src.dtype != torch.int32 or not src.is_contiguous() or host_dst.numel() < src.numel():
        raise ValueError("src must be contiguous int32 and fit in host_dst")
    _check("dsa_signal_host", lib.dsa_signal_host(_ptr(src), src.numel(), _ptr(host_dst), _ptr(host_flag), seq,
                                                  _stream()))


def wait_host_flag(host_flag: torch.Tensor, seq: int, timeout_s: float = 10.0) -> bool:
    """Poll a pinned flag written by signal_host until it equals seq (no
    device synchronisation); False on timeout."""
    import time
    view = host_flag.numpy()
    t_end = time.monotonic() + timeout_s
    while int(view[0]) != seq:
        if time.monotonic() > t_end:
            return False
    return True


def block_sparse_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, streaming: Streaming | None = None,
                         scale: float | None = None, out=None):
    """Prefill attention of one sequence: q [L][Hq][D], k, v [L][Hkv][D]
    (bf16) -> (O [L][Hq][D], l [L][Hq], m [L][Hq]) in float32."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 [L][heads][head_dim] tensor")
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (L, Hkv, D) or tuple(v.shape) != (L, Hkv, D):
        raise ValueError("k and v must be [L][n_kv_heads][head_dim] with q's L and head_dim")
    if out is None:
        out = (torch.empty((L, Hq, D), dtype=torch.float32, device=q.device),
               torch.empty((L, Hq), dtype=torch.float32, device=q.device),
               torch.empty((L, Hq), dtype=torch.float32, device=q.device))
    O, l, m = out
    sc = _default_scale(D) if scale is None else scale
    _check("dsa_block_sparse_prefill", lib.dsa_block_sparse_prefill(
        _ptr(q), _ptr(k), _ptr(v), L, Hq, Hkv, D, _stream_arg(streaming), sc, _ptr(O), _ptr(l), _ptr(m), _stream()))
    return O, l, m
