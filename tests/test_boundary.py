"""The C ABI boundary, on the CPU: the library loads, exports every function
include/dsa.h declares, and rejects bad arguments on the host (these paths
return before any HIP call, so no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


@pytest.fixture(scope="module")
def dsa():
    import dynamic_sparse_attention_page_amd as m
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_seven_steps():
    names = declared_functions()
    for step in ("page_meta_build", "page_score", "page_select_topk", "page_select_progressive",
                 "sparse_decode_attn", "attn_repair", "ema_predict_update"):
        assert f"dsa_{step}" in names


def test_library_exports_every_declared_symbol(dsa):
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (dsa_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    assert set(dsa.EXPORTED) == set(declared_functions())


def test_library_is_gfx950(dsa):
    """The embedded device code object targets gfx950."""
    data = open(dsa.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_status_strings(dsa):
    assert dsa.lib.dsa_status_str(0) == b"ok"
    assert b"workspace" in dsa.lib.dsa_status_str(-5)
    assert dsa.lib.dsa_version() >= 100


def _kv(dsa, **over):
    f = dict(k=16, v=16, dtype=1, num_slots=4, n_kv_heads=2, page_size=16, head_dim=128, batch=1,
             max_pages=4, page_table=32, seq_lens=48)
    f.update(over)
    return dsa._KV(**f)


def test_validation_errors(dsa):
    L = dsa.lib
    kv = _kv(dsa)
    P = ctypes.c_void_p
    ok_ptr = P(4096)
    # null descriptor / pointers
    assert L.dsa_page_meta_build(None, 16, ok_ptr, 0, -1, None) == -1
    assert L.dsa_page_score(None, 4, ctypes.byref(kv), ok_ptr, 16, None, ok_ptr, None) == -1
    # unsupported head_dim / page size / dtype
    assert L.dsa_page_score(ok_ptr, 4, ctypes.byref(_kv(dsa, head_dim=96)), ok_ptr, 16, None, ok_ptr, None) == -4
    assert L.dsa_page_score(ok_ptr, 4, ctypes.byref(_kv(dsa, page_size=48)), ok_ptr, 16, None, ok_ptr, None) == -4
    assert L.dsa_page_score(ok_ptr, 4, ctypes.byref(_kv(dsa, dtype=7)), ok_ptr, 16, None, ok_ptr, None) == -3
    # group size: 6 q heads over 2 kv heads = 3 (not a power of two); 5 not a multiple
    assert L.dsa_page_score(ok_ptr, 6, ctypes.byref(kv), ok_ptr, 16, None, ok_ptr, None) == -4
    assert L.dsa_page_score(ok_ptr, 5, ctypes.byref(kv), ok_ptr, 16, None, ok_ptr, None) == -2
    # logical page must be a multiple of 16 dividing the page
    assert L.dsa_page_meta_build(ctypes.byref(kv), 8, ok_ptr, 0, -1, None) == -2
    assert L.dsa_page_meta_build(ctypes.byref(_kv(dsa, page_size=64)), 48, ok_ptr, 0, -1, None) == -2
    # alignment
    assert L.dsa_page_score(P(4098), 4, ctypes.byref(kv), ok_ptr, 16, None, ok_ptr, None) == -6
    # top-k: k < 1, too many pages
    assert L.dsa_page_select_topk(ok_ptr, 1, 2, 4, ok_ptr, 16, 0, None, ok_ptr, ok_ptr, None) == -2
    assert L.dsa_page_select_topk(ok_ptr, 1, 2, 70000, ok_ptr, 16, 8, None, ok_ptr, ok_ptr, None) == -4
    # streaming list larger than k
    flags = (ctypes.c_uint8 * 2)(1, 0)
    st = dsa._Stream(ctypes.cast(flags, ctypes.c_void_p), 128, 256)
    assert L.dsa_page_select_topk(ok_ptr, 1, 2, 1024, ok_ptr, 64, 4, ctypes.byref(st), ok_ptr, ok_ptr, None) == -2
    # attention: workspace missing / too small, bad scale
    assert L.dsa_sparse_decode_attn(ok_ptr, 4, ctypes.byref(kv), ok_ptr, ok_ptr, 8, None, 0.088, ok_ptr, ok_ptr,
                                    ok_ptr, None, 0, None) == -5
    need = L.dsa_workspace_bytes(1, ctypes.byref(kv), 4, 8)
    assert need > 0
    assert L.dsa_sparse_decode_attn(ok_ptr, 4, ctypes.byref(kv), ok_ptr, ok_ptr, 8, None, 0.088, ok_ptr, ok_ptr,
                                    ok_ptr, ok_ptr, need - 1, None) == -5
    assert L.dsa_sparse_decode_attn(ok_ptr, 4, ctypes.byref(kv), ok_ptr, ok_ptr, 8, None, -1.0, ok_ptr, ok_ptr,
                                    ok_ptr, ok_ptr, need, None) == -2
    assert L.dsa_workspace_bytes(2, ctypes.byref(kv), 4, 8) >= need
    assert L.dsa_workspace_bytes(9, ctypes.byref(kv), 4, 8) == 0
    # progressive: bad stop mode, too many pages, G=8 unsupported
    assert L.dsa_page_select_progressive(ok_ptr, 4, ctypes.byref(kv), ok_ptr, ctypes.c_float(0.9), 2, None,
                                         ctypes.c_float(0.088), ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, None) == -2
    assert L.dsa_page_select_progressive(ok_ptr, 4, ctypes.byref(_kv(dsa, max_pages=65537)), ok_ptr,
                                         ctypes.c_float(0.9), 0, None, ctypes.c_float(0.088), ok_ptr, ok_ptr, ok_ptr,
                                         ok_ptr, ok_ptr, None) == -4
    # progressive: a streaming configuration with a negative window
    flags = ctypes.create_string_buffer(b"\x01\x00")
    bad_st = dsa._Stream(ctypes.cast(flags, ctypes.c_void_p), -1, 4)
    assert L.dsa_page_select_progressive(ok_ptr, 4, ctypes.byref(kv), ok_ptr, ctypes.c_float(0.9), 0,
                                         ctypes.byref(bad_st), ctypes.c_float(0.088), ok_ptr, ok_ptr, ok_ptr, ok_ptr,
                                         ok_ptr, None) == -2
    # psa_decode: bad stop mode, G=8 unsupported, missing metadata, too many pages
    assert L.dsa_psa_decode(ok_ptr, 4, ctypes.byref(kv), ok_ptr, ctypes.c_float(0.9), 2, None, ctypes.c_float(0.088),
                            ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, None) == -2
    assert L.dsa_psa_decode(ok_ptr, 16, ctypes.byref(kv), ok_ptr, ctypes.c_float(0.9), 0, None, ctypes.c_float(0.088),
                            ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, None) == -4
    assert L.dsa_psa_decode(ok_ptr, 4, ctypes.byref(kv), None, ctypes.c_float(0.9), 0, None, ctypes.c_float(0.088),
                            ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, None) == -1
    assert L.dsa_psa_decode(ok_ptr, 4, ctypes.byref(_kv(dsa, max_pages=65537)), ok_ptr, ctypes.c_float(0.9), 0, None,
                            ctypes.c_float(0.088), ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, None) == -4
    # append: null new rows / lengths, misaligned rows or metadata, bad logical page
    assert L.dsa_kv_append(ctypes.byref(kv), 16, None, ok_ptr, ok_ptr, ok_ptr, None, None) == -1
    assert L.dsa_kv_append(ctypes.byref(kv), 16, ok_ptr, ok_ptr, ok_ptr, None, None, None) == -1
    assert L.dsa_kv_append(ctypes.byref(kv), 16, P(4100), ok_ptr, ok_ptr, ok_ptr, None, None) == -6
    assert L.dsa_kv_append(ctypes.byref(kv), 16, ok_ptr, ok_ptr, P(4100), ok_ptr, None, None) == -6
    assert L.dsa_kv_append(ctypes.byref(kv), 32, ok_ptr, ok_ptr, ok_ptr, ok_ptr, None, None) == -2
    assert L.dsa_kv_append(ctypes.byref(_kv(dsa, k=0)), 16, ok_ptr, ok_ptr, ok_ptr, ok_ptr, None, None) == -1
    # calibration: too few steps, too many pages, null outputs, small workspace
    wsz = L.dsa_prr_calibrate_workspace_bytes(4, 2, 1000)
    assert wsz > 0 and L.dsa_prr_calibrate_workspace_bytes(1, 2, 1000) == 0
    assert L.dsa_prr_calibrate_workspace_bytes(4, 2, 70000) == 0
    assert L.dsa_prr_calibrate(ok_ptr, 1, 2, 1000, ok_ptr, 8, 8, ok_ptr, None, ok_ptr, wsz, None) == -2
    assert L.dsa_prr_calibrate(ok_ptr, 4, 2, 70000, ok_ptr, 8, 8, ok_ptr, None, ok_ptr, wsz, None) == -4
    assert L.dsa_prr_calibrate(ok_ptr, 4, 2, 1000, ok_ptr, -1, 8, ok_ptr, None, ok_ptr, wsz, None) == -2
    assert L.dsa_prr_calibrate(ok_ptr, 4, 2, 1000, None, 8, 8, ok_ptr, None, ok_ptr, wsz, None) == -1
    assert L.dsa_prr_calibrate(ok_ptr, 4, 2, 1000, ok_ptr, 8, 8, None, None, ok_ptr, wsz, None) == -1
    assert L.dsa_prr_calibrate(ok_ptr, 4, 2, 1000, ok_ptr, 8, 8, ok_ptr, None, ok_ptr, wsz - 1, None) == -5
    assert L.dsa_prr_calibrate(None, 4, 0, 1000, None, 8, 8, None, None, None, 0, None) == 0
    # prefill: inconsistent heads, head_dim, scale, null output
    F = ctypes.c_float
    assert L.dsa_block_sparse_prefill(ok_ptr, ok_ptr, ok_ptr, 64, 6, 4, 128, None, F(0.1), ok_ptr, ok_ptr, ok_ptr,
                                      None) == -2
    assert L.dsa_block_sparse_prefill(ok_ptr, ok_ptr, ok_ptr, 64, 8, 4, 96, None, F(0.1), ok_ptr, ok_ptr, ok_ptr,
                                      None) == -4
    assert L.dsa_block_sparse_prefill(ok_ptr, ok_ptr, ok_ptr, 64, 8, 4, 128, None, F(0.0), ok_ptr, ok_ptr, ok_ptr,
                                      None) == -2
    assert L.dsa_block_sparse_prefill(ok_ptr, ok_ptr, ok_ptr, 64, 8, 4, 128, None, F(0.1), None, ok_ptr, ok_ptr,
                                      None) == -1
    assert L.dsa_block_sparse_prefill(None, None, None, 0, 8, 4, 128, None, F(0.1), None, None, None, None) == 0
    # PRR selection: missing set without this step's P, or with P aliasing the next one
    args = [ok_ptr, 1, 2, 64, ok_ptr, 16, 8, ok_ptr, ok_ptr, P(8192), P(12288), P(16384), F(0.6), F(0.3), F(0.25), 0, 8,
            ok_ptr, ok_ptr]
    assert L.dsa_prr_select(*args, None, None, ok_ptr, ok_ptr, None, 0, None) == -1
    assert L.dsa_prr_select(*args, ok_ptr, P(20480), ok_ptr, ok_ptr, None, 0, None) == -2
    # the prediction already updated: level and trend both NULL, not one of them
    assert L.dsa_prr_select(ok_ptr, 1, 2, 64, ok_ptr, 16, 8, ok_ptr, ok_ptr, None, P(12288), P(16384), F(0.6), F(0.3),
                            F(0.25), 0, 8, ok_ptr, ok_ptr, None, None, None, None, None, 0, None) == -1
    # split-row selection of long rows: workspace size, too small a workspace
    assert L.dsa_prr_select_workspace_bytes(1, 2, 4096) == 0
    need = L.dsa_prr_select_workspace_bytes(1, 2, 8192)
    assert need >= 2 * 2 * 8192 * 8
    long_args = list(args)
    long_args[3] = 8192
    assert L.dsa_prr_select(*long_args, None, None, None, None, ok_ptr, need - 1, None) == -5
    # scores with the EMA update: missing state, state aliasing the scores
    assert L.dsa_page_score_ema(ok_ptr, 4, ctypes.byref(kv), ok_ptr, 16, None, ok_ptr, None, P(8192), P(12288),
                                F(0.6), F(0.3), F(0.25), 0, None) == -1
    assert L.dsa_page_score_ema(ok_ptr, 4, ctypes.byref(kv), ok_ptr, 16, None, P(8192), P(8192), P(12288), P(16384),
                                F(0.6), F(0.3), F(0.25), 0, None) == -2
    # repair: P ids without counts
    assert L.dsa_attn_repair(ok_ptr, 4, ctypes.byref(kv), ok_ptr, ok_ptr, ok_ptr, None, 8, None, F(0.088), ok_ptr,
                             ok_ptr, ok_ptr, ok_ptr, 1 << 30, None) == -1
    # one-call PRR step (16 q heads over 2 KV heads): bad k, logical pages smaller than the page, fp32 KV,
    # a NULL output, aliased EMA state, P^t aliasing P^{t+1}, too small a workspace; batch 0 is a no-op
    def step(n_q=32, kvd=kv, k=8, lvl=P(8192), p_cur=P(20480), p_nxt=P(24576), O=ok_ptr, wsb=None, lp=16):
        need = L.dsa_workspace_bytes(3, ctypes.byref(kvd), n_q, max(k, 1))
        return L.dsa_prr_decode_step(ok_ptr, n_q, ctypes.byref(kvd), ok_ptr, lp, ok_ptr, lvl, P(12288), P(16384),
                                     F(0.6), F(0.3), F(0.25), k, p_cur, P(28672), ok_ptr, ok_ptr, ok_ptr, ok_ptr,
                                     p_nxt, P(32768), F(0.088), O, ok_ptr, ok_ptr, ok_ptr,
                                     need if wsb is None else wsb, None)
    assert L.dsa_workspace_bytes(3, ctypes.byref(kv), 32, 8) > L.dsa_workspace_bytes(2, ctypes.byref(kv), 32, 8)
    assert step(k=0) == -2
    assert step(kvd=_kv(dsa, page_size=32), lp=16) == -4
    assert step(kvd=_kv(dsa, dtype=0)) == -4
    assert step(O=None) == -1
    assert step(lvl=P(12288)) == -2
    assert step(p_nxt=P(20480)) == -2
    assert step(wsb=1024) == -5
    kv0 = _kv(dsa, batch=0, page_table=0, seq_lens=0)
    assert L.dsa_prr_decode_step(None, 32, ctypes.byref(kv0), None, 16, None, None, None, None, F(0.6), F(0.3),
                                 F(0.25), 8, None, None, None, None, None, None, None, None, F(0.088), None, None,
                                 None, None, 0, None) == 0
    # host signal: negative count, missing flag or destination
    assert L.dsa_signal_host(ok_ptr, -1, ok_ptr, ok_ptr, 1, None) == -2
    assert L.dsa_signal_host(ok_ptr, 4, ok_ptr, None, 1, None) == -1
    assert L.dsa_signal_host(ok_ptr, 4, None, ok_ptr, 1, None) == -1
    # EMA: negative n, aliasing
    assert L.dsa_ema_predict_update(None, ok_ptr, P(8192), ok_ptr, 10, 0.6, 0.3, 0.25, 0, None) == -2
    assert L.dsa_ema_predict_update(None, ok_ptr, P(8192), P(12288), -1, 0.6, 0.3, 0.25, 0, None) == -2


def test_empty_inputs_are_noops(dsa):
    """batch 0 / n 0: nothing to do, nothing enqueued, success."""
    L = dsa.lib
    kv = _kv(dsa, batch=0, page_table=0, seq_lens=0)
    P = ctypes.c_void_p
    assert L.dsa_page_meta_build(ctypes.byref(kv), 16, None, 0, -1, None) == 0
    assert L.dsa_kv_append(ctypes.byref(_kv(dsa, batch=0, page_table=0, seq_lens=0)), 16, None, None, None, None,
                           None, None) == 0
    assert L.dsa_page_score(None, 4, ctypes.byref(kv), None, 16, None, None, None) == 0
    assert L.dsa_page_select_topk(None, 0, 2, 4, None, 16, 4, None, None, None, None) == 0
    assert L.dsa_ema_predict_update(None, None, None, None, 0, 0.6, 0.3, 0.25, 0, None) == 0
    assert L.dsa_sparse_decode_attn(None, 4, ctypes.byref(kv), None, None, 8, None, 0.1, None, None, None, None,
                                    0, None) == 0


def test_noalloc_validation(dsa):
    """The no-allocation variant validates like the workspace call and
    refuses, before any HIP call, a shape whose partials exceed its fixed
    scratch; batch 0 is a no-op."""
    L = dsa.lib
    P, F = ctypes.c_void_p, ctypes.c_float
    ok_ptr = P(4096)
    kv = _kv(dsa)
    assert L.dsa_sparse_decode_attn_noalloc(None, 4, ctypes.byref(kv), ok_ptr, ok_ptr, 8, None, F(0.088), ok_ptr,
                                            ok_ptr, ok_ptr, None) == -1
    assert L.dsa_sparse_decode_attn_noalloc(ok_ptr, 4, ctypes.byref(kv), ok_ptr, ok_ptr, 0, None, F(0.088), ok_ptr,
                                            ok_ptr, ok_ptr, None) == -2
    big = _kv(dsa, max_pages=8192)
    need = L.dsa_workspace_bytes(1, ctypes.byref(big), 32, 8192)
    assert need > dsa.NOALLOC_SCRATCH_BYTES
    assert L.dsa_sparse_decode_attn_noalloc(ok_ptr, 32, ctypes.byref(big), ok_ptr, ok_ptr, 8192, None, F(0.088),
                                            ok_ptr, ok_ptr, ok_ptr, None) == -8
    assert b"no-allocation scratch" in L.dsa_status_str(-8)
    empty = _kv(dsa, batch=0, page_table=0, seq_lens=0)
    assert L.dsa_sparse_decode_attn_noalloc(None, 4, ctypes.byref(empty), None, None, 8, None, F(0.1), None, None,
                                            None, None) == 0
