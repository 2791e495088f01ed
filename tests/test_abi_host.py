"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every function declared in include/lisa.h,
size its workspaces, and reject bad arguments on the host with a status code
before any HIP call.
"""
import ctypes
import os
import re

import pytest

import long_context_attention_lightning_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from long_context_attention_lightning_amd import build as B
        B.build()
    return L.library()


def _declared():
    txt = open(os.path.join(ROOT, "include", "lisa.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lisa_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value
    assert set(names) == set(L.EXPORTED_SYMBOLS)


def _qwen7b_decode_shape(**kw):
    base = dict(B=1, H_q=28, H_kv=4, d=128, H_I=4, H_Ik=4, d_I=64, hidden=3584, M=2048,
                cap=16384, max_len=16384)
    base.update(kw)
    return L.make_shape(**base)


def test_workspace_sizes(lib):
    sh = _qwen7b_decode_shape()
    dec = L.lisa_workspace_bytes(sh, L.LISA_OP_DECODE)
    assert dec > 16384 * 4          # holds at least one score row
    pre = L.lisa_workspace_bytes(sh, L.LISA_OP_PREFILL, 16384)
    assert pre > (16384 - 2048) * 16384 * 4
    # batch 32: one score row per sequence at least
    assert L.lisa_workspace_bytes(_qwen7b_decode_shape(B=32), L.LISA_OP_DECODE) > 32 * 16384 * 4
    assert L.lisa_workspace_bytes(sh, L.LISA_OP_DENSE_DECODE) > 0
    assert L.lisa_workspace_bytes(sh, L.LISA_OP_TOPK_PREFILL, 4096) > 0
    assert L.lisa_workspace_bytes(sh, 99) == 0
    assert "op" in L.lisa_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(H_kv=5), L.LisaError),
    (dict(H_L=27), L.LisaError),
    (dict(M=0), L.LisaError),
    (dict(B=0), L.LisaError),
    (dict(hidden=0), L.LisaError),
    (dict(chunk=32), L.LisaError),
    (dict(d=96), L.LisaError),
    (dict(max_len=20000), L.LisaError),
    (dict(H_Ik=3), L.LisaError),
    (dict(dtype=7), L.LisaError),
])
def test_bad_shapes_are_rejected(lib, kw, code):
    sh = _qwen7b_decode_shape(**{k: v for k, v in kw.items() if k != "dtype"})
    if "dtype" in kw:
        sh.dtype = kw["dtype"]
    assert L.lisa_workspace_bytes(sh, L.LISA_OP_DECODE) == 0
    assert L.lisa_last_error() != ""


def test_unsupported_vs_invalid_codes(lib):
    f = lib.lisa_workspace_bytes
    sh = _qwen7b_decode_shape(d=96)
    assert f(ctypes.byref(sh), 0, 0) == 0
    assert "head dim" in L.lisa_last_error()
    assert L.lisa_status_string(-2) == "unsupported configuration"
    assert L.lisa_status_string(-1) == "invalid argument"
    assert L.lisa_status_string(-3) == "workspace too small"
    assert L.lisa_status_string(-4) == "HIP error"


def _call_decode(sh, ptr=16, ws_bytes=1 << 40, **over):
    args = dict(seq_lens=ptr, q=ptr, k_new=ptr, v_new=ptr, q_idx=ptr, k_idx_new=ptr, q_lin=ptr,
                k_lin=ptr, v_lin=ptr, x=ptr, w_gate=ptr, w_idx=ptr, k_cache=ptr, v_cache=ptr,
                k_idx_cache=ptr, S=ptr, z=ptr, out=ptr, idx_out=None, ws=ptr)
    args.update(over)
    lib = L.library()
    return lib.lisa_decode_step(ctypes.byref(sh), *args.values(), ws_bytes, None)


def test_decode_rejects_null_misaligned_and_small_workspace(lib):
    sh = _qwen7b_decode_shape()
    assert _call_decode(sh, q=None) == -1
    assert "q is NULL" in L.lisa_last_error()
    assert _call_decode(sh, k_cache=24) == -1
    assert "aligned" in L.lisa_last_error()
    assert _call_decode(sh, ws_bytes=100) == -3
    assert _call_decode(_qwen7b_decode_shape(H_q=27, H_kv=4)) == -1
    assert _call_decode(_qwen7b_decode_shape(H_q=72, H_kv=8)) == -2


def test_prefill_and_topk_reject_bad_lengths(lib):
    sh = _qwen7b_decode_shape()
    p = 16
    rc = lib.lisa_prefill(ctypes.byref(sh), 0, *([p] * 16), 1 << 40, None)
    assert rc == -1 and "n 0" in L.lisa_last_error()
    rc = lib.lisa_prefill(ctypes.byref(sh), 20000, *([p] * 16), 1 << 40, None)
    assert rc == -1
    rc = lib.lisa_indexer_topk(ctypes.byref(sh), 7, 10, p, p, p, p, None, 0, None, p, p, 1 << 40, None)
    assert rc == -1 and "rows_mode" in L.lisa_last_error()
    rc = lib.lisa_indexer_topk(ctypes.byref(sh), L.LISA_ROWS_DECODE, 0, p, p, p, p, p, 100, None, p, p,
                               1 << 40, None)
    assert rc == -1 and "scores_ld" in L.lisa_last_error()
    rc = lib.lisa_linear_state_update(ctypes.byref(sh), 0, p, p, p, p, None)
    assert rc == -1


def test_kernel_names(lib):
    names = [L.lisa_kernel_name(i) for i in range(9)]
    assert names[0] == "decode_phase_a" and None not in names
    assert L.lisa_kernel_name(99) is None


def test_segment_correct_rejects_bad_args(lib):
    sh = _qwen7b_decode_shape()
    buf = (ctypes.c_float * 64)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    rc = lib.lisa_segment_correct(ctypes.byref(sh), p, p, p, p, p, p, 0, 0.5, None)
    assert rc == -1 and "segment number" in L.lisa_last_error()
    rc = lib.lisa_segment_correct(ctypes.byref(sh), p, p, p, p, p, p, 1, float("nan"), None)
    assert rc == -1 and "alpha" in L.lisa_last_error()
    rc = lib.lisa_segment_correct(ctypes.byref(sh), p, None, p, p, p, p, 1, 0.5, None)
    assert rc == -1


def test_attention_mass_workspace_and_rejections(lib):
    sh = _qwen7b_decode_shape()
    ws = L.lisa_workspace_bytes(sh, L.LISA_OP_MASS, 3)
    assert ws >= 3 * 28 * 16384 * 4 + 3 * 28 * 2048 * 4  # logits and the bound's index sets
    assert L.lisa_workspace_bytes(sh, L.LISA_OP_MASS, 0) == 0
    buf = (ctypes.c_float * 64)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    rc = lib.lisa_attention_mass(ctypes.byref(sh), -1, None, p, p, p, p, p, None, p, 1 << 40, None)
    assert rc == -1 and "n_rows" in L.lisa_last_error()
    rc = lib.lisa_attention_mass(ctypes.byref(sh), 3, None, None, p, p, p, p, None, p, 1 << 40, None)
    assert rc == -1 and "row_len" in L.lisa_last_error()
    rc = lib.lisa_attention_mass(ctypes.byref(sh), 3, None, p, p, p, p, p, None, p, ws - 1, None)
    assert rc == -3
    assert lib.lisa_attention_mass(ctypes.byref(sh), 0, None, None, None, None, None, None, None, None, 0,
                                   None) == 0  # no rows: nothing to do
    bad = _qwen7b_decode_shape(max_len=0)
    rc = lib.lisa_attention_mass(ctypes.byref(bad), 3, None, p, p, p, p, p, None, p, 1 << 40, None)
    assert rc == -1 and "max_len" in L.lisa_last_error()


def test_indexer_kl_rejections(lib):
    buf = (ctypes.c_float * 64)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    sh = _qwen7b_decode_shape(H_I=8, H_Ik=8)  # 28 teacher heads do not split over 8 indexer heads
    rc = lib.lisa_indexer_kl(ctypes.byref(sh), 64, p, p, p, p, p, None, None)
    assert rc == -2 and "H_I" in L.lisa_last_error()
    sh = _qwen7b_decode_shape()
    rc = lib.lisa_indexer_kl(ctypes.byref(sh), 64, p, p, p, p, None, None, None)
    assert rc == -1 and "kl_out" in L.lisa_last_error()
    rc = lib.lisa_indexer_kl(ctypes.byref(sh), 0, p, p, p, p, p, None, None)
    assert rc == -1
    win = _qwen7b_decode_shape(flags=L.LISA_SLIDING_WINDOW)
    rc = lib.lisa_indexer_kl(ctypes.byref(win), 64, p, p, p, p, p, None, None)
    assert rc == -1 and "sliding-window" in L.lisa_last_error()


def test_candidate_dropout_rejections(lib):
    buf = (ctypes.c_float * 64)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    sh = _qwen7b_decode_shape()
    ws = L.lisa_workspace_bytes(sh, L.LISA_OP_DROPOUT_DECODE)
    assert ws >= 16384 * 4 + 2048 * 4
    assert L.lisa_workspace_bytes(sh, L.LISA_OP_DROPOUT_PREFILL, 4096) > 4096 * 4096 * 4
    f = lib.lisa_candidate_dropout
    assert f(ctypes.byref(sh), 0, 0, p, p, p, 16384, 0, ctypes.c_float(0.2), p, p, ws, None) == -1
    assert "n_cand" in L.lisa_last_error()
    assert f(ctypes.byref(sh), 0, 0, p, p, p, 16384, 2458, ctypes.c_float(float("nan")), p, p, ws, None) == -1
    assert f(ctypes.byref(sh), 0, 0, p, p, p, 16382, 2458, ctypes.c_float(0.2), p, p, ws, None) == -1
    assert "scores_ld" in L.lisa_last_error()
    assert f(ctypes.byref(sh), 0, 0, p, p, None, 16384, 2458, ctypes.c_float(0.2), p, p, ws, None) == -1
    assert f(ctypes.byref(sh), 0, 0, p, p, p, 16384, 2458, ctypes.c_float(0.2), p, p, 100, None) == -3
    assert f(ctypes.byref(sh), 7, 0, p, p, p, 16384, 2458, ctypes.c_float(0.2), p, p, ws, None) == -1
