"""Python binding of liblisa.so, the MI355X LISA attention-layer library.

The functions carry the names of the C entry points declared in
include/lisa.h and only marshal arguments: torch tensors become device
pointers, the current torch stream becomes the HIP stream, and a negative
status raises ``LisaError``.  Every step of the layer runs in the library's
HIP kernels; there is no fallback path.  Importing this module does not load
the library; the first call does, and raises ``LisaLibraryMissing`` if
``liblisa.so`` has not been built (``python -m
long_context_attention_lightning_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "LisaError", "LisaLibraryMissing", "lisa_shape", "make_shape", "library",
    "lisa_workspace_bytes", "lisa_decode_step", "lisa_decode_step_noalloc", "lisa_prefill", "lisa_indexer_topk",
    "lisa_linear_state_update", "lisa_segment_correct", "lisa_dense_decode", "lisa_attention_mass",
    "lisa_indexer_kl", "lisa_candidate_dropout", "lisa_status_string", "lisa_last_error", "lisa_timing_enable",
    "lisa_timing_count", "lisa_kernel_name",
    "LISA_DECODE_SCRATCH_BYTES",
    "workspace", "LISA_F32", "LISA_BF16", "LISA_LINEAR_UNNORMALIZED", "LISA_SLIDING_WINDOW",
    "LISA_OP_DECODE", "LISA_OP_PREFILL", "LISA_OP_TOPK_DECODE", "LISA_OP_TOPK_PREFILL",
    "LISA_OP_LINEAR_UPDATE", "LISA_OP_DENSE_DECODE", "LISA_OP_MASS",
    "LISA_OP_DROPOUT_DECODE", "LISA_OP_DROPOUT_PREFILL", "LISA_ROWS_DECODE", "LISA_ROWS_PREFILL",
    "EXPORTED_SYMBOLS", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblisa.so")

LISA_OK = 0
LISA_F32, LISA_BF16 = 0, 1
LISA_LINEAR_UNNORMALIZED = 1
LISA_SLIDING_WINDOW = 2
(LISA_OP_DECODE, LISA_OP_PREFILL, LISA_OP_TOPK_DECODE, LISA_OP_TOPK_PREFILL,
 LISA_OP_LINEAR_UPDATE, LISA_OP_DENSE_DECODE, LISA_OP_MASS, LISA_OP_DROPOUT_DECODE,
 LISA_OP_DROPOUT_PREFILL) = range(9)
LISA_ROWS_DECODE, LISA_ROWS_PREFILL = 0, 1
LISA_DECODE_SCRATCH_BYTES = 4 << 20

EXPORTED_SYMBOLS = (
    "lisa_workspace_bytes", "lisa_decode_step", "lisa_decode_step_noalloc", "lisa_prefill", "lisa_indexer_topk",
    "lisa_linear_state_update", "lisa_segment_correct", "lisa_dense_decode", "lisa_attention_mass",
    "lisa_indexer_kl", "lisa_candidate_dropout", "lisa_status_string", "lisa_last_error", "lisa_timing_enable",
    "lisa_timing_count", "lisa_kernel_name",
)


class LisaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status}")


class LisaLibraryMissing(ImportError):
    pass


class lisa_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "B", "H_q", "H_kv", "d", "H_I", "H_Ik", "d_I", "H_L", "hidden", "M", "cap",
        "max_len", "chunk", "dtype")] + [("flags", ctypes.c_uint32)]

    def __repr__(self):
        return "lisa_shape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


def make_shape(B, H_q, H_kv, d, H_I, H_Ik, d_I, hidden, M, cap, max_len=0, H_L=None,
               chunk=64, dtype="bf16", flags=0) -> lisa_shape:
    dt = {"bf16": LISA_BF16, "f32": LISA_F32, torch.bfloat16: LISA_BF16,
          torch.float32: LISA_F32, LISA_BF16: LISA_BF16, LISA_F32: LISA_F32}[dtype]
    return lisa_shape(B, H_q, H_kv, d, H_I, H_Ik, d_I, H_q if H_L is None else H_L, hidden,
                      M, cap, max_len, chunk, dt, flags)


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def library() -> ctypes.CDLL:
    """Load liblisa.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LisaLibraryMissing(
            f"{LIB_PATH} is missing: build it with __graft_entry__.build() or "
            "python -m long_context_attention_lightning_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    sp = ctypes.POINTER(lisa_shape)
    lib.lisa_workspace_bytes.argtypes = [sp, ctypes.c_int, _I32]
    lib.lisa_workspace_bytes.restype = ctypes.c_size_t
    lib.lisa_decode_step.argtypes = [sp] + [_P] * 20 + [ctypes.c_size_t, _P]
    lib.lisa_decode_step_noalloc.argtypes = [sp] + [_P] * 19 + [_P]
    lib.lisa_decode_step.restype = ctypes.c_int
    lib.lisa_prefill.argtypes = [sp, _I32] + [_P] * 16 + [ctypes.c_size_t, _P]
    lib.lisa_prefill.restype = ctypes.c_int
    lib.lisa_indexer_topk.argtypes = [sp, ctypes.c_int, _I32, _P, _P, _P, _P, _P, ctypes.c_int64,
                                      _P, _P, _P, ctypes.c_size_t, _P]
    lib.lisa_indexer_topk.restype = ctypes.c_int
    lib.lisa_linear_state_update.argtypes = [sp, _I32, _P, _P, _P, _P, _P]
    lib.lisa_linear_state_update.restype = ctypes.c_int
    lib.lisa_segment_correct.argtypes = [sp, _P, _P, _P, _P, _P, _P, _I32, ctypes.c_float, _P]
    lib.lisa_segment_correct.restype = ctypes.c_int
    lib.lisa_dense_decode.argtypes = [sp, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.lisa_dense_decode.restype = ctypes.c_int
    lib.lisa_attention_mass.argtypes = [sp, _I32, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.lisa_attention_mass.restype = ctypes.c_int
    lib.lisa_indexer_kl.argtypes = [sp, _I32, _P, _P, _P, _P, _P, _P, _P]
    lib.lisa_indexer_kl.restype = ctypes.c_int
    lib.lisa_candidate_dropout.argtypes = [sp, ctypes.c_int, _I32, _P, _P, _P, ctypes.c_int64, _I32, ctypes.c_float,
                                           _P, _P, ctypes.c_size_t, _P]
    lib.lisa_candidate_dropout.restype = ctypes.c_int
    lib.lisa_status_string.argtypes = [ctypes.c_int]
    lib.lisa_status_string.restype = ctypes.c_char_p
    lib.lisa_last_error.argtypes = []
    lib.lisa_last_error.restype = ctypes.c_char_p
    lib.lisa_timing_enable.argtypes = [ctypes.c_int, _P, _P, ctypes.c_int]
    lib.lisa_timing_enable.restype = ctypes.c_int
    lib.lisa_timing_count.argtypes = []
    lib.lisa_timing_count.restype = ctypes.c_int
    lib.lisa_kernel_name.argtypes = [ctypes.c_int]
    lib.lisa_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def lisa_status_string(status: int) -> str:
    return library().lisa_status_string(status).decode()


def lisa_last_error() -> str:
    return library().lisa_last_error().decode()


def lisa_kernel_name(kernel_id: int) -> Optional[str]:
    r = library().lisa_kernel_name(kernel_id)
    return None if r is None else r.decode()


def _check(rc: int, what: str):
    if rc != LISA_OK:
        raise LisaError(rc, f"{what}: {lisa_status_string(rc)}: {lisa_last_error()}")


def _ptr(t, name: str = "", dtype=None):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _act(shape: lisa_shape):
    return torch.bfloat16 if shape.dtype == LISA_BF16 else torch.float32


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def lisa_workspace_bytes(shape: lisa_shape, op: int, n: int = 0) -> int:
    return int(library().lisa_workspace_bytes(ctypes.byref(shape), op, n))


def workspace(shape: lisa_shape, op: int, n: int = 0, device="cuda") -> torch.Tensor:
    nb = lisa_workspace_bytes(shape, op, n)
    if nb == 0:
        raise LisaError(-1, f"lisa_workspace_bytes: {lisa_last_error()}")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def lisa_decode_step(shape, seq_lens, q, k_new, v_new, q_idx, k_idx_new, q_lin, k_lin, v_lin,
                     x, w_gate, w_idx, k_cache, v_cache, k_idx_cache, S, z, out, idx_out, ws,
                     stream=None):
    T = _act(shape)
    rc = library().lisa_decode_step(
        ctypes.byref(shape), _ptr(seq_lens, "seq_lens", torch.int32),
        _ptr(q, "q", T), _ptr(k_new, "k_new", T), _ptr(v_new, "v_new", T),
        _ptr(q_idx, "q_idx", T), _ptr(k_idx_new, "k_idx_new", T),
        _ptr(q_lin, "q_lin", T), _ptr(k_lin, "k_lin", T), _ptr(v_lin, "v_lin", T),
        _ptr(x, "x", T), _ptr(w_gate, "w_gate", T), _ptr(w_idx, "w_idx", torch.float32),
        _ptr(k_cache, "k_cache", T), _ptr(v_cache, "v_cache", T), _ptr(k_idx_cache, "k_idx_cache", T),
        _ptr(S, "S", torch.float32), _ptr(z, "z", torch.float32), _ptr(out, "out", T),
        _ptr(idx_out, "idx_out", torch.int32), _ptr(ws, "ws"), 0 if ws is None else ws.numel(),
        _stream(stream))
    _check(rc, "lisa_decode_step")


def lisa_decode_step_noalloc(shape, seq_lens, q, k_new, v_new, q_idx, k_idx_new, q_lin, k_lin, v_lin,
                             x, w_gate, w_idx, k_cache, v_cache, k_idx_cache, S, z, out, idx_out, stream=None):
    T = _act(shape)
    rc = library().lisa_decode_step_noalloc(
        ctypes.byref(shape), _ptr(seq_lens, "seq_lens", torch.int32),
        _ptr(q, "q", T), _ptr(k_new, "k_new", T), _ptr(v_new, "v_new", T),
        _ptr(q_idx, "q_idx", T), _ptr(k_idx_new, "k_idx_new", T),
        _ptr(q_lin, "q_lin", T), _ptr(k_lin, "k_lin", T), _ptr(v_lin, "v_lin", T),
        _ptr(x, "x", T), _ptr(w_gate, "w_gate", T), _ptr(w_idx, "w_idx", torch.float32),
        _ptr(k_cache, "k_cache", T), _ptr(v_cache, "v_cache", T), _ptr(k_idx_cache, "k_idx_cache", T),
        _ptr(S, "S", torch.float32), _ptr(z, "z", torch.float32), _ptr(out, "out", T),
        _ptr(idx_out, "idx_out", torch.int32), _stream(stream))
    _check(rc, "lisa_decode_step_noalloc")


def lisa_prefill(shape, n, q, k_cache, v_cache, k_idx_cache, q_idx, q_lin, k_lin, v_lin, x,
                 w_gate, w_idx, S, z, out, idx_out, ws, stream=None):
    T = _act(shape)
    rc = library().lisa_prefill(
        ctypes.byref(shape), int(n), _ptr(q, "q", T), _ptr(k_cache, "k_cache", T),
        _ptr(v_cache, "v_cache", T), _ptr(k_idx_cache, "k_idx_cache", T), _ptr(q_idx, "q_idx", T),
        _ptr(q_lin, "q_lin", T), _ptr(k_lin, "k_lin", T), _ptr(v_lin, "v_lin", T), _ptr(x, "x", T),
        _ptr(w_gate, "w_gate", T), _ptr(w_idx, "w_idx", torch.float32),
        _ptr(S, "S", torch.float32), _ptr(z, "z", torch.float32), _ptr(out, "out", T),
        _ptr(idx_out, "idx_out", torch.int32), _ptr(ws, "ws"), 0 if ws is None else ws.numel(),
        _stream(stream))
    _check(rc, "lisa_prefill")


def lisa_indexer_topk(shape, rows_mode, n, seq_lens, q_idx, k_idx_cache, w_idx, scores_in,
                      scores_ld, scores_out, idx_out, ws, stream=None):
    T = _act(shape)
    rc = library().lisa_indexer_topk(
        ctypes.byref(shape), int(rows_mode), int(n), _ptr(seq_lens, "seq_lens", torch.int32),
        _ptr(q_idx, "q_idx", T), _ptr(k_idx_cache, "k_idx_cache", T),
        _ptr(w_idx, "w_idx", torch.float32), _ptr(scores_in, "scores_in", torch.float32),
        int(scores_ld), _ptr(scores_out, "scores_out", torch.float32),
        _ptr(idx_out, "idx_out", torch.int32), _ptr(ws, "ws"), 0 if ws is None else ws.numel(),
        _stream(stream))
    _check(rc, "lisa_indexer_topk")


def lisa_linear_state_update(shape, n_tokens, k_lin, v_lin, S, z, stream=None):
    T = _act(shape)
    rc = library().lisa_linear_state_update(
        ctypes.byref(shape), int(n_tokens), _ptr(k_lin, "k_lin", T), _ptr(v_lin, "v_lin", T),
        _ptr(S, "S", torch.float32), _ptr(z, "z", torch.float32), _stream(stream))
    _check(rc, "lisa_linear_state_update")


def lisa_segment_correct(shape, S, z, S_start, z_start, mean_S, mean_z, t, alpha, stream=None):
    """Segment state correction after segment t (all tensors fp32, updated in place)."""
    f = torch.float32
    rc = library().lisa_segment_correct(
        ctypes.byref(shape), _ptr(S, "S", f), _ptr(z, "z", f), _ptr(S_start, "S_start", f),
        _ptr(z_start, "z_start", f), _ptr(mean_S, "mean_S", f), _ptr(mean_z, "mean_z", f), int(t),
        float(alpha), _stream(stream))
    _check(rc, "lisa_segment_correct")


def lisa_dense_decode(shape, seq_lens, q, k_cache, v_cache, out, ws, stream=None):
    T = _act(shape)
    rc = library().lisa_dense_decode(
        ctypes.byref(shape), _ptr(seq_lens, "seq_lens", torch.int32), _ptr(q, "q", T),
        _ptr(k_cache, "k_cache", T), _ptr(v_cache, "v_cache", T), _ptr(out, "out", T),
        _ptr(ws, "ws"), 0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "lisa_dense_decode")


def lisa_attention_mass(shape, n_rows, row_seq, row_len, q, k_cache, idx, mass, bound, ws, stream=None):
    """Attention coverage of each row's selected set, per query head (and the
    per-head top-M bound when ``bound`` is given)."""
    T = _act(shape)
    rc = library().lisa_attention_mass(
        ctypes.byref(shape), int(n_rows), _ptr(row_seq, "row_seq", torch.int32),
        _ptr(row_len, "row_len", torch.int32), _ptr(q, "q", T), _ptr(k_cache, "k_cache", T),
        _ptr(idx, "idx", torch.int32), _ptr(mass, "mass", torch.float32), _ptr(bound, "bound", torch.float32),
        _ptr(ws, "ws"), 0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "lisa_attention_mass")


def lisa_indexer_kl(shape, n, q, k_cache, q_idx, k_idx_cache, kl_out, loss_out=None, stream=None):
    """Per-row, per-indexer-head KL of the indexer training objective (and its mean)."""
    T = _act(shape)
    rc = library().lisa_indexer_kl(
        ctypes.byref(shape), int(n), _ptr(q, "q", T), _ptr(k_cache, "k_cache", T), _ptr(q_idx, "q_idx", T),
        _ptr(k_idx_cache, "k_idx_cache", T), _ptr(kl_out, "kl_out", torch.float32),
        _ptr(loss_out, "loss_out", torch.float32), _stream(stream))
    _check(rc, "lisa_indexer_kl")


def lisa_candidate_dropout(shape, rows_mode, n, seq_lens, scores, u, scores_ld, n_cand, p, idx_out, ws,
                           stream=None):
    """Top n_cand candidates per score row, dropped where u < p, the M best survivors kept."""
    f = torch.float32
    rc = library().lisa_candidate_dropout(
        ctypes.byref(shape), int(rows_mode), int(n), _ptr(seq_lens, "seq_lens", torch.int32),
        _ptr(scores, "scores", f), _ptr(u, "u", f), int(scores_ld), int(n_cand), float(p),
        _ptr(idx_out, "idx_out", torch.int32), _ptr(ws, "ws"), 0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "lisa_candidate_dropout")


def lisa_timing_enable(kernel_id: int, starts=None, stops=None) -> None:
    """Record the next len(starts) launches of a kernel into torch.cuda.Event pairs."""
    lib = library()
    if not starts:
        _check(lib.lisa_timing_enable(0, None, None, 0), "lisa_timing_enable")
        lisa_timing_enable._keep = None
        return
    arr_t = ctypes.c_void_p * len(starts)
    a = arr_t(*[e.cuda_event for e in starts])
    b = arr_t(*[e.cuda_event for e in stops])
    lisa_timing_enable._keep = (a, b, starts, stops)
    _check(lib.lisa_timing_enable(kernel_id, a, b, len(starts)), "lisa_timing_enable")


def lisa_timing_count() -> int:
    return int(library().lisa_timing_count())
