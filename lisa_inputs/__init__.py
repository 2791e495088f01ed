"""Seeded synthetic inputs for one LISA attention layer.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It only draws random numbers and rounds them to the storage
precision; it holds none of the method's arithmetic (no scores, no selection,
no attention, no feature map, no gate).

Every tensor comes from its own stream,
``numpy.random.default_rng([20260723, seed_id, tensor_id])``, drawn in
float32 and then rounded to bfloat16 (round to nearest even) for the bf16
configurations; ``seed_id`` is the workload's ``sid`` unless a caller passes
its own.  Arrays are returned as float32 numpy arrays whose values are
exactly representable in the storage dtype, so that torch can upload them to
bf16 without a second rounding and the oracle can upcast them to float64
exactly.

Shapes follow the workloads the layer is measured on (module constants of
the same names in capitals):

* ``tiny_fp32_prefill``   one sequence of 256 tokens, 2/1 heads, head dim 32
* ``qwen7b_decode_16k``   Qwen-7B-shaped decode step at 16384 cached tokens
* ``qwen7b_ragged_decode`` batch 32, context lengths uniform in [4096, 16384]
* ``qwen7b_prefill_16k``  causal prefill of 16384 tokens
* ``qwen14b_decode_32k``  Qwen-14B-shaped decode, batch 8 at 32768 tokens,
                          top-M in {512, 2048, 8192, 32768}
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

SEED_BASE = 20260723

# Fixed enumeration of tensor streams.  Changing a number changes the data.
T_SEQ_LENS = 0
T_Q = 1
T_K = 2
T_V = 3
T_Q_IDX = 4
T_K_IDX = 5
T_Q_LIN = 6
T_K_LIN = 7
T_V_LIN = 8
T_X = 9
T_W_GATE = 10
T_W_IDX = 11
T_K_NEW = 12
T_V_NEW = 13
T_K_IDX_NEW = 14
T_S0 = 15
T_Z0 = 16


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    sid: int             # seed stream id of the workload's inputs
    mode: str            # "prefill" | "decode"
    dtype: str           # "f32" | "bf16"
    B: int
    H_q: int
    H_kv: int
    d: int
    H_I: int
    H_Ik: int
    d_I: int
    H_L: int
    hidden: int
    M: int
    n: int = 0           # prefill tokens per sequence
    L: int = 0           # decode: context length incl. the new token (uniform)
    L_lo: int = 0        # decode ragged: lower bound of the uniform draw
    L_hi: int = 0        # decode ragged: upper bound (inclusive)
    cap: int = 0         # cache capacity (rows per sequence)
    chunk: int = 64
    M_sweep: tuple = ()

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


TINY_FP32_PREFILL = LayerConfig(
    name="tiny_fp32_prefill", sid=0, mode="prefill", dtype="f32", B=1,
    H_q=2, H_kv=1, d=32, H_I=1, H_Ik=1, d_I=16, H_L=2, hidden=64,
    M=32, n=256, cap=256, chunk=64)
QWEN7B_DECODE_16K = LayerConfig(
    name="qwen7b_decode_16k", sid=1, mode="decode", dtype="bf16", B=1,
    H_q=28, H_kv=4, d=128, H_I=4, H_Ik=4, d_I=64, H_L=28,
    hidden=3584, M=2048, L=16384, cap=16384)
QWEN7B_RAGGED_DECODE = LayerConfig(
    name="qwen7b_ragged_decode", sid=2, mode="decode", dtype="bf16", B=32,
    H_q=28, H_kv=4, d=128, H_I=4, H_Ik=4, d_I=64, H_L=28,
    hidden=3584, M=2048, L_lo=4096, L_hi=16384, cap=16384)
QWEN7B_PREFILL_16K = LayerConfig(
    name="qwen7b_prefill_16k", sid=3, mode="prefill", dtype="bf16", B=1,
    H_q=28, H_kv=4, d=128, H_I=4, H_Ik=4, d_I=64, H_L=28,
    hidden=3584, M=2048, n=16384, cap=16384, chunk=64)
QWEN14B_DECODE_32K = LayerConfig(
    name="qwen14b_decode_32k", sid=4, mode="decode", dtype="bf16", B=8,
    H_q=40, H_kv=8, d=128, H_I=4, H_Ik=4, d_I=64, H_L=40,
    hidden=5120, M=2048, L=32768, cap=32768,
    M_sweep=(512, 2048, 8192, 32768))

WORKLOADS: Dict[str, LayerConfig] = {
    c.name: c for c in (TINY_FP32_PREFILL, QWEN7B_DECODE_16K, QWEN7B_RAGGED_DECODE,
                        QWEN7B_PREFILL_16K, QWEN14B_DECODE_32K)}


# ----------------------------------------------------------------------------
# rounding helpers (storage precision only)
# ----------------------------------------------------------------------------
def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    Inputs must be finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else np.ascontiguousarray(a)


def rng(seed_id: int, tensor_id: int, salt: int = 0) -> np.random.Generator:
    key = [SEED_BASE, int(seed_id), int(tensor_id)]
    if salt:
        key.append(int(salt))
    return np.random.default_rng(key)


def normal(seed_id: int, tensor_id: int, shape, dtype: str, std: float = 1.0,
           salt: int = 0) -> np.ndarray:
    g = rng(seed_id, tensor_id, salt)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_storage(a, dtype)


# ----------------------------------------------------------------------------
# input sets
# ----------------------------------------------------------------------------
def prefill_inputs(cfg: LayerConfig, n: Optional[int] = None, salt: int = 0,
                   seed_id: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All inputs of a causal prefill of ``n`` tokens per sequence.

    Activations are N(0,1); the gate weight is N(0, 1/hidden); the indexer
    head weights are 1; the initial linear state is zero.
    """
    n = cfg.n if n is None else n
    B, dt = cfg.B, cfg.dtype
    c = cfg.sid if seed_id is None else seed_id
    return {
        "q": normal(c, T_Q, (B, n, cfg.H_q, cfg.d), dt, salt=salt),
        "k": normal(c, T_K, (B, n, cfg.H_kv, cfg.d), dt, salt=salt),
        "v": normal(c, T_V, (B, n, cfg.H_kv, cfg.d), dt, salt=salt),
        "q_idx": normal(c, T_Q_IDX, (B, n, cfg.H_I, cfg.d_I), dt, salt=salt),
        "k_idx": normal(c, T_K_IDX, (B, n, cfg.H_Ik, cfg.d_I), dt, salt=salt),
        "q_lin": normal(c, T_Q_LIN, (B, n, cfg.H_L, cfg.d), dt, salt=salt),
        "k_lin": normal(c, T_K_LIN, (B, n, cfg.H_L, cfg.d), dt, salt=salt),
        "v_lin": normal(c, T_V_LIN, (B, n, cfg.H_L, cfg.d), dt, salt=salt),
        "x": normal(c, T_X, (B, n, cfg.hidden), dt, salt=salt),
        "w_gate": normal(c, T_W_GATE, (cfg.hidden, cfg.H_q), dt,
                         std=1.0 / np.sqrt(cfg.hidden), salt=salt),
        "w_idx": np.ones((cfg.H_I,), dtype=np.float32),
        "S0": np.zeros((B, cfg.H_L, cfg.d, cfg.d), dtype=np.float32),
        "z0": np.zeros((B, cfg.H_L, cfg.d), dtype=np.float32),
    }


def ragged_lengths(cfg: LayerConfig, seed_id: Optional[int] = None) -> np.ndarray:
    if cfg.L:
        return np.full((cfg.B,), cfg.L, dtype=np.int32)
    g = rng(cfg.sid if seed_id is None else seed_id, T_SEQ_LENS)
    return g.integers(cfg.L_lo, cfg.L_hi + 1, size=cfg.B, dtype=np.int64).astype(np.int32)


def decode_inputs(cfg: LayerConfig, seq_lens: Optional[np.ndarray] = None, salt: int = 0,
                  seed_id: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of one decode step.

    ``seq_lens[b]`` counts the new token: the caches hold rows
    ``0 .. seq_lens[b]-2`` and the step appends row ``seq_lens[b]-1``.
    Cache rows at and beyond ``seq_lens[b]-1`` hold unrelated random data that
    the step must neither read nor depend on (the append overwrites one row).

    The incoming linear state stands for a state accumulated over the
    sequence's ``L-1`` earlier tokens of N(0,1) data: entries of ``S0`` are
    drawn N(0, 2(L-1)), and ``z0`` is drawn around 1.16(L-1) with standard
    deviation sqrt(0.62(L-1)) and clipped below at 1.  (These are the first
    two moments of such a sum; only their order of magnitude matters.)
    """
    B, dt = cfg.B, cfg.dtype
    c = cfg.sid if seed_id is None else seed_id
    if seq_lens is None:
        seq_lens = ragged_lengths(cfg, c)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    cap = cfg.cap if cfg.cap else int(seq_lens.max())
    hist = np.maximum(seq_lens.astype(np.float64) - 1.0, 0.0)
    s_std = np.sqrt(2.0 * hist)[:, None, None, None]
    S0 = rng(c, T_S0, salt).standard_normal((B, cfg.H_L, cfg.d, cfg.d), dtype=np.float32)
    S0 = (S0 * s_std).astype(np.float32)
    zr = rng(c, T_Z0, salt).standard_normal((B, cfg.H_L, cfg.d), dtype=np.float32)
    z0 = 1.16 * hist[:, None, None] + np.sqrt(0.62 * hist)[:, None, None] * zr
    z0 = np.maximum(z0, 1.0).astype(np.float32)
    return {
        "seq_lens": seq_lens,
        "k_cache": normal(c, T_K, (B, cap, cfg.H_kv, cfg.d), dt, salt=salt),
        "v_cache": normal(c, T_V, (B, cap, cfg.H_kv, cfg.d), dt, salt=salt),
        "k_idx_cache": normal(c, T_K_IDX, (B, cap, cfg.H_Ik, cfg.d_I), dt, salt=salt),
        "q": normal(c, T_Q, (B, cfg.H_q, cfg.d), dt, salt=salt),
        "k_new": normal(c, T_K_NEW, (B, cfg.H_kv, cfg.d), dt, salt=salt),
        "v_new": normal(c, T_V_NEW, (B, cfg.H_kv, cfg.d), dt, salt=salt),
        "q_idx": normal(c, T_Q_IDX, (B, cfg.H_I, cfg.d_I), dt, salt=salt),
        "k_idx_new": normal(c, T_K_IDX_NEW, (B, cfg.H_Ik, cfg.d_I), dt, salt=salt),
        "q_lin": normal(c, T_Q_LIN, (B, cfg.H_L, cfg.d), dt, salt=salt),
        "k_lin": normal(c, T_K_LIN, (B, cfg.H_L, cfg.d), dt, salt=salt),
        "v_lin": normal(c, T_V_LIN, (B, cfg.H_L, cfg.d), dt, salt=salt),
        "x": normal(c, T_X, (B, cfg.hidden), dt, salt=salt),
        "w_gate": normal(c, T_W_GATE, (cfg.hidden, cfg.H_q), dt,
                         std=1.0 / np.sqrt(cfg.hidden), salt=salt),
        "w_idx": np.ones((cfg.H_I,), dtype=np.float32),
        "S0": S0,
        "z0": z0,
    }


def signed_head_weights(H_I: int, seed_id: int = 99) -> np.ndarray:
    """Seeded signed indexer head weights (exercise negative and -0.0 scores)."""
    w = rng(seed_id, T_W_IDX).standard_normal((H_I,), dtype=np.float32)
    return w


def row_sample(n: int, M: int, stride: int = 16) -> List[int]:
    """Rows of a prefill checked one by one at full size: every ``stride``-th
    row, the rows around the point where the prefix reaches M, and the last."""
    rows = set(range(0, n, stride))
    rows.update(range(max(0, M - 8), min(n, M + 252)))
    rows.add(n - 1)
    return sorted(rows)
