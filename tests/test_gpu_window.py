"""Sliding-window mode ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 1, Eq. 1:
each query attends to its M most recent positions, no indexer) of the HIP
path against the fp64 oracle's window mode, through the C ABI."""
import numpy as np
import pytest
import torch

import long_context_attention_lightning_amd as L
import oracle
from lisa_inputs import TINY_FP32_PREFILL, QWEN7B_DECODE_16K, QWEN7B_PREFILL_16K, prefill_inputs, decode_inputs
from gpu_helpers import (assert_out_close, assert_state_close, dev, gpu_decode, gpu_prefill, host,
                         saturate_gate, shape_of, tdtype)

pytestmark = pytest.mark.gpu
W = L.LISA_SLIDING_WINDOW


def _window_rows(n, M):
    return [oracle.window_positions(t, M) for t in range(n)]


def _check_prefill(cfg, inp, M, label):
    g = gpu_prefill(cfg, inp, M=M, flags=W)
    ref = oracle.prefill(inp, M, window=True)
    B, n = inp["q"].shape[:2]
    for b in range(B):
        for t, P in enumerate(_window_rows(n, M)):
            row = g["idx"][b, t]
            assert row[: len(P)].tolist() == P.tolist() and np.all(row[len(P):] == -1), (label, b, t)
    assert_out_close(cfg, g["out"], ref["out"], label)
    assert_state_close(g["S"], g["z"], ref["S"], ref["z"], label)
    sat = saturate_gate(inp, 1.0)  # the sparse branch alone
    gs = gpu_prefill(cfg, sat, M=M, flags=W, want_idx=False)
    assert_out_close(cfg, gs["out"], ref["o_sparse"], f"{label} o_sparse")


def test_window_prefill_tiny_fp32():
    cfg = TINY_FP32_PREFILL
    _check_prefill(cfg, prefill_inputs(cfg), cfg.M, "window tiny fp32 prefill")


@pytest.mark.parametrize("n,M,B", [(700, 128, 2), (333, 64, 1), (129, 200, 1), (300, 1, 1)])
def test_window_prefill_bf16(n, M, B):
    """MFMA path: the band mask is formed from positions, and key tiles that
    lie before every row's window are skipped."""
    cfg = QWEN7B_PREFILL_16K.replace(B=B, n=n, cap=n + 3)
    _check_prefill(cfg, prefill_inputs(cfg, n=n, salt=n + 7), M, f"window bf16 n={n} M={M}")


def test_window_prefill_bf16_g7_long_band():
    cfg = QWEN7B_PREFILL_16K.replace(n=1100, cap=1100)
    _check_prefill(cfg, prefill_inputs(cfg, n=1100, salt=5), 200, "window bf16 G7 n=1100 M=200")


@pytest.mark.parametrize("small,M", [(False, 64), (False, 2048), (True, 8)],
                         ids=["bf16 qwen7b heads M=64", "bf16 qwen7b heads M=2048", "fp32 small heads M=8"])
def test_window_decode(small, M):
    if not small:
        cfg = QWEN7B_DECODE_16K.replace(B=3, L=0, L_lo=40, L_hi=3000, cap=3072)
    else:  # fp32, small heads
        cfg = QWEN7B_DECODE_16K.replace(dtype="f32", B=2, L=0, L_lo=5, L_hi=60, cap=64, H_q=2, H_kv=1, H_L=2, d=32,
                                 H_I=1, H_Ik=1, d_I=16, hidden=64)
    inp = decode_inputs(cfg, salt=M)
    T = tdtype(cfg)
    seq = inp["seq_lens"]
    cap = inp["k_cache"].shape[1]
    sh = shape_of(cfg, M=M, max_len=int(seq.max()), cap=cap, B=len(seq), flags=W)
    t = {k: dev(inp[k], T) for k in ("q", "k_new", "v_new", "q_lin", "k_lin", "v_lin", "x", "w_gate",
                                     "k_cache", "v_cache")}
    S = dev(inp["S0"], torch.float32)
    z = dev(inp["z0"], torch.float32)
    out = torch.empty((len(seq), cfg.H_q, cfg.d), dtype=T, device="cuda")
    idx = torch.full((len(seq), M), -7, dtype=torch.int32, device="cuda")
    ws = L.workspace(sh, L.LISA_OP_DECODE)
    # the indexer arguments may be NULL in window mode
    L.lisa_decode_step(sh, torch.from_numpy(seq.astype(np.int32)).cuda(), t["q"], t["k_new"], t["v_new"],
                       None, None, t["q_lin"], t["k_lin"], t["v_lin"], t["x"], t["w_gate"], None,
                       t["k_cache"], t["v_cache"], None, S, z, out, idx, ws)
    torch.cuda.synchronize()
    ref = oracle.decode_step(inp, M, window=True)
    label = f"window decode {'fp32 small heads' if small else 'bf16 qwen7b heads'} M={M}"
    for b in range(len(seq)):
        P = ref["idx"][b]
        row = host(idx)[b]
        assert row[: len(P)].tolist() == P.tolist() and np.all(row[len(P):] == -1), (label, b)
        Lb = int(seq[b])
        np.testing.assert_array_equal(host(t["k_cache"][b, Lb - 1]), host(dev(inp["k_new"][b], T)))
        np.testing.assert_array_equal(host(t["v_cache"][b, Lb - 1]), host(dev(inp["v_new"][b], T)))
    assert_out_close(cfg, host(out), ref["out"], label)
    assert_state_close(host(S), host(z), ref["S"], ref["z"], label)


def test_window_matches_indexed_path_with_tied_scores():
    """All indexer weights zero: every score ties and top-M keeps the most
    recent positions, so the indexed path selects exactly the window."""
    cfg = QWEN7B_DECODE_16K.replace(B=2, L=0, L_lo=100, L_hi=900, cap=1024)
    inp = decode_inputs(cfg, salt=3)
    inp["w_idx"] = np.zeros_like(inp["w_idx"])
    for M in (50, 512):
        a = gpu_decode(cfg, inp, M=M, flags=W)
        b = gpu_decode(cfg, inp, M=M)
        np.testing.assert_array_equal(a["idx"], b["idx"])
        np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=2e-2)


def test_window_flag_rejected_by_indexer_topk():
    cfg = QWEN7B_DECODE_16K
    sh = shape_of(cfg, max_len=cfg.L, flags=W)
    idx = torch.zeros((1, cfg.M), dtype=torch.int32, device="cuda")
    with pytest.raises(Exception):
        L.lisa_indexer_topk(sh, L.LISA_ROWS_DECODE, 0, torch.ones(1, dtype=torch.int32, device="cuda"),
                            None, None, None, torch.zeros((1, cfg.L), device="cuda"), cfg.L, None, idx, None)
