"""Top-M selection on the GPU, bit-exact against the oracle's selection of the
same fp32 score rows ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 2; ties
to the later position, -0.0 equal to +0.0, ascending output, -1 padding)."""
import numpy as np
import pytest
import torch

import long_context_attention_lightning_amd as L
import oracle
from lisa_inputs import (TINY_FP32_PREFILL, QWEN7B_DECODE_16K, QWEN7B_RAGGED_DECODE, QWEN7B_PREFILL_16K,
                         QWEN14B_DECODE_32K, decode_inputs, prefill_inputs, row_sample)
from gpu_helpers import dev, gpu_select_rows, host, padded

pytestmark = pytest.mark.gpu


def _expect(rows, M):
    return np.stack([padded(oracle.select_topm(r.astype(np.float64), M), M) for r in rows])


def _check(rows, M, label):
    got = gpu_select_rows(rows, M)
    exp = _expect(rows, M)
    bad = np.nonzero(np.any(got != exp, axis=1))[0]
    print(f"[{label}] rows={len(rows)} M={M} mismatched_rows={len(bad)}", flush=True)
    assert len(bad) == 0, (label, bad[:5])


@pytest.mark.parametrize("L,M", [(1, 1), (2, 1), (5, 3), (1023, 64), (1024, 1024), (1025, 1024),
                                 (4096, 100), (4097, 4096), (16384, 2048), (16385, 2048),
                                 (32768, 8192), (65536, 2048), (3000, 1)])
def test_select_edge_lengths(L, M):
    r = np.random.default_rng(L * 7 + M)
    rows = [
        r.standard_normal(L).astype(np.float32),
        (np.round(r.standard_normal(L) * 2) / 2).astype(np.float32),          # heavy ties
        np.zeros(L, np.float32),                                              # sliding window
        np.where(r.random(L) < 0.5, np.float32(-0.0), np.float32(0.0)),     # signed zeros
        np.abs(r.standard_normal(L)).astype(np.float32) * (r.random(L) < 0.1),  # ReLU-like
        -np.abs(r.standard_normal(L)).astype(np.float32),                     # all negative
    ]
    _check(rows, M, f"edge L={L}")


def test_select_mixed_lengths_one_launch():
    r = np.random.default_rng(3)
    lens = [1, 7, 64, 2047, 2048, 2049, 9000, 16384, 4096, 12345]
    rows = [(np.round(r.standard_normal(n) * 4) / 4).astype(np.float32) for n in lens]
    _check(rows, 2048, "mixed")


@pytest.mark.parametrize("cfg", [QWEN7B_DECODE_16K, QWEN7B_RAGGED_DECODE, QWEN14B_DECODE_32K],
                         ids=lambda c: c.name)
def test_select_on_oracle_decode_scores(cfg):
    inp = decode_inputs(cfg)
    Ms = cfg.M_sweep or (cfg.M,)
    for M in Ms:
        ref = oracle.decode_step(inp, M)
        rows = [s.astype(np.float32) for s in ref["scores"]]
        _check(rows, M, f"{cfg.name} M={M}")


def test_select_on_oracle_prefill_scores_tiny_fp32():
    cfg = TINY_FP32_PREFILL
    inp = prefill_inputs(cfg)
    res = oracle.prefill_rows(inp, cfg.M, range(cfg.n))
    rows = [res["scores"][t].astype(np.float32) for t in range(cfg.n)]
    _check(rows, cfg.M, "tiny fp32 prefill, all rows")


@pytest.mark.slow
def test_select_on_oracle_prefill_scores_qwen7b_16k_rows():
    cfg = QWEN7B_PREFILL_16K
    inp = prefill_inputs(cfg)
    rows_t = row_sample(cfg.n, cfg.M, stride=16)
    rows = []
    for t in rows_t:
        s = oracle.index_scores(inp["q_idx"][0, t], inp["k_idx"][0, : t + 1], inp["w_idx"])
        rows.append(s.astype(np.float32))
    _check(rows, cfg.M, f"qwen7b prefill 16K, {len(rows)} rows")


def test_select_prefill_rows_all_item_bands():
    """Prefill rows from given fp32 scores, one launch: rows of up to 4096,
    8192 and 16384 positions are selected with different per-thread item
    counts, longest rows first; every band edge is checked."""
    n, M = 9000, 2048
    r = np.random.default_rng(11)
    sc = (np.round(r.standard_normal((n, n)) * 8) / 8).astype(np.float32)  # many ties
    sc[5000] = 0.0  # a whole row of ties: the most recent positions win
    sh = L.make_shape(B=1, H_q=1, H_kv=1, d=32, H_I=1, H_Ik=1, d_I=16, hidden=1, M=M, cap=n, max_len=n)
    idx = torch.full((1, n, M), -7, dtype=torch.int32, device="cuda")
    L.lisa_indexer_topk(sh, L.LISA_ROWS_PREFILL, n, None, None, None, None, dev(sc, torch.float32), n, None,
                        idx, None)
    torch.cuda.synchronize()
    got = host(idx)[0]
    rows = sorted(set(range(0, n, 61)) | {0, 1, 2046, 2047, 2048, 4094, 4095, 4096, 5000, 8190, 8191, 8192,
                                          n - 1})
    bad = [t for t in rows if not np.array_equal(got[t], padded(oracle.select_topm(sc[t, : t + 1].astype(np.float64),
                                                                                    M), M))]
    print(f"[prefill rows] checked={len(rows)} mismatched={len(bad)}", flush=True)
    assert not bad, bad[:5]


def test_select_many_decode_rows_one_launch():
    """600 decode rows (a launch of at least 512 rows takes 256-thread blocks
    with per-row item counts) of lengths spread over 1..16384."""
    r = np.random.default_rng(12)
    lens = np.concatenate([[1, 2047, 2048, 2049, 4096, 4097, 8192, 8193, 16384], r.integers(1, 16385, 591)])
    rows = [(np.round(r.standard_normal(int(n)) * 8) / 8).astype(np.float32) for n in lens]
    rows[5][:] = 0.0  # all ties
    _check(rows, 2048, "600 decode rows")
