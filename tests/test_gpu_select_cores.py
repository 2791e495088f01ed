"""Bit-exact top-M selection by each of the library's two select cores,
fed the oracle's fp32 score rows ("LISA", arXiv 2607.19358v1, Section 3.2
Stage 2: per query the M positions ranked highest by the head-summed indexer
score; ties to the later position, -0.0 equal to +0.0, ascending output, -1
padding).

The decode step selects with the core its shape routes to: the core inside
the fused select + attention launch ('runs': thread-contiguous runs, keys
held in LDS) for few sequences with rows of up to 32K, and the
separate select launch ('general') otherwise.  lisa_indexer_topk in decode-row mode
routes the same way, so feeding it oracle scores under a shape tests the
very core the decode step of that shape runs."""
import numpy as np
import pytest
import torch

import long_context_attention_lightning_amd as L
import oracle
from lisa_inputs import QWEN7B_DECODE_16K, QWEN7B_RAGGED_DECODE, QWEN14B_DECODE_32K, decode_inputs
from gpu_helpers import (decode_select_core, dev, gpu_decode, gpu_select_rows, host, padded, shape_of,
                         tdtype)

pytestmark = pytest.mark.gpu

# heads and head dim that route a few rows to each core
CORE_SHAPE = {"runs": dict(H_q=1, H_kv=1, d=128), "general": dict(H_q=64, H_kv=64, d=32)}


def _edge_rows(Lr, seed):
    r = np.random.default_rng(seed)
    return [
        r.standard_normal(Lr).astype(np.float32),
        (np.round(r.standard_normal(Lr) * 2) / 2).astype(np.float32),            # heavy ties
        np.zeros(Lr, np.float32),                                                 # one value: most recent win
        np.where(r.random(Lr) < 0.5, np.float32(-0.0), np.float32(0.0)),        # signed zeros
        np.abs(r.standard_normal(Lr)).astype(np.float32) * (r.random(Lr) < 0.1),  # ReLU-like, mostly 0
        -np.abs(r.standard_normal(Lr)).astype(np.float32),                        # all negative
        (np.maximum(r.standard_normal((4, Lr)) * 8, 0).sum(0)).astype(np.float32),  # four ReLU heads
    ]


def _check_core(rows, M, core, label):
    kw = CORE_SHAPE[core]
    B = len(rows)
    if core == "general":
        rows = rows + rows[: max(0, 9 - B)]  # enough blocks to leave the fused paths
        B = len(rows)
    Lmax = max(len(r) for r in rows)
    routed = decode_select_core(B, kw["H_kv"], kw["d"], M, Lmax)
    if routed != core:
        pytest.skip(f"{label}: this shape runs the {routed} core")
    got = gpu_select_rows(rows, M, **kw)
    exp = np.stack([padded(oracle.select_topm(r.astype(np.float64), M), M) for r in rows])
    bad = np.nonzero(np.any(got != exp, axis=1))[0]
    print(f"[{label}] core={core} rows={len(rows)} M={M} mismatched_rows={len(bad)}", flush=True)
    assert len(bad) == 0, (label, bad[:5])


@pytest.mark.parametrize("core", ["runs", "general"])
@pytest.mark.parametrize("Lr,M", [(1, 1), (2, 1), (5, 3), (1023, 64), (1024, 1024), (1025, 1024), (3000, 1),
                                  (4096, 100), (4097, 4096), (9000, 2048), (16383, 2048), (16384, 2048),
                                  (16384, 8192), (16384, 16383), (16385, 2048), (32768, 512)])
def test_select_core_edge_rows(core, Lr, M):
    _check_core(_edge_rows(Lr, Lr * 13 + M), M, core, f"edge L={Lr}")


def test_runs_core_ragged_rows_one_launch():
    r = np.random.default_rng(5)
    lens = [2049, 3000, 4096, 7777, 12000, 16384]
    rows = [(np.maximum(r.standard_normal((4, n)) * 8, 0).sum(0)).astype(np.float32) for n in lens]
    rows[2][100:3000] = 7.25  # a long run of ties straddling the threshold
    _check_core(rows, 2048, "runs", "ragged")


@pytest.mark.parametrize("cfg", [QWEN7B_DECODE_16K, QWEN7B_RAGGED_DECODE, QWEN14B_DECODE_32K],
                         ids=lambda c: c.name)
def test_decode_shape_core_on_oracle_scores(cfg):
    """The decode workload's own shape (batch, heads, head dim, longest row),
    so the rows go through the core its decode step runs."""
    inp = decode_inputs(cfg)
    seq = inp["seq_lens"]
    for M in (cfg.M_sweep or (cfg.M,)):
        ref = oracle.decode_step(inp, M)
        rows = [s.astype(np.float32) for s in ref["scores"]]
        core = decode_select_core(len(seq), cfg.H_kv, cfg.d, M, int(seq.max()))
        got = gpu_select_rows(rows, M, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d)
        exp = np.stack([padded(oracle.select_topm(r.astype(np.float64), M), M) for r in rows])
        bad = np.nonzero(np.any(got != exp, axis=1))[0]
        print(f"[{cfg.name} M={M}] core={core} rows={len(rows)} mismatched_rows={len(bad)}", flush=True)
        assert len(bad) == 0, (cfg.name, M, bad[:5])


def test_decode_scores_and_step_index_list_qwen7b_16k():
    """Decode-mode scoring (lisa_indexer_topk writing scores_out) against the
    oracle's index scores, and the decode step's own index list (assembled by
    its attention blocks split by split) against the oracle's selection on
    those same fp32 scores."""
    cfg = QWEN7B_DECODE_16K
    inp = decode_inputs(cfg)
    d = gpu_decode(cfg, inp)  # appends the new token; returns the caches after the step
    seq = inp["seq_lens"]
    Lb = int(seq[0])
    T = tdtype(cfg)
    sh = shape_of(cfg, max_len=Lb, cap=d["k_idx_cache"].shape[1], B=1)
    ld = (Lb + 63) // 64 * 64
    scores = torch.zeros((1, ld), dtype=torch.float32, device="cuda")
    idx = torch.full((1, cfg.M), -7, dtype=torch.int32, device="cuda")
    ws = L.workspace(sh, L.LISA_OP_TOPK_DECODE)
    L.lisa_indexer_topk(sh, L.LISA_ROWS_DECODE, 0, torch.from_numpy(seq.astype(np.int32)).cuda(),
                        dev(inp["q_idx"], T), d["k_idx_cache"], dev(inp["w_idx"], torch.float32), None, ld,
                        scores, idx, ws)
    torch.cuda.synchronize()
    s_gpu = host(scores)[0, :Lb]
    kic = host(d["k_idx_cache"])[0, :Lb].astype(np.float64)
    s_ref = oracle.index_scores(inp["q_idx"][0].astype(np.float64), kic, inp["w_idx"])
    rel = np.max(np.abs(s_gpu - s_ref)) / np.max(np.abs(s_ref))
    print(f"[decode scores] max rel err {rel:.3e}", flush=True)
    assert rel <= 1e-5
    exp = padded(oracle.select_topm(s_gpu.astype(np.float64), cfg.M), cfg.M)
    assert np.array_equal(host(idx)[0], exp)
    assert np.array_equal(d["idx"][0], exp), "decode step index list"
