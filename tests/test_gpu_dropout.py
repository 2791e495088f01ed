"""Indexer candidate dropout ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 2:
the top 1.2 M candidates, a random share of them masked out, the rest fill
the sparse attention) on the GPU, bit-exact against the oracle on the same
fp32 score rows and the same fp32 uniforms."""
import math

import numpy as np
import pytest
import torch

import long_context_attention_lightning_amd as L
import oracle
from gpu_helpers import dev, host, padded

pytestmark = pytest.mark.gpu


def _shape(B, M, longest):
    return L.make_shape(B=B, H_q=1, H_kv=1, d=32, H_I=1, H_Ik=1, d_I=16, hidden=1, M=M, cap=longest,
                        max_len=longest)


def _decode_rows(rows, us, M, n_cand, p):
    lens = np.array([len(r) for r in rows], dtype=np.int32)
    ld = int(math.ceil(lens.max() / 4) * 4)
    S = np.zeros((len(rows), ld), np.float32)
    U = np.zeros((len(rows), ld), np.float32)
    for i, (r, u) in enumerate(zip(rows, us)):
        S[i, : len(r)] = r
        U[i, : len(u)] = u
    sh = _shape(len(rows), M, int(lens.max()))
    idx = torch.full((len(rows), M), -7, dtype=torch.int32, device="cuda")
    ws = L.workspace(sh, L.LISA_OP_DROPOUT_DECODE)
    L.lisa_candidate_dropout(sh, L.LISA_ROWS_DECODE, 0, torch.from_numpy(lens).cuda(), dev(S, torch.float32),
                             dev(U, torch.float32), ld, n_cand, p, idx, ws)
    torch.cuda.synchronize()
    return host(idx)


def _expect(rows, us, M, n_cand, p):
    return np.stack([padded(oracle.candidate_dropout(r.astype(np.float64), M, n_cand, np.float32(p), u), M)
                     for r, u in zip(rows, us)])


def _check_decode(rows, us, M, n_cand, p, label):
    got = _decode_rows(rows, us, M, n_cand, p)
    exp = _expect(rows, us, M, n_cand, p)
    bad = np.nonzero(np.any(got != exp, axis=1))[0]
    kept = float(np.mean(np.sum(exp >= 0, axis=1)))
    print(f"[{label}] rows={len(rows)} mismatched={len(bad)} mean kept={kept:.1f}", flush=True)
    assert len(bad) == 0, (label, bad[:5])
    return got


def _rows(seed, lens, ties=True):
    r = np.random.default_rng(seed)
    rows = [((np.round(r.standard_normal(n) * 4) / 4) if ties else r.standard_normal(n)).astype(np.float32)
            for n in lens]
    us = [r.random(n, dtype=np.float32) for n in lens]
    return rows, us


def test_dropout_decode_rows_paper_ratios():
    """n_cand = ceil(1.2 M), p = 0.2 (the paper's early-training setting)."""
    lens = [1, 5, 100, 307, 308, 309, 2047, 3000, 5000]
    rows, us = _rows(1, lens)
    rows[7][:] = 0.0  # all ties: the latest positions are the candidates
    M = 256
    _check_decode(rows, us, M, math.ceil(1.2 * M), 0.2, "decode 1.2M / 0.2")


def test_dropout_limits():
    """p = 0 keeps every candidate: the top-M select itself; p > 1 keeps none."""
    rows, us = _rows(2, [10, 999, 4096, 4097])
    M = 300
    got = _check_decode(rows, us, M, 360, 0.0, "p=0")
    for g, r in zip(got, rows):
        assert g.tolist() == padded(oracle.select_topm(r.astype(np.float64), M), M).tolist()
    got = _check_decode(rows, us, M, 360, 1.5, "p=1.5")
    assert np.all(got == -1)


def test_dropout_many_rows_truncation():
    """600 rows up to 16384 positions (the 256-thread select); with p = 0.01
    nearly every candidate survives and the M best must be cut from them."""
    r = np.random.default_rng(3)
    lens = r.integers(1, 16385, 600)
    rows, us = _rows(4, lens, ties=False)
    _check_decode(rows, us, 2048, 2458, 0.01, "600 rows p=0.01")
    _check_decode(rows, us, 2048, 2458, 0.2, "600 rows p=0.2")


def test_dropout_prefill_rows():
    n, B, M, C, p = 600, 2, 50, 60, 0.3
    r = np.random.default_rng(5)
    S = (np.round(r.standard_normal((B, n, n)) * 4) / 4).astype(np.float32)
    U = r.random((B, n, n), dtype=np.float32)
    sh = _shape(B, M, n)
    idx = torch.full((B, n, M), -7, dtype=torch.int32, device="cuda")
    ws = L.workspace(sh, L.LISA_OP_DROPOUT_PREFILL, n)
    L.lisa_candidate_dropout(sh, L.LISA_ROWS_PREFILL, n, None, dev(S, torch.float32), dev(U, torch.float32), n, C, p,
                             idx, ws)
    torch.cuda.synchronize()
    got = host(idx)
    bad = []
    for b in range(B):
        for t in range(n):
            exp = padded(oracle.candidate_dropout(S[b, t, : t + 1].astype(np.float64), M, C, np.float32(p),
                                                  U[b, t, : t + 1]), M)
            if got[b, t].tolist() != exp.tolist():
                bad.append((b, t))
    print(f"[prefill rows] rows={B * n} mismatched={len(bad)}", flush=True)
    assert not bad, bad[:5]
