"""Indexer training objective ("LISA", arXiv 2607.19358v1, Section 3.2 Stage 2,
Eq. 2) of the HIP path against the fp64 oracle, through the C ABI: the KL of
each row's indexer softmax from the mean of its teacher heads' causal
attention rows, and the loss (their mean).

Tolerance: every row is a sum of up to n fp32 terms T ln T, T S and the
index log-sum-exp (the scores S reach about 30 for N(0,1) index vectors at
d_I = 64), each with a relative rounding error of a few 2^-24, so the result
carries an absolute error of about 1e-5 of the row's magnitude; 1e-4 (1 + |KL|)
bounds it with a margin.
"""
import numpy as np
import pytest
import torch

import long_context_attention_lightning_amd as L
import oracle
from lisa_inputs import TINY_FP32_PREFILL, QWEN7B_PREFILL_16K, prefill_inputs
from gpu_helpers import dev, host, shape_of, tdtype

pytestmark = pytest.mark.gpu
KL_REL = 1e-4


def _gpu_kl(cfg, inp, n):
    T = tdtype(cfg)
    B = inp["q"].shape[0]
    sh = shape_of(cfg, cap=n, B=B)
    kl = torch.full((B, n, cfg.H_I), -1.0, dtype=torch.float32, device="cuda")
    loss = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    L.lisa_indexer_kl(sh, n, dev(inp["q"], T), dev(inp["k"], T), dev(inp["q_idx"], T), dev(inp["k_idx"], T), kl, loss)
    torch.cuda.synchronize()
    return host(kl), float(host(loss)[0])


def _check(cfg, inp, n, rows, label):
    kl, loss = _gpu_kl(cfg, inp, n)
    worst = 0.0
    for b in range(inp["q"].shape[0]):
        ref = oracle.indexer_kl(inp["q"][b], inp["k"][b], inp["q_idx"][b], inp["k_idx"][b], rows)
        err = np.abs(kl[b, rows] - ref) / (1.0 + np.abs(ref))
        worst = max(worst, float(err.max()))
    mean = float(np.mean(kl.astype(np.float64)))
    print(f"[{label}] rows={len(rows)} worst rel err {worst:.2e} loss={loss:.6f} mean KL={mean:.6f}", flush=True)
    assert worst <= KL_REL, label
    assert loss == pytest.approx(mean, rel=1e-5, abs=1e-6)
    return kl


def test_kl_mfma_grouped_teacher_qwen7b_heads():
    """28 query heads as 4 teacher groups of 7, one per indexer head (the
    matrix-core path); 300 rows span five 64-row blocks with a ragged tail."""
    n = 300
    cfg = QWEN7B_PREFILL_16K.replace(n=n, cap=n)
    inp = prefill_inputs(cfg, n=n, salt=33)
    kl = _check(cfg, inp, n, list(range(n)), "mfma G_T=7")
    assert abs(kl[0, 0, 0]) < 1e-4  # one key: T = Q


def test_kl_mfma_two_teacher_heads_batch2():
    n = 200
    cfg = QWEN7B_PREFILL_16K.replace(B=2, n=n, cap=n, H_q=8, H_kv=2, H_L=8, H_I=4, H_Ik=4)
    inp = prefill_inputs(cfg, n=n, salt=34)
    _check(cfg, inp, n, list(range(n)), "mfma G_T=2 B=2")


@pytest.mark.parametrize("gt,H_q,H_kv,n", [(1, 4, 2, 150), (4, 16, 4, 131), (8, 32, 4, 140)])
def test_kl_mfma_teacher_group_sizes(gt, H_q, H_kv, n):
    """Matrix-core path for other teacher-group sizes (4 indexer heads)."""
    cfg = QWEN7B_PREFILL_16K.replace(n=n, cap=n, H_q=H_q, H_kv=H_kv, H_L=H_q, H_I=4, H_Ik=4)
    assert H_q // 4 == gt
    inp = prefill_inputs(cfg, n=n, salt=36 + gt)
    _check(cfg, inp, n, list(range(n)), f"mfma G_T={gt}")


def test_kl_mfma_teacher_logits_growing_along_keys():
    """Teacher logits that grow along the keys (every query 1, key j = j/8 in
    every dimension: logit sqrt(d) j / 8, about 2 j in base 2), so a row's
    logits span several hundred in base 2 and its later keys dominate.  The
    running maximum of the first pass must rescale its sums all along the
    row; an offset fixed by a row's first keys would leave the fp32 range."""
    n = 200
    cfg = QWEN7B_PREFILL_16K.replace(n=n, cap=n)
    inp = prefill_inputs(cfg, n=n, salt=43)
    q = np.ones_like(inp["q"])
    k = np.empty_like(inp["k"])
    k[:] = (np.arange(n, dtype=np.float32) / 8.0)[None, :, None, None]  # exact in bf16 for j < 256
    inp["q"], inp["k"] = q, k
    _check(cfg, inp, n, list(range(n)), "mfma growing logits")


@pytest.mark.parametrize("label,base,over,n", [
    ("valu fp32 tiny prefill", TINY_FP32_PREFILL, {}, 256),
    ("valu bf16 d64 shared key", QWEN7B_PREFILL_16K, dict(H_q=6, H_kv=2, H_L=6, d=64, H_I=2, H_Ik=1, d_I=32, hidden=96), 150),
])
def test_kl_vector_path(label, base, over, n):
    cfg = base.replace(n=n, cap=n, **over)
    inp = prefill_inputs(cfg, n=n, salt=35)
    _check(cfg, inp, n, list(range(n)), label)


@pytest.mark.slow
def test_kl_qwen7b_prefill_16k_sampled_rows():
    cfg = QWEN7B_PREFILL_16K
    inp = prefill_inputs(cfg)
    n = cfg.n
    rows = sorted(set(range(0, n, 509)) | {1, 63, 64, 2047, 2048, n - 65, n - 64, n - 1})
    _check(cfg, inp, n, rows, "qwen7b prefill 16K")

