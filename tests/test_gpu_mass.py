"""Attention coverage ("LISA", arXiv 2607.19358v1, Section 4, "Optimal Window
Size M and Attention Coverage", Eq. 10) of the HIP path against the fp64
oracle, through the C ABI: the share of each query head's dense softmax
weight on a selected set, and the share on the head's own M largest weights.

Tolerance: a logit is an fp32 sum of d exact products of bf16 (or fp32)
inputs, off by about d * 2^-24 of the sum of |q_i k_i| (under 1e-5 of a
logit of N(0,1) data at d = 128), which moves a weight by the same relative
amount; exp and the fp32 sums over up to 32768 weights add about 1e-6.  A
share lies in [0, 1], so 2e-5 absolute bounds the error with room to spare.
"""
import numpy as np
import pytest
import torch

import long_context_attention_lightning_amd as L
import oracle
from lisa_inputs import QWEN7B_DECODE_16K, QWEN7B_PREFILL_16K, decode_inputs, prefill_inputs
from gpu_helpers import dev, gpu_decode, gpu_prefill, host, shape_of, tdtype

pytestmark = pytest.mark.gpu
MASS_ABS = 2e-5


def _gpu_mass(cfg, q_rows, k_cache_t, idx_rows, lens, M, row_seq=None, want_bound=True):
    T = tdtype(cfg)
    n_rows = len(lens)
    sh = shape_of(cfg, M=M, max_len=int(max(lens)), cap=k_cache_t.shape[1], B=1)
    ws = L.workspace(sh, L.LISA_OP_MASS, n_rows)
    mass = torch.full((n_rows, cfg.H_q), -1.0, dtype=torch.float32, device="cuda")
    bound = torch.full((n_rows, cfg.H_q), -1.0, dtype=torch.float32, device="cuda") if want_bound else None
    rs = None if row_seq is None else torch.tensor(np.asarray(row_seq, np.int32)).cuda()
    L.lisa_attention_mass(sh, n_rows, rs, torch.tensor(np.asarray(lens, np.int32)).cuda(), dev(q_rows, T),
                          k_cache_t, torch.from_numpy(np.ascontiguousarray(idx_rows, dtype=np.int32)).cuda(),
                          mass, bound, ws)
    torch.cuda.synchronize()
    return host(mass), None if bound is None else host(bound)


def _check(got_mass, got_bound, q_rows, K_rows, idx_rows, lens, M, label):
    worst = 0.0
    for r, (q, K, P, n) in enumerate(zip(q_rows, K_rows, idx_rows, lens)):
        P = np.asarray(P)
        P = P[(P >= 0) & (P < n)]
        m, b = oracle.attention_mass(q, K[:n], P, M)
        worst = max(worst, float(np.max(np.abs(got_mass[r] - m))))
        if got_bound is not None:
            worst = max(worst, float(np.max(np.abs(got_bound[r] - b))))
            assert np.all(got_bound[r] >= got_mass[r] - MASS_ABS), (label, r)
    print(f"[{label}] rows={len(lens)} worst abs err {worst:.2e}", flush=True)
    assert worst <= MASS_ABS, label


def test_mass_after_decode_step_on_its_selection():
    """Decode rows (row_seq NULL): the coverage of the step's own index sets,
    with the caches as the step left them (the new key appended)."""
    cfg = QWEN7B_DECODE_16K.replace(B=3, L=0, L_lo=500, L_hi=3000, cap=3072)
    M = 256
    inp = decode_inputs(cfg, salt=21)
    g = gpu_decode(cfg, inp, M=M)
    lens = inp["seq_lens"]
    K_rows = []
    for b, n in enumerate(lens):
        K = np.array(inp["k_cache"][b, :n], dtype=np.float64)
        K[n - 1] = inp["k_new"][b]
        K_rows.append(K)
    mass, bound = _gpu_mass(cfg, inp["q"], g["k_cache"], g["idx"], lens, M)
    _check(mass, bound, inp["q"], K_rows, g["idx"], lens, M, "decode selection")


def test_mass_prefill_rows_share_one_sequence():
    """Sampled prefill rows of one sequence (row_seq all 0, row_len t+1) with
    the prefill's index lists, rows at and around M included."""
    n, M = 700, 100
    cfg = QWEN7B_PREFILL_16K.replace(n=n, cap=n)
    inp = prefill_inputs(cfg, n=n, salt=12)
    g = gpu_prefill(cfg, inp, M=M)
    rows = [0, 1, 2, 98, 99, 100, 101, 257, 512, 698, 699]
    T = tdtype(cfg)
    kc = dev(inp["k"], T)
    lens = [t + 1 for t in rows]
    idx = g["idx"][0, rows]
    mass, bound = _gpu_mass(cfg, inp["q"][0, rows], kc, idx, lens, M, row_seq=[0] * len(rows))
    _check(mass, bound, inp["q"][0, rows], [inp["k"][0]] * len(rows), idx, lens, M, "prefill rows")
    assert np.all(np.abs(mass[:5] - 1.0) <= MASS_ABS)  # rows 0..99 have at most M positions: all taken


@pytest.mark.parametrize("label,over,dtype", [
    ("fp32 d32 G2", dict(H_q=2, H_kv=1, d=32), "f32"),
    ("bf16 d64 G8", dict(H_q=16, H_kv=2, d=64), "bf16"),
    ("fp32 d128 G1", dict(H_q=3, H_kv=3, d=128), "f32"),
])
def test_mass_shapes_and_degenerate_sets(label, over, dtype):
    """Several rows per sequence, in any order; sets with -1 padding and with
    entries past the row (skipped), empty sets (mass 0), a one-key row and a
    budget that covers the whole row (mass = bound = 1)."""
    cfg = QWEN7B_DECODE_16K.replace(dtype=dtype, B=2, L=0, cap=1500, H_L=over["H_q"], **over)
    r = np.random.default_rng(8)
    inp = decode_inputs(cfg, seq_lens=np.array([1400, 1500]), salt=3)
    K_all = inp["k_cache"]
    M = 300
    specs = [(1, 1500), (0, 1400), (1, 1), (0, 250), (1, 777), (0, 1024)]
    row_seq = [s for s, _ in specs]
    lens = [n for _, n in specs]
    q = np.stack([inp["q"][s] for s in row_seq])
    idx = np.full((len(specs), M), -1, dtype=np.int64)
    for i, (s, n) in enumerate(specs):
        k = min(M, n) if i != 3 else 0  # row 3: empty set
        sel = r.choice(n, k, replace=False) if k else np.zeros(0, np.int64)
        idx[i, :k] = sel
        if i == 4:
            idx[i, -5:] = n + np.arange(5)  # past the row: skipped
    T = tdtype(cfg)
    mass, bound = _gpu_mass(cfg, q, dev(K_all, T), idx, lens, M, row_seq=row_seq)
    _check(mass, bound, q, [K_all[s] for s in row_seq], idx, lens, M, label)
    assert np.all(mass[3] == 0.0)
    assert np.all(np.abs(mass[2] - 1.0) <= MASS_ABS) and np.all(np.abs(bound[2] - 1.0) <= MASS_ABS)
    m_only, no_bound = _gpu_mass(cfg, q, dev(K_all, T), idx, lens, M, row_seq=row_seq, want_bound=False)
    assert no_bound is None
    np.testing.assert_array_equal(m_only, mass)  # the bound does not change the mass


@pytest.mark.slow
def test_mass_qwen7b_16k_full_context():
    """One 16384-position decode row at the 28/4-head, d = 128 shape with
    M = 2048 (a random selected set and the per-head bound)."""
    cfg = QWEN7B_DECODE_16K
    inp = decode_inputs(cfg, salt=4)
    n = int(inp["seq_lens"][0])
    r = np.random.default_rng(9)
    idx = np.sort(r.choice(n, cfg.M, replace=False))[None, :]
    T = tdtype(cfg)
    mass, bound = _gpu_mass(cfg, inp["q"], dev(inp["k_cache"], T), idx, [n], cfg.M)
    _check(mass, bound, inp["q"], [inp["k_cache"][0]], idx, [n], cfg.M, "qwen7b decode 16K")
