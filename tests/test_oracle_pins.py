"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each test checks the oracle against something it does not compute the same
way: values worked out by hand (tests/golden), exhaustive brute force in
scalar Python, library routines (torch's ELU and scaled-dot-product
attention in float64), closed forms and invariants of the method
("LISA", arXiv 2607.19358v1).
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from lisa_inputs import TINY_FP32_PREFILL, QWEN7B_DECODE_16K, QWEN7B_RAGGED_DECODE, prefill_inputs, decode_inputs, round_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([[float(t) for t in part.split()] for part in line.split("|")])
    return rows


# ----------------------------------------------------------------------------
# feature map and gate
# ----------------------------------------------------------------------------
def test_phi_matches_torch_elu_plus_one():
    x = np.concatenate([np.linspace(-30, 30, 2001), [0.0, -0.0, 1e-300, -1e-300]])
    ref = torch.nn.functional.elu(torch.tensor(x, dtype=torch.float64), alpha=1.0) + 1.0
    # torch forms elu(x)+1 as (exp(x)-1)+1, which loses ~1 ulp of 1.0 for x < 0
    np.testing.assert_allclose(oracle.phi(x), ref.numpy(), rtol=1e-15, atol=2.3e-16)
    neg = x[x < 0]
    np.testing.assert_allclose(oracle.phi(neg), [math.exp(a) for a in neg], rtol=4.5e-16, atol=0)
    assert oracle.phi(np.array([0.0]))[0] == 1.0
    assert np.all(oracle.phi(x) > 0)


def test_gate_special_cases():
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    w = np.array([[200.0, -200.0], [0.0, 0.0]])
    g = oracle.gate(x, w)
    assert g[0, 0] == 1.0 and g[0, 1] < 1e-80
    np.testing.assert_array_equal(oracle.gate(x, np.zeros((2, 2))), 0.5)
    # sigma(a) + sigma(-a) = 1
    a = np.linspace(-10, 10, 41)[None, :]
    np.testing.assert_allclose(oracle.gate(np.ones((1, 1)), a) + oracle.gate(np.ones((1, 1)), -a), 1.0,
                               rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------
# indexer scores
# ----------------------------------------------------------------------------
def _scores_brute(q, k, w):
    H_I, d_I = q.shape
    L, H_Ik, _ = k.shape
    out = []
    for j in range(L):
        tot = 0.0
        for h in range(H_I):
            kh = (h * H_Ik) // H_I
            dot = 0.0
            for c in range(d_I):
                dot += float(q[h, c]) * float(k[j, kh, c])
            tot += float(w[h]) * max(0.0, dot)
        out.append(tot)
    return np.array(out)


@pytest.mark.parametrize("H_I,H_Ik", [(1, 1), (4, 4), (4, 1), (4, 2)])
def test_index_scores_brute_force(H_I, H_Ik):
    r = np.random.default_rng(5)
    q = r.standard_normal((H_I, 5))
    k = r.standard_normal((23, H_Ik, 5))
    w = r.standard_normal(H_I)
    np.testing.assert_allclose(oracle.index_scores(q, k, w), _scores_brute(q, k, w),
                               rtol=1e-13, atol=1e-13)


def test_index_scores_single_head_is_relu_dot():
    r = np.random.default_rng(6)
    q = r.standard_normal((1, 16))
    k = r.standard_normal((40, 1, 16))
    s = oracle.index_scores(q, k, np.ones(1))
    np.testing.assert_allclose(s, np.maximum(k[:, 0, :] @ q[0], 0.0), rtol=1e-14)
    assert (s == 0).sum() > 5           # ReLU zeros are exact


def test_index_scores_head_permutation_invariant():
    r = np.random.default_rng(7)
    q = r.standard_normal((4, 8))
    k = r.standard_normal((30, 4, 8))
    w = np.abs(r.standard_normal(4))
    perm = [2, 0, 3, 1]
    np.testing.assert_allclose(oracle.index_scores(q, k, w),
                               oracle.index_scores(q[perm], k[:, perm], w[perm]), rtol=1e-13)


# ----------------------------------------------------------------------------
# top-M selection
# ----------------------------------------------------------------------------
def _select_brute(s, M):
    order = sorted(range(len(s)), key=lambda j: (float(s[j]), j), reverse=True)
    return sorted(order[:min(M, len(s))])


def test_select_golden_by_hand():
    rows = _read_rows("select_by_hand.txt")
    assert len(rows) >= 10
    for scores, (M,), expect in rows:
        got = oracle.select_topm(np.array(scores), int(M))
        assert got.tolist() == [int(e) for e in expect], (scores, M)


def test_select_exhaustive_tiny():
    vals = [-1.0, -0.0, 0.0, 0.5, 2.0]
    for L in range(1, 6):
        for combo in itertools.product(vals, repeat=L):
            s = np.array(combo)
            for M in range(1, L + 2):
                assert oracle.select_topm(s, M).tolist() == _select_brute(s, M)


def test_select_random_against_sort_and_invariants():
    r = np.random.default_rng(8)
    for _ in range(200):
        L = int(r.integers(1, 300))
        M = int(r.integers(1, 320))
        s = np.round(r.standard_normal(L) * 3) / 2      # many ties
        P = oracle.select_topm(s, M)
        assert P.tolist() == _select_brute(s, M)
        assert len(P) == min(M, L)
        mask = np.zeros(L, bool)
        mask[P] = True
        if mask.all():
            continue
        assert s[mask].min() >= s[~mask].max()


def test_select_all_equal_is_sliding_window():
    # Stage-1 static window ("LISA" Section 3.2 Stage 1): equal scores -> last M.
    for L, M in [(10, 3), (100, 100), (64, 1), (5, 9)]:
        assert oracle.select_topm(np.zeros(L), M).tolist() == list(range(max(0, L - M), L))


def test_select_float32_rounding_changes_ties():
    s64 = np.array([1.0, 1.0 + 1e-12, 0.5])
    assert oracle.select_topm(s64, 1).tolist() == [1]
    s32 = s64.astype(np.float32)
    assert oracle.select_topm(s32, 1).tolist() == [1]      # tie -> later position
    s64b = np.array([1.0 + 1e-12, 1.0, 0.5])
    assert oracle.select_topm(s64b, 1).tolist() == [0]
    assert oracle.select_topm(s64b.astype(np.float32), 1).tolist() == [1]


# ----------------------------------------------------------------------------
# sparse attention
# ----------------------------------------------------------------------------
def test_attention_golden_by_hand():
    (q, ka, kb, va, vb, o), = _read_rows("attention_by_hand.txt")
    K = np.array([[ka], [kb]])
    V = np.array([[va], [vb]])
    got = oracle.sparse_attention(np.array([q]), K, V, [0, 1])
    np.testing.assert_allclose(got[0], o, rtol=0, atol=1e-14)


@pytest.mark.parametrize("H_q,H_kv", [(2, 1), (28, 4), (5, 5), (6, 2)])
def test_full_selection_equals_torch_sdpa_causal(H_q, H_kv):
    """M >= t+1 selects the whole causal prefix: SA_M becomes full attention."""
    r = np.random.default_rng(9)
    n, d = 37, 16
    q = r.standard_normal((n, H_q, d))
    K = r.standard_normal((n, H_kv, d))
    V = r.standard_normal((n, H_kv, d))
    rep = H_q // H_kv
    qt = torch.tensor(q).permute(1, 0, 2)[None]
    kt = torch.tensor(K).permute(1, 0, 2).repeat_interleave(rep, dim=0)[None]
    vt = torch.tensor(V).permute(1, 0, 2).repeat_interleave(rep, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    for t in range(n):
        P = oracle.select_topm(r.standard_normal(t + 1), t + 1 + int(r.integers(0, 4)))
        got = oracle.sparse_attention(q[t], K, V, P)
        np.testing.assert_allclose(got, ref[t], rtol=1e-12, atol=1e-12)


def test_attention_single_key_and_order_invariance():
    r = np.random.default_rng(10)
    q = r.standard_normal((4, 8))
    K = r.standard_normal((20, 2, 8))
    V = r.standard_normal((20, 2, 8))
    got = oracle.sparse_attention(q, K, V, [13])
    np.testing.assert_array_equal(got[:2], np.repeat(V[13, 0][None], 2, 0))
    np.testing.assert_array_equal(got[2:], np.repeat(V[13, 1][None], 2, 0))
    P = [3, 17, 5, 0, 11]
    np.testing.assert_allclose(oracle.sparse_attention(q, K, V, P),
                               oracle.sparse_attention(q, K, V, sorted(P)), rtol=1e-14)


def test_attention_brute_force_scalar_loops():
    r = np.random.default_rng(11)
    H_q, H_kv, d = 4, 2, 3
    q = r.standard_normal((H_q, d))
    K = r.standard_normal((9, H_kv, d))
    V = r.standard_normal((9, H_kv, d))
    P = [1, 4, 8]
    got = oracle.sparse_attention(q, K, V, P)
    for h in range(H_q):
        g = h // (H_q // H_kv)
        logits = [sum(q[h, c] * K[j, g, c] for c in range(d)) / math.sqrt(d) for j in P]
        m = max(logits)
        e = [math.exp(a - m) for a in logits]
        for c in range(d):
            ref = sum(e[i] * V[j, g, c] for i, j in enumerate(P)) / sum(e)
            assert abs(got[h, c] - ref) < 1e-13


# ----------------------------------------------------------------------------
# linear branch
# ----------------------------------------------------------------------------
def test_linear_golden_by_hand():
    (k, v, q, o_n, o_u, (S_fin,), (z_fin,)), = _read_rows("linear_by_hand.txt")
    arr = lambda a: np.array(a, dtype=np.float64).reshape(-1, 1, 1)
    S0, z0 = np.zeros((1, 1, 1)), np.zeros((1, 1))
    o, S, z = oracle.linear_recurrent(arr(q), arr(k), arr(v), S0, z0, normalized=True)
    np.testing.assert_allclose(o[:, 0, 0], o_n, rtol=0, atol=1e-14)
    assert S[0, 0, 0] == S_fin and z[0, 0] == z_fin
    o, _, _ = oracle.linear_recurrent(arr(q), arr(k), arr(v), S0, z0, normalized=False)
    np.testing.assert_allclose(o[:, 0, 0], o_u, rtol=0, atol=1e-13)


def _lin_inputs(n=150, H=3, d=8, seed=12, zero_state=False):
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((n, H, d)) for _ in range(3))
    if zero_state:
        S0, z0 = np.zeros((H, d, d)), np.zeros((H, d))
    else:
        S0 = r.standard_normal((H, d, d)) * 5
        z0 = np.abs(r.standard_normal((H, d))) * 10 + 1
    return q, k, v, S0, z0


@pytest.mark.parametrize("normalized", [True, False])
@pytest.mark.parametrize("chunk", [1, 7, 64, 200])
def test_linear_recurrent_equals_chunked(normalized, chunk):
    q, k, v, S0, z0 = _lin_inputs()
    o1, S1, z1 = oracle.linear_recurrent(q, k, v, S0, z0, normalized)
    o2, S2, z2 = oracle.linear_chunked(q, k, v, S0, z0, chunk, normalized)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(z2, z1, rtol=1e-12)


def test_linear_closed_form_state_and_rows():
    q, k, v, S0, z0 = _lin_inputs()
    o1, S1, z1 = oracle.linear_recurrent(q, k, v, S0, z0)
    fk = torch.nn.functional.elu(torch.tensor(k)) + 1.0          # library phi
    S_cf = S0 + torch.einsum("nhd,nhe->hde", fk, torch.tensor(v)).numpy()
    np.testing.assert_allclose(S1, S_cf, rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(z1, z0 + fk.sum(0).numpy(), rtol=1e-13)
    rows = [0, 3, 77, 149]
    res, S2, z2 = oracle.linear_rows(q, k, v, S0, z0, rows)
    for t in rows:
        np.testing.assert_allclose(res[t], o1[t], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-11)
    S3, z3 = oracle.linear_state_update(k, v, S0, z0)
    np.testing.assert_allclose(S3, S1, rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(z3, z1, rtol=1e-13)


def test_linear_first_token_returns_its_value_and_convexity():
    q, k, v, S0, z0 = _lin_inputs(zero_state=True)
    o, _, _ = oracle.linear_recurrent(q, k, v, S0, z0)
    np.testing.assert_allclose(o[0], v[0], rtol=1e-14, atol=1e-15)
    # each output channel is a convex combination of the values so far
    for t in range(len(o)):
        lo = v[: t + 1].min(axis=0) - 1e-12
        hi = v[: t + 1].max(axis=0) + 1e-12
        assert np.all(o[t] >= lo) and np.all(o[t] <= hi)


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------
def _layer_brute(inp, M, t):
    """Scalar-loop layer output for row t of sequence 0 (tiny sizes)."""
    q, K, V = inp["q"][0], inp["k"][0], inp["v"][0]
    qi, ki, w = inp["q_idx"][0], inp["k_idx"][0], inp["w_idx"]
    H_q, d = q.shape[1:]
    H_kv = K.shape[1]
    s = _scores_brute(qi[t], ki[: t + 1], w)
    P = _select_brute(s, M)
    elu1 = lambda a: a + 1.0 if a > 0 else math.exp(a)
    out = np.zeros((H_q, d))
    for h in range(H_q):
        g = (h * H_kv) // H_q
        lg = [sum(float(q[t, h, c]) * float(K[j, g, c]) for c in range(d)) / math.sqrt(d) for j in P]
        m = max(lg)
        e = [math.exp(a - m) for a in lg]
        osp = [sum(e[i] * float(V[j, g, c]) for i, j in enumerate(P)) / sum(e) for c in range(d)]
        num = [0.0] * d
        den = 0.0
        for c in range(d):
            fq = elu1(float(inp["q_lin"][0, t, h, c]))
            zc = float(inp["z0"][0, h, c])
            for i in range(t + 1):
                zc += elu1(float(inp["k_lin"][0, i, h, c]))
            den += fq * zc
            for e2 in range(d):
                sce = float(inp["S0"][0, h, c, e2])
                for i in range(t + 1):
                    sce += elu1(float(inp["k_lin"][0, i, h, c])) * float(inp["v_lin"][0, i, h, e2])
                num[e2] += fq * sce
        a = sum(float(inp["x"][0, t, c]) * float(inp["w_gate"][c, h]) for c in range(inp["x"].shape[2]))
        gg = 1.0 / (1.0 + math.exp(-a))
        for c in range(d):
            out[h, c] = gg * osp[c] + (1.0 - gg) * num[c] / den
    return out, P


def test_prefill_against_scalar_brute_force():
    cfg = TINY_FP32_PREFILL.replace(d=4, d_I=3, hidden=5, H_q=4, H_kv=2, H_L=4, M=3, H_I=2, H_Ik=2)
    inp = prefill_inputs(cfg, n=9, salt=1)
    r = np.random.default_rng(13)
    inp["S0"] = r.standard_normal(inp["S0"].shape).astype(np.float32)
    inp["z0"] = (np.abs(r.standard_normal(inp["z0"].shape)) + 1).astype(np.float32)
    inp["w_idx"] = np.array([1.0, 0.5], dtype=np.float32)
    ref = oracle.prefill(inp, cfg.M)
    for t in range(9):
        out, P = _layer_brute(inp, cfg.M, t)
        assert ref["idx"][0][t].tolist() == P
        np.testing.assert_allclose(ref["out"][0, t], out, rtol=1e-11, atol=1e-12)
    rows = oracle.prefill_rows(inp, cfg.M, [2, 8])
    np.testing.assert_allclose(rows["out"][8], ref["out"][0, 8], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(rows["S"], ref["S"][0], rtol=1e-12)


def test_gate_saturation_selects_one_branch():
    cfg = TINY_FP32_PREFILL
    inp = prefill_inputs(cfg, n=40)
    inp["x"] = np.zeros_like(inp["x"])
    inp["x"][..., 0] = 1.0
    for sign, key in [(1.0, "o_sparse"), (-1.0, "o_linear")]:
        inp["w_gate"] = np.zeros_like(inp["w_gate"])
        inp["w_gate"][0, :] = 200.0 * sign
        ref = oracle.prefill(inp, cfg.M)
        np.testing.assert_array_equal(ref["out"], ref[key])
    inp["w_gate"] = np.zeros_like(inp["w_gate"])
    ref = oracle.prefill(inp, cfg.M)
    np.testing.assert_allclose(ref["out"], 0.5 * (ref["o_sparse"] + ref["o_linear"]), rtol=1e-15)


def test_decode_continues_prefill():
    """prefill(n) followed by one decode step equals the last row of prefill(n+1)."""
    cfg = TINY_FP32_PREFILL.replace(H_q=4, H_kv=2, H_L=4, H_I=2, H_Ik=2, M=16)
    n = 50
    full = prefill_inputs(cfg, n=n + 1, salt=3)
    part = {k: (v[:, :n] if k in ("q", "k", "v", "q_idx", "k_idx", "q_lin", "k_lin", "v_lin", "x") else v)
            for k, v in full.items()}
    ref_full = oracle.prefill(full, cfg.M)
    ref_part = oracle.prefill(part, cfg.M)
    cap = n + 4
    B = 1

    def cache(a):
        c = np.random.default_rng(1).standard_normal((B, cap) + a.shape[2:])
        c[:, :n] = a[:, :n]
        return c

    dec = {
        "seq_lens": np.array([n + 1]),
        "k_cache": cache(full["k"]), "v_cache": cache(full["v"]), "k_idx_cache": cache(full["k_idx"]),
        "q": full["q"][:, n], "k_new": full["k"][:, n], "v_new": full["v"][:, n],
        "q_idx": full["q_idx"][:, n], "k_idx_new": full["k_idx"][:, n],
        "q_lin": full["q_lin"][:, n], "k_lin": full["k_lin"][:, n], "v_lin": full["v_lin"][:, n],
        "x": full["x"][:, n], "w_gate": full["w_gate"], "w_idx": full["w_idx"],
        "S0": ref_part["S"], "z0": ref_part["z"],
    }
    d = oracle.decode_step(dec, cfg.M)
    np.testing.assert_allclose(d["out"][0], ref_full["out"][0, n], rtol=1e-11, atol=1e-13)
    assert d["idx"][0].tolist() == ref_full["idx"][0][n].tolist()
    np.testing.assert_allclose(d["S"][0], ref_full["S"][0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(d["z"][0], ref_full["z"][0], rtol=1e-13)


def test_decode_full_budget_equals_dense():
    cfg = QWEN7B_DECODE_16K.replace(B=3, L=0, L_lo=20, L_hi=90, cap=96, H_q=8, H_kv=2, H_L=8, d=16,
                             d_I=8, hidden=32)
    inp = decode_inputs(cfg)
    inp["w_gate"] = np.zeros_like(inp["w_gate"])
    inp["x"] = np.ones_like(inp["x"])
    inp["w_gate"][0, :] = 300.0                   # g = 1: output is the sparse branch
    d = oracle.decode_step(inp, M=10_000)
    dense = oracle.dense_decode(inp)
    np.testing.assert_array_equal(d["out"], d["o_sparse"])
    np.testing.assert_allclose(d["o_sparse"], dense, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------
# sliding-window mode ([LISA] §3.2 Stage 1, Eq. 1: the M most recent tokens)
# ----------------------------------------------------------------------------
def test_window_positions_brute_force():
    for M in (1, 2, 5, 64):
        for t in range(0, 70):
            want = [j for j in range(t + 1) if t - j < M]
            assert oracle.window_positions(t, M).tolist() == want


@pytest.mark.parametrize("M", [1, 7, 64, 300])
def test_window_prefill_equals_topm_with_tied_scores(M):
    """With every indexer score equal, top-M keeps the largest positions (the
    tie rule), which is the sliding window: the windowed layer must equal the
    indexed layer with all head weights zero."""
    cfg = TINY_FP32_PREFILL.replace(n=129, cap=129, M=M)
    inp = prefill_inputs(cfg)
    tied = dict(inp, w_idx=np.zeros_like(inp["w_idx"]))
    a = oracle.prefill(inp, M, window=True)
    b = oracle.prefill(tied, M)
    for t in range(cfg.n):
        assert a["idx"][0][t].tolist() == b["idx"][0][t].tolist()
    np.testing.assert_array_equal(a["out"], b["out"])


def test_window_prefill_full_window_equals_torch_sdpa_causal():
    """A window at least as long as the sequence is full causal attention."""
    cfg = TINY_FP32_PREFILL.replace(n=96, cap=96, M=96)
    inp = prefill_inputs(cfg)
    inp["w_gate"] = np.zeros_like(inp["w_gate"])
    inp["x"] = np.ones_like(inp["x"])
    inp["w_gate"][0, :] = 300.0                   # g = 1: the sparse branch alone
    a = oracle.prefill(inp, 96, window=True)
    rep = cfg.H_q // cfg.H_kv
    qt = torch.tensor(inp["q"][0], dtype=torch.float64).permute(1, 0, 2)[None]
    kt = torch.tensor(inp["k"][0], dtype=torch.float64).permute(1, 0, 2).repeat_interleave(rep, dim=0)[None]
    vt = torch.tensor(inp["v"][0], dtype=torch.float64).permute(1, 0, 2).repeat_interleave(rep, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(a["out"][0], ref, rtol=1e-12, atol=1e-12)


def test_window_decode_equals_tied_topm_and_dense_when_wide():
    cfg = QWEN7B_DECODE_16K.replace(B=3, L=0, L_lo=20, L_hi=90, cap=96, H_q=8, H_kv=2, H_L=8, d=16,
                             d_I=8, hidden=32)
    inp = decode_inputs(cfg)
    tied = dict(inp, w_idx=np.zeros_like(inp["w_idx"]))
    for M in (1, 16, 50):
        a = oracle.decode_step(inp, M, window=True)
        b = oracle.decode_step(tied, M)
        for i in range(3):
            L = int(inp["seq_lens"][i])
            assert a["idx"][i].tolist() == list(range(max(0, L - M), L))
            assert a["idx"][i].tolist() == b["idx"][i].tolist()
        np.testing.assert_array_equal(a["out"], b["out"])
    wide = oracle.decode_step(inp, 10_000, window=True)
    np.testing.assert_allclose(wide["o_sparse"], oracle.dense_decode(inp), rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------
# segment state correction ([LISA] §3.3, Eqs. 6-9)
# ----------------------------------------------------------------------------
def test_segment_correct_scalar_by_hand():
    # segment 2: start 1, end 4 (direction 3); mean of segment 1's direction 1;
    # alpha 0.5: corrected 0.5*3 + 0.5*1 = 2, state 1 + 2 = 3, new mean (1+3)/2 = 2
    S, z, mS, mz = oracle.segment_correct(np.array([4.0]), np.array([10.0]), np.array([1.0]), np.array([6.0]),
                                          np.array([1.0]), np.array([2.0]), 2, 0.5)
    assert S.tolist() == [3.0] and mS.tolist() == [2.0]
    # z: direction 4, prior mean 2 -> corrected 3, state 9, mean 3
    assert z.tolist() == [9.0] and mz.tolist() == [3.0]


def test_segment_correct_first_segment_ignores_the_mean_buffer():
    r = np.random.default_rng(21)
    S, S0 = r.standard_normal((2, 3, 3)), r.standard_normal((2, 3, 3))
    z, z0 = r.standard_normal((2, 3)), r.standard_normal((2, 3))
    junk = np.full((2, 3, 3), 1e30)
    Sn, zn, mS, mz = oracle.segment_correct(S, z, S0, z0, junk, junk[..., 0], 1, 0.3)
    np.testing.assert_allclose(Sn, S0 + 0.7 * (S - S0), rtol=1e-14)
    np.testing.assert_allclose(mS, S - S0, rtol=1e-14)
    np.testing.assert_allclose(mz, z - z0, rtol=1e-14)


def test_segment_correct_invariants_over_a_run():
    """alpha = 0 leaves every state as reached; a constant direction is left
    unchanged at any alpha; the mean after t segments is the mean of the raw
    directions."""
    r = np.random.default_rng(22)
    dirs = [r.standard_normal((4, 4)) for _ in range(6)]
    for alpha in (0.0, 0.35, 1.0):
        S_start = np.zeros((4, 4))
        mean = np.zeros((4, 4))
        for t, dlt in enumerate(dirs, start=1):
            S_end = S_start + dlt
            S_new, _, mean, _ = oracle.segment_correct(S_end, np.zeros(1), S_start, np.zeros(1), mean,
                                                       np.zeros(1), t, alpha)
            if alpha == 0.0:
                np.testing.assert_allclose(S_new, S_end, rtol=0, atol=1e-14)
            want = (1 - alpha) * dlt + alpha * (np.mean(dirs[: t - 1], axis=0) if t > 1 else 0.0)
            np.testing.assert_allclose(S_new - S_start, want, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(mean, np.mean(dirs[:t], axis=0), rtol=1e-12, atol=1e-12)
            S_start = S_new
    const = r.standard_normal((4, 4))
    S_new, _, _, _ = oracle.segment_correct(5 + const, np.zeros(1), np.full((4, 4), 5.0), np.zeros(1), const,
                                            np.zeros(1), 4, 0.8)
    np.testing.assert_allclose(S_new, 5 + const, rtol=1e-14)


# ----------------------------------------------------------------------------
# input generator
# ----------------------------------------------------------------------------
def test_round_bf16_matches_torch():
    r = np.random.default_rng(14)
    a = (r.standard_normal(100000) * np.exp(r.uniform(-20, 20, 100000))).astype(np.float32)
    a[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]   # ties to even
    ref = torch.tensor(a).to(torch.bfloat16).to(torch.float32).numpy()
    got = round_bf16(a)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_generator_is_seeded_and_shaped():
    cfg = QWEN7B_RAGGED_DECODE.replace(B=4, cap=64, L_lo=5, L_hi=60)
    a = decode_inputs(cfg)
    b = decode_inputs(cfg)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert a["k_cache"].shape == (4, 64, 4, 128)
    assert np.all((a["seq_lens"] >= 5) & (a["seq_lens"] <= 60))
    assert np.all(round_bf16(a["q"]) == a["q"])


# ---------------------------------------------------------------------------
# attention coverage ([LISA] §4, Eq. 10)
# ---------------------------------------------------------------------------
def test_mass_by_hand():
    """Logits 0, ln 2, ln 4 give weights in the ratio 1 : 2 : 4 (of 7)."""
    d = 4
    q = np.array([[2.0, 0.0, 0.0, 0.0]])  # q . k / sqrt(d) = k[0]
    K = np.zeros((3, 1, d))
    K[:, 0, 0] = [0.0, math.log(2.0), math.log(4.0)]
    for P, M, mass, bound in (([0, 2], 1, 5 / 7, 4 / 7), ([1], 2, 2 / 7, 6 / 7), ([2, 1, 0], 3, 1.0, 1.0),
                              ([], 1, 0.0, 4 / 7)):
        m, b = oracle.attention_mass(q, K, P, M)
        assert m[0] == pytest.approx(mass, abs=1e-15) and b[0] == pytest.approx(bound, abs=1e-15), (P, M)


def test_mass_bound_is_the_best_m_set_brute_force():
    r = np.random.default_rng(4)
    L, M = 7, 3
    q = r.standard_normal((2, 8)) * 2
    K = r.standard_normal((L, 1, 8))
    _, bound = oracle.attention_mass(q, K, [], M)
    best = np.zeros(2)
    for P in itertools.combinations(range(L), M):
        m, _ = oracle.attention_mass(q, K, list(P), M)
        assert np.all(m <= bound + 1e-15)
        best = np.maximum(best, m)
    np.testing.assert_allclose(best, bound, rtol=0, atol=1e-15)


def test_mass_uniform_weights_and_full_set():
    r = np.random.default_rng(5)
    K = r.standard_normal((50, 2, 16))
    q0 = np.zeros((4, 16))  # every logit 0: uniform weights
    m, b = oracle.attention_mass(q0, K, oracle.window_positions(49, 20), 20)
    np.testing.assert_allclose(m, 20 / 50, rtol=0, atol=1e-15)
    np.testing.assert_allclose(b, 20 / 50, rtol=0, atol=1e-15)
    q = r.standard_normal((4, 16))
    m, b = oracle.attention_mass(q, K, np.arange(50), 50)
    np.testing.assert_allclose(m, 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(b, 1.0, rtol=0, atol=1e-15)


def test_mass_splits_dense_attention():
    """Dense attention is the mass-weighted mix of attention over P and over
    the rest: out_dense = m out_P + (1 - m) out_rest, per head, with the
    attention outputs from the oracle's sparse attention and from torch's
    scaled-dot-product attention in float64."""
    r = np.random.default_rng(6)
    L, H_q, H_kv, d = 40, 6, 2, 16
    q = r.standard_normal((H_q, d))
    K = r.standard_normal((L, H_kv, d))
    V = r.standard_normal((L, H_kv, d))
    P = r.choice(L, 13, replace=False)
    rest = np.setdiff1d(np.arange(L), P)
    m, _ = oracle.attention_mass(q, K, P, 13)
    mix = m[:, None] * oracle.sparse_attention(q, K, V, P) + (1 - m[:, None]) * oracle.sparse_attention(q, K, V, rest)
    G = H_q // H_kv
    tq = torch.from_numpy(q)[:, None, :]                                   # [H_q, 1, d]
    tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [H_q, L, d]
    tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
    dense = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, 0].numpy()
    np.testing.assert_allclose(mix, dense, rtol=0, atol=1e-12)


def test_mass_reads_the_grouped_kv_head():
    """Heads 0-1 read KV head 0, whose keys point the query at position 0;
    heads 2-3 read KV head 1, pointing at position 1."""
    d = 8
    q = np.zeros((4, d))
    q[:, 0] = 10.0
    K = np.zeros((3, 2, d))
    K[0, 0, 0] = 10.0
    K[1, 1, 0] = 10.0
    m, _ = oracle.attention_mass(q, K, [0], 1)
    assert np.all(m[:2] > 0.999) and np.all(m[2:] < 1e-3), m


# ---------------------------------------------------------------------------
# indexer training objective ([LISA] §3.2 Stage 2, Eq. 2) and candidate dropout
# ---------------------------------------------------------------------------
def test_indexer_kl_by_hand():
    """Row 1 has keys 0 and 1: teacher logits 0 and ln 2 give T = (1/3, 2/3);
    equal indexer scores give Q = (1/2, 1/2).  Row 0 has one key: KL = 0."""
    d, dI = 4, 2
    q = np.zeros((2, 1, d))
    q[:, 0, 0] = 2.0                      # q . k / sqrt(d) = k[0]
    K = np.zeros((2, 1, d))
    K[:, 0, 0] = [0.0, math.log(2.0)]
    qi = np.zeros((2, 1, dI))
    qi[:, 0, 0] = 1.0
    ki = np.zeros((2, 1, dI))
    ki[:, 0, 0] = 1.0                     # S = (1, 1)
    kl = oracle.indexer_kl(q, K, qi, ki)
    want = (1 / 3) * math.log((1 / 3) / (1 / 2)) + (2 / 3) * math.log((2 / 3) / (1 / 2))
    assert kl[0, 0] == pytest.approx(0.0, abs=1e-15)
    assert kl[1, 0] == pytest.approx(want, abs=1e-15)


def test_indexer_kl_zero_when_the_indexer_matches_the_teacher():
    """One teacher head per indexer head, index query q/sqrt(d) and index key
    k with positive entries: ReLU is inactive and S equals the teacher's
    logits, so the two distributions coincide."""
    r = np.random.default_rng(14)
    n, d = 30, 8
    q = r.random((n, 2, d))
    K = r.random((n, 1, d))
    kl = oracle.indexer_kl(q, K, q / np.sqrt(d), K)
    np.testing.assert_allclose(kl, 0.0, atol=1e-14)


def test_indexer_kl_matches_torch_kl_div():
    """Grouped teacher (three heads per indexer head, two KV heads, one shared
    index key) against torch: softmax / log_softmax / kl_div in float64."""
    r = np.random.default_rng(15)
    n, H_q, H_kv, d, H_I, dI = 25, 6, 2, 16, 2, 8
    q = r.standard_normal((n, H_q, d))
    K = r.standard_normal((n, H_kv, d))
    qi = r.standard_normal((n, H_I, dI))
    ki = r.standard_normal((n, 1, dI))
    kl = oracle.indexer_kl(q, K, qi, ki)
    tq, tk, tqi, tki = (torch.from_numpy(a) for a in (q, K, qi, ki))
    for t in range(n):
        for j in range(H_I):
            heads = range(3 * j, 3 * j + 3)
            T = sum(torch.softmax(tk[: t + 1, h * H_kv // H_q] @ tq[t, h] / math.sqrt(d), 0) for h in heads) / 3
            logQ = torch.log_softmax(torch.relu(tki[: t + 1, 0] @ tqi[t, j]), 0)
            want = torch.nn.functional.kl_div(logQ, T, reduction="sum").item()
            assert kl[t, j] == pytest.approx(want, abs=1e-12), (t, j)
    assert np.all(kl >= -1e-15)


def _dropout_brute(s, M, C, p, u):
    order = sorted(range(len(s)), key=lambda j: (-s[j], -j))
    surv = [j for j in order[:C] if u[j] >= p]
    return sorted(surv[:M])


def test_candidate_dropout_brute_force():
    r = np.random.default_rng(16)
    for trial in range(300):
        L = int(r.integers(1, 12))
        M = int(r.integers(1, 6))
        C = int(r.integers(M, 9))
        s = (np.round(r.standard_normal(L) * 2) / 2).astype(np.float32)  # ties
        u = r.random(L).astype(np.float32)
        p = np.float32(r.choice([0.0, 0.2, 0.5, 1.0]))
        got = oracle.candidate_dropout(s.astype(np.float64), M, C, p, u)
        assert got.tolist() == _dropout_brute(s.tolist(), M, C, p, u.tolist()), (trial, s, u, p, M, C)


def test_candidate_dropout_special_cases():
    r = np.random.default_rng(17)
    s = r.standard_normal(500)
    u = r.random(500)
    np.testing.assert_array_equal(oracle.candidate_dropout(s, 40, 48, 0.0, u), oracle.select_topm(s, 40))
    assert oracle.candidate_dropout(s, 40, 48, 1.0, u).size == 0
    got = oracle.candidate_dropout(s, 40, 48, 0.2, u)
    cand = set(oracle.select_topm(s, 48).tolist())
    assert set(got.tolist()) <= cand and np.all(u[got] >= 0.2) and got.size == min(40, sum(u[j] >= 0.2 for j in cand))
