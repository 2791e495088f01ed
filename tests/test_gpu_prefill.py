"""Prefill parity of the HIP path (lisa_prefill, lisa_indexer_topk,
lisa_linear_state_update) against the fp64 oracle on seeded inputs."""
import numpy as np
import pytest
import torch

import long_context_attention_lightning_amd as L
import oracle
from lisa_inputs import TINY_FP32_PREFILL, QWEN7B_PREFILL_16K, prefill_inputs, decode_inputs, row_sample
from gpu_helpers import (RECALL_MIN, assert_out_close, assert_state_close, check_idx_format,
                         dev, gpu_decode, gpu_prefill, host, recall, saturate_gate, shape_of, tdtype)

pytestmark = pytest.mark.gpu


def _full_parity(cfg, inp, M, label):
    g = gpu_prefill(cfg, inp, M=M)
    ref = oracle.prefill(inp, M)
    B, n = inp["q"].shape[:2]
    for b in range(B):
        check_idx_format(g["idx"][b], np.arange(1, n + 1), M)
        rc = recall(g["idx"][b], ref["idx"][b])
        print(f"[{label}] b={b} recall={rc:.6f}", flush=True)
        assert rc >= RECALL_MIN
    assert_out_close(cfg, g["out"], ref["out"], label)
    assert_state_close(g["S"], g["z"], ref["S"], ref["z"], label)
    for sign, key in ((1.0, "o_sparse"), (-1.0, "o_linear")):
        sat = saturate_gate(inp, sign)
        gs = gpu_prefill(cfg, sat, M=M, want_idx=False)
        assert_out_close(cfg, gs["out"], ref[key], f"{label} {key}")
    return g, ref


def test_prefill_tiny_fp32():
    cfg = TINY_FP32_PREFILL
    _full_parity(cfg, prefill_inputs(cfg), cfg.M, "tiny fp32")


def test_prefill_tiny_fp32_selection_bit_exact_on_oracle_scores():
    cfg = TINY_FP32_PREFILL
    inp = prefill_inputs(cfg)
    n = cfg.n
    res = oracle.prefill_rows(inp, cfg.M, range(n))
    ld = n
    sc = np.zeros((1, n, ld), np.float32)
    for t in range(n):
        sc[0, t, : t + 1] = res["scores"][t]
    sh = shape_of(cfg)
    idx = torch.full((1, n, cfg.M), -7, dtype=torch.int32, device="cuda")
    L.lisa_indexer_topk(sh, L.LISA_ROWS_PREFILL, n, None, None, None, None, dev(sc, torch.float32), ld,
                        None, idx, None)
    torch.cuda.synchronize()
    got = host(idx)[0]
    for t in range(n):
        exp = oracle.select_topm(sc[0, t, : t + 1].astype(np.float64), cfg.M)
        assert got[t, : len(exp)].tolist() == exp.tolist() and np.all(got[t, len(exp):] == -1), t


@pytest.mark.parametrize("n,M,B", [(700, 128, 2), (129, 128, 1), (64, 256, 1), (333, 1, 1), (1, 32, 1), (2, 1, 2)])
def test_prefill_small_bf16(n, M, B):
    cfg = QWEN7B_PREFILL_16K.replace(B=B, n=n, cap=n + 5)
    _full_parity(cfg, prefill_inputs(cfg, n=n, salt=n), M, f"bf16 n={n} M={M}")


PREFILL_SHAPES = [
    # (label, overrides, n, M): head dim 64 and a shared index key; GQA groups of 3 and 8
    ("bf16 G3 d64 shared key", dict(H_q=6, H_kv=2, H_L=6, d=64, H_I=2, H_Ik=1, d_I=32, hidden=96), 300, 40),
    ("bf16 G8 d128", dict(H_q=16, H_kv=2, H_L=16, H_I=2, H_Ik=2, d_I=64, hidden=160), 257, 100),
]


@pytest.mark.parametrize("label,over,n,M", PREFILL_SHAPES, ids=[s[0] for s in PREFILL_SHAPES])
def test_prefill_bf16_shapes(label, over, n, M):
    cfg = QWEN7B_PREFILL_16K.replace(n=n, cap=n + 1, **over)
    inp = prefill_inputs(cfg, n=n, salt=31)
    # start from a state carried over from an earlier part of the sequence
    r = np.random.default_rng(17)
    inp["S0"] = (r.standard_normal(inp["S0"].shape) * 30).astype(np.float32)
    inp["z0"] = (np.abs(r.standard_normal(inp["z0"].shape)) * 100 + 1).astype(np.float32)
    _full_parity(cfg, inp, M, label)


def test_prefill_bf16_offset_fallback():
    """Rows whose selected keys all score far below the first key tile: a
    softmax offset taken from the first tile leaves every selected
    probability below 2^-126, so the attention must recompute with the exact
    maximum over the selected keys, and still match."""
    cfg = QWEN7B_PREFILL_16K.replace(n=300, cap=300)
    n, M = 300, 64
    inp = prefill_inputs(cfg, n=n, salt=41)
    from lisa_inputs import round_bf16
    u = np.ones(cfg.d) / np.sqrt(cfg.d)
    q = inp["q"].astype(np.float64) + 10.0 * u          # every query shares a direction
    k = inp["k"].astype(np.float64)
    k[:, :64] = 150.0 * u                                # the first tile scores about 1500: from an offset
    kidx = inp["k_idx"].copy()
    # there, every selected probability underflows to zero (l = 0), so only
    # the exact-maximum recomputation gives finite outputs
    kidx[:, :64] = 0.0                                   # the first tile is never selected past row M
    inp["q"], inp["k"], inp["k_idx"] = round_bf16(q.astype(np.float32)), round_bf16(k.astype(np.float32)), kidx
    ref = oracle.prefill(inp, M)
    assert all(np.all(np.asarray(ref["idx"][0][t]) >= 64) for t in range(128, n))  # construction holds
    _full_parity(cfg, inp, M, "offset fallback")


@pytest.mark.parametrize("heads", [dict(), dict(H_q=4, H_kv=4, H_L=4)], ids=["gqa7", "mha"])
def test_prefill_clustered_selection(heads):
    """Selections clustered in a few key tiles: a sink tile [0, 64) and a band
    [640, 704) score positive for every query, every other key scores 0, and
    the select breaks the ties at 0 toward the larger position, so each row
    takes the two clusters plus its most recent keys.  Most key tiles are
    then selected by no row of a block; the attention skips them and must
    still match the oracle on every sampled row.  Rows [1696, 1760) also
    score a third cluster [1280, 1344) above the other two, which no row
    within 32 rows of that band selects.  With one query head per KV head
    (mha) an attention block spans four query tiles of 32 rows, and for the
    block of rows [1664, 1792) only its two middle tiles select that
    cluster's key tile, which it must still walk."""
    n, M = 2048, 256
    cfg = QWEN7B_PREFILL_16K.replace(n=n, cap=n, M=M, **heads)
    inp = prefill_inputs(cfg, n=n, salt=58)
    from lisa_inputs import round_bf16
    q_idx = np.zeros_like(inp["q_idx"])
    q_idx[..., 0] = 1.0
    k_idx = np.zeros_like(inp["k_idx"])
    for lo, hi in ((0, 64), (640, 704)):
        j = np.arange(lo, hi)
        k_idx[:, lo:hi, :, 0] = (1.0 + (j % 64) / 64.0)[None, :, None]  # distinct in bf16
    band, third = (1696, 1760), (1280, 1344)
    q_idx[:, band[0]:band[1], :, 1] = 1.0
    k_idx[:, third[0]:third[1], :, 1] = 2.0  # scores 4.0 for the band's rows, above the others' < 4
    inp["q_idx"], inp["k_idx"] = q_idx, round_bf16(k_idx)
    inp["w_idx"] = np.full_like(inp["w_idx"], 0.5)
    rows = [0, 63, 64, 255, 256, 300, 639, 640, 703, 704, 705, 831, 832, 1000, 1337, 1500,
            1663, 1664, 1695, 1696, 1700, 1727, 1759, 1760, 1791, 2000, 2047]
    ref = oracle.prefill_rows(inp, M, rows)
    clusters = set(range(64)) | set(range(640, 704))
    for t in (1000, 1695, 2047):  # construction holds: both clusters, then the most recent keys
        want = clusters | set(range(t - (M - len(clusters)) + 1, t + 1))
        assert set(int(v) for v in ref["idx"][t]) == want, t
    for t in (1700, 1759):  # the band: the third cluster too
        c3 = clusters | set(range(*third))
        want = c3 | set(range(t - (M - len(c3)) + 1, t + 1))
        assert set(int(v) for v in ref["idx"][t]) == want, t
    g = gpu_prefill(cfg, inp, M=M)
    for t in rows:
        assert [int(v) for v in g["idx"][0][t] if v >= 0] == [int(v) for v in ref["idx"][t]], t
    got = np.stack([g["out"][0, t] for t in rows])
    exp = np.stack([ref["out"][t] for t in rows])
    assert_out_close(cfg, got, exp, "clustered selection")
    sat = saturate_gate(inp, 1.0)  # the sparse branch alone
    gs = gpu_prefill(cfg, sat, M=M, want_idx=False)
    ref_s = oracle.prefill_rows(sat, M, rows)
    assert_out_close(cfg, np.stack([gs["out"][0, t] for t in rows]), np.stack([ref_s["out"][t] for t in rows]),
                     "clustered selection, sparse branch")


def test_prefill_fp32_shared_key_small_heads():
    cfg = TINY_FP32_PREFILL.replace(H_q=6, H_kv=2, H_L=6, H_I=2, H_Ik=1, n=300, cap=300, d=64, d_I=16)
    _full_parity(cfg, prefill_inputs(cfg, n=300, salt=5), 40, "fp32 shared key")


SCORE_SHAPES = [
    # (label, indexer heads, n): the streaming score kernel (query rows in
    # registers, key tiles walked) for the first three; head shapes without a
    # streaming instantiation take the per-head tile kernel
    ("4 heads d64", dict(), 600),
    ("4 heads d64, n=1500", dict(), 1500),
    ("2 heads on 1 shared key d32", dict(H_I=2, H_Ik=1, d_I=32), 600),
    ("4 heads on 2 keys d64", dict(H_I=4, H_Ik=2), 600),
    ("8 heads d32", dict(H_I=8, H_Ik=8, d_I=32), 600),
]


@pytest.mark.parametrize("label,over,n", SCORE_SHAPES, ids=[s[0] for s in SCORE_SHAPES])
def test_prefill_scores_out_and_topk_match_oracle(label, over, n):
    cfg = QWEN7B_PREFILL_16K.replace(n=n, cap=n, **over)
    M = 100
    inp = prefill_inputs(cfg, n=n, salt=2)
    sh = shape_of(cfg, M=M, cap=n)
    T = tdtype(cfg)
    kic = dev(inp["k_idx"], T)
    sc = torch.zeros((1, n, n), dtype=torch.float32, device="cuda")
    idx = torch.full((1, n, M), -7, dtype=torch.int32, device="cuda")
    L.lisa_indexer_topk(sh, L.LISA_ROWS_PREFILL, n, None, dev(inp["q_idx"], T), kic,
                        dev(inp["w_idx"], torch.float32), None, n, sc, idx, None)
    torch.cuda.synchronize()
    sc_h, idx_h = host(sc)[0], host(idx)[0]
    res = oracle.prefill_rows(inp, M, range(n))
    worst = 0.0
    for t in range(n):
        ref = res["scores"][t]
        worst = max(worst, float(np.max(np.abs(sc_h[t, : t + 1] - ref) / (1.0 + np.abs(ref)))))
        # the GPU selection of the GPU's own fp32 scores is exact
        exp = oracle.select_topm(sc_h[t, : t + 1].astype(np.float64), M)
        assert idx_h[t, : len(exp)].tolist() == exp.tolist(), t
    print(f"[scores_out {label}] worst rel err {worst:.3e}")
    assert worst < 1e-5
    assert recall(idx_h, res["idx"].values()) >= RECALL_MIN


def test_linear_state_update_matches_oracle():
    cfg = QWEN7B_PREFILL_16K.replace(B=2)
    n = 333
    inp = prefill_inputs(cfg, n=n, salt=9)
    r = np.random.default_rng(4)
    S0 = (r.standard_normal(inp["S0"].shape) * 30).astype(np.float32)
    z0 = (np.abs(r.standard_normal(inp["z0"].shape)) * 100 + 1).astype(np.float32)
    T = tdtype(cfg)
    S, z = dev(S0, torch.float32), dev(z0, torch.float32)
    sh = shape_of(cfg, B=2)
    L.lisa_linear_state_update(sh, n, dev(inp["k_lin"], T), dev(inp["v_lin"], T), S, z)
    torch.cuda.synchronize()
    for b in range(2):
        rS, rz = oracle.linear_state_update(inp["k_lin"][b], inp["v_lin"][b], S0[b], z0[b])
        assert_state_close(host(S)[b], host(z)[b], rS, rz, f"update b={b}")


def test_prefill_then_decode_continues_the_sequence():
    cfg = QWEN7B_PREFILL_16K.replace(n=401, cap=410)
    n, M = 400, 64
    full = prefill_inputs(cfg, n=n + 1, salt=7)
    part = {k: (v[:, :n] if v.ndim >= 3 and v.shape[1] == n + 1 else v) for k, v in full.items()}
    g = gpu_prefill(cfg, part, M=M)
    ref_full = oracle.prefill(full, M)
    T = tdtype(cfg)

    def cache(a):
        c = np.zeros((1, cfg.cap) + a.shape[2:], np.float32)
        c[:, :n] = a[:, :n]
        return c

    dec = {
        "seq_lens": np.array([n + 1], np.int32),
        "k_cache": cache(full["k"]), "v_cache": cache(full["v"]), "k_idx_cache": cache(full["k_idx"]),
        "q": full["q"][:, n], "k_new": full["k"][:, n], "v_new": full["v"][:, n],
        "q_idx": full["q_idx"][:, n], "k_idx_new": full["k_idx"][:, n],
        "q_lin": full["q_lin"][:, n], "k_lin": full["k_lin"][:, n], "v_lin": full["v_lin"][:, n],
        "x": full["x"][:, n], "w_gate": full["w_gate"], "w_idx": full["w_idx"],
        "S0": g["S"], "z0": g["z"],
    }
    d = gpu_decode(cfg.replace(B=1), dec, M=M)
    assert_out_close(cfg, d["out"][0], ref_full["out"][0, n], "prefill+decode")
    assert_state_close(d["S"], d["z"], ref_full["S"], ref_full["z"], "prefill+decode")
    assert recall(d["idx"], [ref_full["idx"][0][n]]) >= RECALL_MIN


@pytest.mark.slow
def test_prefill_qwen7b_16k_sampled_rows():
    cfg = QWEN7B_PREFILL_16K
    inp = prefill_inputs(cfg)
    g = gpu_prefill(cfg, inp)
    rows = row_sample(cfg.n, cfg.M, stride=256)
    ref = oracle.prefill_rows(inp, cfg.M, rows)
    got = np.stack([g["out"][0, t] for t in rows])
    exp = np.stack([ref["out"][t] for t in rows])
    assert_out_close(cfg, got, exp, f"qwen7b prefill 16K, {len(rows)} rows")
    check_idx_format(g["idx"][0][rows], np.array(rows) + 1, cfg.M)
    rc = recall(g["idx"][0][rows], [ref["idx"][t] for t in rows])
    print(f"[qwen7b prefill 16K] recall={rc:.6f}")
    assert rc >= RECALL_MIN
    assert_state_close(g["S"][0], g["z"][0], ref["S"], ref["z"], "qwen7b prefill 16K state")


def test_prefill_graph_replays_match_eager():
    """The prefill runs its gate and linear branch on a side stream next to
    the indexer and select.  Captured in a graph (the fork and the join become
    graph edges), every replay must reproduce the eager result bit for bit,
    with eager work (state resets) between the replays."""
    n = 700
    cfg = QWEN7B_PREFILL_16K.replace(n=n, cap=n)
    inp = prefill_inputs(cfg, n=n, salt=77)
    T = tdtype(cfg)
    sh = shape_of(cfg, cap=n)
    t = {k: dev(inp[k], T) for k in ("q", "k", "v", "k_idx", "q_idx", "q_lin", "k_lin", "v_lin", "x", "w_gate")}
    w_idx = dev(inp["w_idx"], torch.float32)
    S0, z0 = dev(inp["S0"], torch.float32), dev(inp["z0"], torch.float32)
    ws = L.workspace(sh, L.LISA_OP_PREFILL, n)

    def run(S, z, out):
        L.lisa_prefill(sh, n, t["q"], t["k"], t["v"], t["k_idx"], t["q_idx"], t["q_lin"], t["k_lin"], t["v_lin"],
                       t["x"], t["w_gate"], w_idx, S, z, out, None, ws)

    s = torch.cuda.Stream()
    S_e, z_e = S0.clone(), z0.clone()
    out_e = torch.empty((1, n, cfg.H_q, cfg.d), dtype=T, device="cuda")
    with torch.cuda.stream(s):  # eager, on the stream the graph is captured on
        run(S_e, z_e, out_e)
    torch.cuda.synchronize()
    S_g, z_g = S0.clone(), z0.clone()
    out_g = torch.empty_like(out_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(S_g, z_g, out_g)
    for rep in range(3):
        S_g.copy_(S0)
        z_g.copy_(z0)
        out_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), rep
        assert torch.equal(S_g, S_e) and torch.equal(z_g, z_e), rep
    ref = oracle.prefill_rows(inp, cfg.M, [0, 350, n - 1])
    assert_out_close(cfg, host(out_e)[0, [0, 350, n - 1]], np.stack([ref["out"][t_] for t_ in (0, 350, n - 1)]),
                     "eager prefill")
