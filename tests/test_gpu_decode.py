"""Decode-step parity of the HIP path (lisa_decode_step, lisa_dense_decode)
against the fp64 oracle on seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
from lisa_inputs import QWEN7B_DECODE_16K, QWEN7B_RAGGED_DECODE, QWEN14B_DECODE_32K, decode_inputs
import long_context_attention_lightning_amd as L
from gpu_helpers import (RECALL_MIN, assert_out_close, assert_state_close, check_idx_format, dev,
                         gpu_decode, gpu_dense_decode, out_errors, recall, host, saturate_gate, shape_of,
                         tdtype)

pytestmark = pytest.mark.gpu


def _parity(cfg, inp, M, label, flags=0):
    g = gpu_decode(cfg, inp, M=M, flags=flags)
    ref = oracle.decode_step(inp, M, normalized=not flags)
    check_idx_format(g["idx"], inp["seq_lens"], M)
    rc = recall(g["idx"], ref["idx"])
    print(f"[{label}] recall={rc:.6f}", flush=True)
    assert rc >= RECALL_MIN
    assert_out_close(cfg, g["out"], ref["out"], label)
    assert_state_close(g["S"], g["z"], ref["S"], ref["z"], label)
    # the new token is appended to every cache
    for b, L in enumerate(inp["seq_lens"]):
        assert torch.equal(g["k_cache"][b, L - 1].float().cpu(), torch.from_numpy(inp["k_new"][b]))
        assert torch.equal(g["v_cache"][b, L - 1].float().cpu(), torch.from_numpy(inp["v_new"][b]))
        assert torch.equal(g["k_idx_cache"][b, L - 1].float().cpu(), torch.from_numpy(inp["k_idx_new"][b]))
    return g, ref


def _branches(cfg, inp, M, label):
    """Each branch alone, through an exactly saturated gate."""
    for sign, key in ((1.0, "o_sparse"), (-1.0, "o_linear")):
        sat = saturate_gate(inp, sign)
        g = gpu_decode(cfg, sat, M=M)
        ref = oracle.decode_step(sat, M)
        np.testing.assert_array_equal(ref["out"], ref[key])
        assert_out_close(cfg, g["out"], ref[key], f"{label} {key}")


def test_decode_qwen7b_16k():
    cfg = QWEN7B_DECODE_16K
    inp = decode_inputs(cfg)
    _parity(cfg, inp, cfg.M, "qwen7b 16K")
    _branches(cfg, inp, cfg.M, "qwen7b 16K")


def test_decode_qwen7b_ragged_batch32():
    cfg = QWEN7B_RAGGED_DECODE
    inp = decode_inputs(cfg)
    assert inp["seq_lens"].min() >= 4096 and inp["seq_lens"].max() <= 16384
    _parity(cfg, inp, cfg.M, "qwen7b ragged B=32")
    _branches(cfg, inp, cfg.M, "qwen7b ragged B=32")


@pytest.mark.slow
def test_decode_qwen14b_32k_m_sweep_and_dense():
    cfg = QWEN14B_DECODE_32K
    inp = decode_inputs(cfg)
    for M in cfg.M_sweep:
        g, ref = _parity(cfg, inp, M, f"qwen14b 32K M={M}")
    # M = L: the sparse branch is full causal attention; compare the dense kernel
    dense_gpu = gpu_dense_decode(cfg, inp, g["k_cache"], g["v_cache"])
    dense_ref = oracle.dense_decode(inp)
    assert_out_close(cfg, dense_gpu, dense_ref, "qwen14b 32K dense kernel")
    np.testing.assert_allclose(ref["o_sparse"], dense_ref, rtol=1e-10, atol=1e-12)


SMALL = [
    # (label, overrides, seq_lens, M)
    ("fp32 G2 d32", dict(dtype="f32", H_q=2, H_kv=1, d=32, H_I=1, H_Ik=1, d_I=16, H_L=2, hidden=64),
     [1, 2, 31, 32, 33, 300], 32),
    ("bf16 G7 d128", dict(), [1, 2, 127, 128, 129, 700, 1500], 128),
    ("bf16 G5 shared key", dict(H_q=10, H_kv=2, H_L=10, H_I=4, H_Ik=1, hidden=200), [5, 64, 65, 999], 64),
    ("bf16 G4 d64 R2", dict(H_q=8, H_kv=2, H_L=8, d=64, H_I=4, H_Ik=2, d_I=32, hidden=96),
     [3, 255, 256, 257, 1024], 256),
    ("fp32 G7 d128", dict(dtype="f32"), [1, 100, 600], 64),
    ("bf16 M=1", dict(), [1, 2, 50], 1),
    # budgets that cover every position: no scoring or selection, the index key still appended
    ("bf16 M > every length", dict(), [1, 2, 100, 700], 1000),
    ("fp32 M = longest", dict(dtype="f32", H_q=2, H_kv=1, d=32, H_I=1, H_Ik=1, d_I=16, H_L=2, hidden=64),
     [1, 33, 300], 300),
]


@pytest.mark.parametrize("label,over,lens,M", SMALL, ids=[s[0] for s in SMALL])
def test_decode_small_shapes(label, over, lens, M):
    base = QWEN7B_DECODE_16K.replace(B=len(lens), L=0, cap=max(lens) + 3, **over)
    inp = decode_inputs(base, seed_id=11, seq_lens=np.array(lens, np.int32))
    _parity(base, inp, M, label)
    _branches(base, inp, M, label)


def test_decode_signed_head_weights():
    cfg = QWEN7B_DECODE_16K.replace(B=3, L=0, cap=3000)
    inp = decode_inputs(cfg, seed_id=12, seq_lens=np.array([100, 2048, 2999], np.int32))
    inp["w_idx"] = np.array([1.0, -0.5, 0.0, 2.0], np.float32)
    _parity(cfg, inp, 256, "signed w")


def test_decode_unnormalized_linear():
    cfg = QWEN7B_DECODE_16K.replace(B=2, L=0, cap=600, hidden=64)
    inp = decode_inputs(cfg, seed_id=13, seq_lens=np.array([10, 500], np.int32))
    inp["S0"] = inp["S0"] * 0.01
    g = gpu_decode(cfg, inp, M=64, flags=1)
    ref = oracle.decode_step(inp, 64, normalized=False)
    _, _, nrm = out_errors(g["out"], ref["out"])
    print(f"[unnormalized] rel_rms={nrm:.3e}")
    assert nrm < 1e-2


def test_decode_gate_saturated_equals_dense_at_full_budget():
    cfg = QWEN7B_DECODE_16K.replace(B=3, L=0, cap=5000)
    inp = decode_inputs(cfg, seed_id=14, seq_lens=np.array([1, 777, 4999], np.int32))
    inp["x"] = np.zeros_like(inp["x"])
    inp["x"][:, 0] = 1.0
    inp["w_gate"] = np.zeros_like(inp["w_gate"])
    inp["w_gate"][0, :] = 200.0                     # g = 1 exactly: output = sparse branch
    g = gpu_decode(cfg, inp, M=5000)
    dense_gpu = gpu_dense_decode(cfg, inp, g["k_cache"], g["v_cache"])
    ref = oracle.dense_decode(inp)
    assert_out_close(cfg, g["out"], ref, "g=1 sparse")
    assert_out_close(cfg, dense_gpu, ref, "dense")


def test_decode_is_deterministic():
    cfg = QWEN7B_RAGGED_DECODE.replace(B=4, L_lo=2000, L_hi=9000, cap=9000)
    inp = decode_inputs(cfg, seed_id=15)
    a, b = gpu_decode(cfg, inp, repeat=2)
    assert torch.equal(a["out_t"], b["out_t"])
    assert np.array_equal(a["S"], b["S"]) and np.array_equal(a["idx"], b["idx"])


ROUTES = [(512, 8), (2048, 8), (2048, 40), (6000, 8)]
ROUTE_IDS = ["fused select", "wide fused select", "separate select", "every position"]


@pytest.mark.parametrize("M,B", ROUTES, ids=ROUTE_IDS)
def test_decode_graph_replays_match_eager(M, B):
    """A decode step captured in a graph: every replay must reproduce the
    eager step bit for bit (output, index list, state, caches), with eager
    work (state resets) between the replays.  Eight sequences at M = 512 take
    the fused select + attention with 64-position splits, at 2048 the same
    launch with 256-position splits on all eight waves; forty sequences at
    2048 take the separate select and gather; M = 6000 (>= every length) the
    path without scoring."""
    cfg = QWEN7B_RAGGED_DECODE.replace(B=B, L_lo=1000, L_hi=5000, cap=5000)
    inp = decode_inputs(cfg, salt=78)
    seq = inp["seq_lens"]
    T = tdtype(cfg)
    sh = shape_of(cfg, M=M, max_len=int(seq.max()), cap=cfg.cap, B=cfg.B)
    t = {k: dev(inp[k], T) for k in ("q", "k_new", "v_new", "q_idx", "k_idx_new", "q_lin", "k_lin", "v_lin",
                                     "x", "w_gate")}
    w_idx = dev(inp["w_idx"], torch.float32)
    seq_t = torch.from_numpy(seq.astype(np.int32)).cuda()
    S0, z0 = dev(inp["S0"], torch.float32), dev(inp["z0"], torch.float32)
    caches = [dev(inp[k], T) for k in ("k_cache", "v_cache", "k_idx_cache")]
    ws = L.workspace(sh, L.LISA_OP_DECODE)

    def bufs():
        return dict(S=S0.clone(), z=z0.clone(), kc=[c.clone() for c in caches],
                    out=torch.empty((cfg.B, cfg.H_q, cfg.d), dtype=T, device="cuda"),
                    idx=torch.full((cfg.B, M), -7, dtype=torch.int32, device="cuda"))

    def run(b):
        L.lisa_decode_step(sh, seq_t, t["q"], t["k_new"], t["v_new"], t["q_idx"], t["k_idx_new"], t["q_lin"],
                           t["k_lin"], t["v_lin"], t["x"], t["w_gate"], w_idx, *b["kc"], b["S"], b["z"], b["out"],
                           b["idx"], ws)

    s = torch.cuda.Stream()
    e = bufs()
    with torch.cuda.stream(s):  # eager, on the stream the graph is captured on
        run(e)
    torch.cuda.synchronize()
    gb = bufs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(gb)
    for rep in range(3):
        gb["S"].copy_(S0)
        gb["z"].copy_(z0)
        gb["out"].zero_()
        gb["idx"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gb["out"], e["out"]) and torch.equal(gb["idx"], e["idx"]), rep
        assert torch.equal(gb["S"], e["S"]) and torch.equal(gb["z"], e["z"]), rep
        for c_g, c_e in zip(gb["kc"], e["kc"]):
            assert torch.equal(c_g, c_e), rep
    ref = oracle.decode_step(inp, M)
    assert recall(host(e["idx"]), ref["idx"]) >= RECALL_MIN
    assert_out_close(cfg, host(e["out"]), ref["out"], f"eager decode M={M}")
    assert_state_close(host(e["S"]), host(e["z"]), ref["S"], ref["z"], f"eager decode M={M}")


@pytest.mark.parametrize("M,B", ROUTES, ids=ROUTE_IDS)
def test_decode_without_index_list_matches(M, B):
    """idx_out is optional: without it the step must produce the same output,
    state and caches bit for bit (the fused kernel then keeps the selection in
    LDS, the separate select writes it to the workspace, and the path without
    scoring writes none)."""
    cfg = QWEN7B_RAGGED_DECODE.replace(B=B, L_lo=1000, L_hi=5000, cap=5000)
    inp = decode_inputs(cfg, salt=79)
    seq = inp["seq_lens"]
    T = tdtype(cfg)
    sh = shape_of(cfg, M=M, max_len=int(seq.max()), cap=cfg.cap, B=cfg.B)
    t = {k: dev(inp[k], T) for k in ("q", "k_new", "v_new", "q_idx", "k_idx_new", "q_lin", "k_lin", "v_lin",
                                     "x", "w_gate")}
    w_idx = dev(inp["w_idx"], torch.float32)
    seq_t = torch.from_numpy(seq.astype(np.int32)).cuda()
    caches = [dev(inp[k], T) for k in ("k_cache", "v_cache", "k_idx_cache")]
    ws = L.workspace(sh, L.LISA_OP_DECODE)
    res = []
    for with_idx in (True, False):
        S, z = dev(inp["S0"], torch.float32), dev(inp["z0"], torch.float32)
        kc = [c.clone() for c in caches]
        out = torch.empty((cfg.B, cfg.H_q, cfg.d), dtype=T, device="cuda")
        idx = torch.full((cfg.B, M), -7, dtype=torch.int32, device="cuda") if with_idx else None
        L.lisa_decode_step(sh, seq_t, t["q"], t["k_new"], t["v_new"], t["q_idx"], t["k_idx_new"], t["q_lin"],
                           t["k_lin"], t["v_lin"], t["x"], t["w_gate"], w_idx, *kc, S, z, out, idx, ws)
        torch.cuda.synchronize()
        res.append((out, S, z, kc))
    (o1, S1, z1, k1), (o2, S2, z2, k2) = res
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(z1, z2)
    for a, b in zip(k1, k2):
        assert torch.equal(a, b)
    assert_out_close(cfg, host(o2), oracle.decode_step(inp, M)["out"], f"no index list M={M}")


@pytest.mark.parametrize("H_q", [16, 32, 64], ids=["G2", "G4", "G8"])
@pytest.mark.parametrize("B", [2, 8], ids=["narrow splits", "wide splits"])
def test_decode_fused_routes_gqa_groups(B, H_q):
    """The fused select + attention at 8 KV heads with 2, 4 and 8 query heads
    per KV head: two sequences take 64-position splits, eight take wide
    splits (256 positions on all eight waves) so that the launch stays at one
    block per CU; both against the oracle."""
    from gpu_helpers import decode_select_core, decode_step_split
    cfg = QWEN7B_RAGGED_DECODE.replace(B=B, L_lo=1500, L_hi=4000, cap=4000, H_q=H_q, H_kv=8, H_L=H_q,
                                       hidden=512)
    M = 1024
    inp = decode_inputs(cfg, seed_id=30 + H_q)
    L_max = int(inp["seq_lens"].max())
    sl, ns = decode_step_split(B, 8, cfg.d, M, L_max)
    assert decode_select_core(B, 8, cfg.d, M, L_max) == "runs"
    assert (sl > 64) == (B == 8), (sl, ns)
    _parity(cfg, inp, M, f"G={H_q // 8} B={B} split {sl}")
