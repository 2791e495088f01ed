"""Helpers of the GPU parity tests: upload seeded inputs, call the C ABI
through the Python binding, download results, and the parity metrics."""
from __future__ import annotations

import numpy as np
import torch

import long_context_attention_lightning_amd as L
from lisa_inputs import LayerConfig

BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-5
STATE_REL = 1e-4
RECALL_MIN = 0.999


def tdtype(cfg: LayerConfig):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda").to(dtype).contiguous()


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def shape_of(cfg: LayerConfig, M=None, max_len=0, cap=None, B=None, flags=0):
    return L.make_shape(B=cfg.B if B is None else B, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d,
                        H_I=cfg.H_I, H_Ik=cfg.H_Ik, d_I=cfg.d_I, hidden=cfg.hidden,
                        M=cfg.M if M is None else M, cap=cfg.cap if cap is None else cap,
                        max_len=max_len, H_L=cfg.H_L, chunk=cfg.chunk, dtype=cfg.dtype,
                        flags=flags)


def gpu_decode(cfg: LayerConfig, inp, M=None, flags=0, repeat=1):
    """One lisa_decode_step on uploaded copies of ``inp``; returns host arrays."""
    T = tdtype(cfg)
    M = cfg.M if M is None else M
    seq = inp["seq_lens"]
    cap = inp["k_cache"].shape[1]
    sh = shape_of(cfg, M=M, max_len=int(seq.max()), cap=cap, B=len(seq), flags=flags)
    t = {k: dev(inp[k], T) for k in ("q", "k_new", "v_new", "q_idx", "k_idx_new", "q_lin",
                                     "k_lin", "v_lin", "x", "w_gate", "k_cache", "v_cache",
                                     "k_idx_cache")}
    seq_t = torch.from_numpy(seq.astype(np.int32)).cuda()
    w_idx = dev(inp["w_idx"], torch.float32)
    outs = []
    for _ in range(repeat):
        S = dev(inp["S0"], torch.float32)
        z = dev(inp["z0"], torch.float32)
        kc, vc, kic = t["k_cache"].clone(), t["v_cache"].clone(), t["k_idx_cache"].clone()
        out = torch.empty((len(seq), cfg.H_q, cfg.d), dtype=T, device="cuda")
        idx = torch.full((len(seq), M), -7, dtype=torch.int32, device="cuda")
        ws = L.workspace(sh, L.LISA_OP_DECODE)
        L.lisa_decode_step(sh, seq_t, t["q"], t["k_new"], t["v_new"], t["q_idx"], t["k_idx_new"],
                           t["q_lin"], t["k_lin"], t["v_lin"], t["x"], t["w_gate"], w_idx,
                           kc, vc, kic, S, z, out, idx, ws)
        torch.cuda.synchronize()
        outs.append({"out": host(out), "idx": host(idx), "S": host(S), "z": host(z),
                     "k_cache": kc, "v_cache": vc, "k_idx_cache": kic, "out_t": out})
    return outs[0] if repeat == 1 else outs


def gpu_dense_decode(cfg: LayerConfig, inp, k_cache_t, v_cache_t):
    """lisa_dense_decode over caches that already hold the new token."""
    T = tdtype(cfg)
    seq = inp["seq_lens"]
    sh = shape_of(cfg, max_len=int(seq.max()), cap=k_cache_t.shape[1], B=len(seq))
    out = torch.empty((len(seq), cfg.H_q, cfg.d), dtype=T, device="cuda")
    ws = L.workspace(sh, L.LISA_OP_DENSE_DECODE)
    L.lisa_dense_decode(sh, torch.from_numpy(seq.astype(np.int32)).cuda(), dev(inp["q"], T),
                        k_cache_t, v_cache_t, out, ws)
    torch.cuda.synchronize()
    return host(out)


def gpu_prefill(cfg: LayerConfig, inp, M=None, flags=0, want_idx=True, S0=None, z0=None):
    T = tdtype(cfg)
    M = cfg.M if M is None else M
    B, n = inp["q"].shape[:2]
    cap = max(n, cfg.cap if cfg.cap else n)
    sh = shape_of(cfg, M=M, cap=cap, B=B, flags=flags)

    def cache(a):
        c = torch.zeros((B, cap) + a.shape[2:], dtype=T, device="cuda")
        c[:, :n] = dev(a, T)
        return c

    kc, vc, kic = cache(inp["k"]), cache(inp["v"]), cache(inp["k_idx"])
    t = {k: dev(inp[k], T) for k in ("q", "q_idx", "q_lin", "k_lin", "v_lin", "x", "w_gate")}
    S = dev(inp["S0"] if S0 is None else S0, torch.float32)
    z = dev(inp["z0"] if z0 is None else z0, torch.float32)
    out = torch.empty((B, n, cfg.H_q, cfg.d), dtype=T, device="cuda")
    idx = torch.full((B, n, M), -7, dtype=torch.int32, device="cuda") if want_idx else None
    ws = L.workspace(sh, L.LISA_OP_PREFILL, n)
    L.lisa_prefill(sh, n, t["q"], kc, vc, kic, t["q_idx"], t["q_lin"], t["k_lin"], t["v_lin"],
                   t["x"], t["w_gate"], dev(inp["w_idx"], torch.float32), S, z, out, idx, ws)
    torch.cuda.synchronize()
    del ws
    return {"out": host(out), "idx": None if idx is None else host(idx), "S": host(S), "z": host(z)}


def decode_split(P, B, H_kv):
    """Split length and count of the decode attention over P selected entries
    (the library's rule, mirrored to name the select core a shape uses)."""
    sl = 64
    while -(-P // sl) > 32:
        sl *= 2
    if B * H_kv * -(-P // sl) > 1024 and sl < 128:
        sl = 128
    while B * H_kv * -(-P // sl) > 4096 and sl < P:
        sl *= 2
    return sl, -(-P // sl)


def decode_step_split(B, H_kv, d, M, max_len, bf16=True):
    """The decode step's attention splits (the library's rule): decode_split's,
    or where those need more than 256 fused blocks, the shortest wide split
    (128..2048 positions, bf16 and head dim 128) that fits 256."""
    P = min(M, max_len)
    sl, ns = decode_split(P, B, H_kv)
    if M >= max_len or _fused_fits(B, H_kv, d, max_len, sl, ns, bf16):
        return sl, ns
    w = 128
    while w <= 2048:
        if _fused_fits(B, H_kv, d, max_len, w, -(-P // w), bf16):
            return w, -(-P // w)
        w *= 2
    return sl, ns


def _fused_fits(B, H_kv, d, max_len, sl, ns, bf16):
    wide_ok = bf16 and d == 128 and sl <= 2048
    return max_len <= 32768 and (sl <= 64 or wide_ok) and ns <= 32 and B * H_kv * ns <= 256


def decode_select_core(B, H_kv, d, M, max_len, bf16=True):
    """Which select core the decode step of this shape runs: 'runs' (inside
    the fused select + attention launch, few sequences with rows of up to
    32K) or 'general' (the separate select launch)."""
    sl, ns = decode_step_split(B, H_kv, d, M, max_len, bf16)
    if _fused_fits(B, H_kv, d, max_len, sl, ns, bf16):
        return "runs"
    return "general"


def gpu_select_rows(rows, M, scores_ld=None, dtype="bf16", H_q=1, H_kv=1, d=32):
    """lisa_indexer_topk in decode-row mode over given fp32 score rows; the
    shape's heads and head dim pick the select core (decode_select_core)."""
    lens = np.array([len(r) for r in rows], dtype=np.int32)
    ld = int(scores_ld or max(4, int(np.ceil(lens.max() / 4) * 4)))
    buf = np.zeros((len(rows), ld), dtype=np.float32)
    for i, r in enumerate(rows):
        buf[i, :len(r)] = r
    sh = L.make_shape(B=len(rows), H_q=H_q, H_kv=H_kv, d=d, H_I=1, H_Ik=1, d_I=16, hidden=1, M=M,
                      cap=int(lens.max()), max_len=int(lens.max()), dtype=dtype)
    idx = torch.full((len(rows), M), -7, dtype=torch.int32, device="cuda")
    L.lisa_indexer_topk(sh, L.LISA_ROWS_DECODE, 0, torch.from_numpy(lens).cuda(), None, None, None,
                        dev(buf, torch.float32), ld, None, idx, None)
    torch.cuda.synchronize()
    return host(idx)


def padded(P, M):
    a = np.full((M,), -1, dtype=np.int64)
    a[:len(P)] = P
    return a


def recall(gpu_idx_rows, ref_sets):
    hit = tot = 0
    for g, r in zip(gpu_idx_rows, ref_sets):
        g = set(int(v) for v in g if v >= 0)
        r = set(int(v) for v in r)
        hit += len(g & r)
        tot += len(r)
    return hit / max(tot, 1)


def check_idx_format(idx_rows, lens, M):
    for row, n in zip(idx_rows, lens):
        m = min(M, int(n))
        assert np.all(row[m:] == -1), "padding"
        sel = row[:m]
        assert np.all(sel >= 0) and np.all(sel < n), "range"
        assert np.all(np.diff(sel) > 0), "ascending and unique"


def out_errors(gpu, ref):
    e = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    nrm = np.linalg.norm(np.asarray(gpu, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)
    return float(e.max()), float(e.mean()), float(nrm)


# Beyond the absolute bounds, the relative RMS error of the whole output must
# stay at the level of the output rounding (bf16: 2^-9 per element).  At long
# contexts both branches are small (|O_L| ~ 1e-2), so the absolute bounds
# alone would not notice a wrong branch.
BF16_REL_RMS, F32_REL_RMS = 1e-2, 1e-5


def assert_out_close(cfg, gpu, ref, label=""):
    mx, mean, nrm = out_errors(gpu, ref)
    print(f"[{label}] out max_abs={mx:.3e} mean_abs={mean:.3e} rel_rms={nrm:.3e}", flush=True)
    if cfg.dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
        assert nrm <= BF16_REL_RMS, nrm
    else:
        assert mx <= F32_MAX_ABS, mx
        assert nrm <= F32_REL_RMS, nrm


def saturate_gate(inp, sign):
    """Copy of the inputs whose gate is exactly 1 (sign=+1: output = sparse
    branch) or exactly 0 (sign=-1: output = linear branch): x = e_0 and
    W_g[0, :] = +-200 make x . W_g = +-200, whose sigmoid rounds to 1 or 0."""
    out = dict(inp)
    x = np.zeros_like(inp["x"])
    x[..., 0] = 1.0
    w = np.zeros_like(inp["w_gate"])
    w[0, :] = 200.0 * sign
    out["x"], out["w_gate"] = x, w
    return out


def state_rel(gpu_S, ref_S, axes):
    d = np.abs(np.asarray(gpu_S, np.float64) - ref_S).max(axis=axes)
    s = np.abs(ref_S).max(axis=axes)
    return float((d / s).max())


def assert_state_close(gS, gz, rS, rz, label=""):
    eS = state_rel(gS, rS, (-2, -1))
    ez = state_rel(gz, rz, (-1,))
    print(f"[{label}] state rel S={eS:.3e} z={ez:.3e}", flush=True)
    assert eS <= STATE_REL and ez <= STATE_REL, (eS, ez)
