#!/usr/bin/env python3
"""Throughput of one LISA attention layer on one MI355X.

A step is one lisa_decode_step of the Qwen-7B-shaped layer (batch 1, 16384
cached tokens including the new one, 28/4 heads, head dim 128, indexer 4 x 64,
top-M 2048): cache append, indexer scan, top-M select, sparse GQA attention,
linear-state update and gate, all in the library's HIP kernels.  Steps are
replayed from a HIP graph that cycles over NBUF independent buffer sets
(caches, state, outputs), so consecutive steps never reuse a working set
that could still sit in the 256 MB Infinity Cache.

Printed JSON (one line): decode tokens/s of the layer as ``value``; the
dominant kernel's roofline fraction measured with HIP events recorded
around that kernel inside the timed graph; the fp64 CPU oracle timed on a
bounded sample on the host; and, under ``extra``, the per-kernel times, the
dense-attention decode baseline on the same GPU and the prefill rate.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "decode tok/s/layer @16K ctx, M=2048 (+prefill tok/s); % HBM/MFMA roofline"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=640)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--nbuf", type=int, default=32, help="rotating buffer sets (>= 512 MB total)")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-dense", action="store_true", help="skip the dense-attention decode baseline")
    p.add_argument("--no-batched", action="store_true", help="skip the batch-32 ragged decode leg")
    p.add_argument("--batched-only", action="store_true", help="only the batch-32 ragged decode leg (profiling)")
    p.add_argument("--batched-steps", type=int, default=64)
    p.add_argument("--no-sweep", action="store_true", help="skip the batch-8 32K M-sweep decode leg")
    p.add_argument("--no-window", action="store_true", help="skip the sliding-window decode and prefill legs")
    p.add_argument("--no-kl", action="store_true",
                   help="skip the legs of the adjacent operations (indexer KL, candidate dropout, segment correction)")
    p.add_argument("--prefill-only", action="store_true",
                   help="run only the prefill leg (for kernel profiling; prints the prefill numbers)")
    p.add_argument("--prefill-iters", type=int, default=20)
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--cpu-all", action="store_true", help="also time the oracle on a 16K prefill row (~30 s)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run four 256 MiB device copies (a counter-scaling reference)")
    p.add_argument("--write-traffic", nargs=3, metavar=("LEG", "FETCH_CSV", "WRITE_CSV"),
                   help="no GPU work: read two rocprofv3 --pmc counter CSVs (FETCH_SIZE, then WRITE_SIZE) of a "
                        "--copy-calibration run of one leg (decode: the default decode leg; prefill: "
                        "--prefill-only) and record each library kernel's HBM bytes per launch in "
                        "profiles/traffic.json")
    return p.parse_args()


# ----------------------------------------------------------------------------
# algorithmic traffic (bytes the method must move), per launch
# ----------------------------------------------------------------------------
def _lens(L, B):
    """Context lengths of the B sequences (L: one length, or one per sequence)."""
    return np.broadcast_to(np.asarray(L, dtype=np.int64), (B,))


def decode_bytes(cfg, L, M, B, indexer=True):
    """Per-step algorithmic bytes of the whole decode step (all sequences):
    every index key once (the indexer's scan), the min(M, L) gathered K/V
    rows, the linear state read and written, the per-token vectors and W_g.
    The index keys count at any M, also where the library skips the scan
    because M covers every position; only the sliding-window mode, which has
    no indexer, leaves them out (indexer=False)."""
    tot = 0
    for l in _lens(L, B):
        m = min(M, int(l))
        tot += (int(l) * cfg.H_Ik * cfg.d_I * 2 * indexer         # index keys
                + m * cfg.H_kv * cfg.d * 4                        # gathered K and V
                + 8 * cfg.H_L * cfg.d * (cfg.d + 1)               # S and z, read + write
                + 2 * (2 * cfg.H_q * cfg.d + 3 * cfg.H_L * cfg.d + cfg.H_I * cfg.d_I
                       + 2 * cfg.H_kv * cfg.d + cfg.H_Ik * cfg.d_I + cfg.hidden))
    return tot + 2 * cfg.hidden * cfg.H_q


def phase_a_bytes(cfg, L, B, indexer=True):
    tot = 0
    for l in _lens(L, B):
        tot += (int(l) * cfg.H_Ik * cfg.d_I * 2 * indexer + 8 * cfg.H_L * cfg.d * (cfg.d + 1)
                + 2 * (3 * cfg.H_L * cfg.d + cfg.H_I * cfg.d_I + cfg.hidden)
                + 2 * 2 * (2 * cfg.H_kv * cfg.d + cfg.H_Ik * cfg.d_I))   # new rows read + appended
    return tot + 2 * cfg.hidden * cfg.H_q


def attention_bytes(cfg, L, M, B, dense=False):
    """Gathered K and V rows (bf16) and the query of every sequence."""
    tot = 0
    for l in _lens(L, B):
        m = int(l) if dense else min(M, int(l))
        tot += m * cfg.H_kv * cfg.d * 4 + 2 * cfg.H_q * cfg.d
    return tot


def combine_bytes(cfg, B):
    """The split merge's algorithmic bytes: the bf16 output only (the split
    partials, linear numerators and gate partials it reads are the library's
    own intermediates)."""
    return B * cfg.H_q * cfg.d * 2


# Integer work a radix select must do per score: order-preserving key (2),
# bin index (3), histogram increment (1), threshold compare (1), output
# compaction (1).
SELECT_OPS_PER_KEY = 8
# Chip-wide 32-bit VALU lane operations per second: 256 CUs x 4 SIMDs x 16
# lanes per cycle x 2.4 GHz (fp32 FMA counted as 2 flops gives 157.3 TFLOP/s).
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def kernel_roofline(name, avg_ms, work, bound, traffic_key=None):
    """Roofline entry of one kernel: algorithmic work per launch over its
    average launch duration against the published (or derived) peak."""
    if bound == "hbm":
        achieved = work / (avg_ms * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    elif bound == "mfma":
        achieved = work / (avg_ms * 1e-3) / 1e12
        peak, unit = MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved = work / (avg_ms * 1e-3) / 1e12
        peak, unit = ALU_PEAK_TOPS, "TOP/s"
    return {"kernel": name, "bound": bound, "achieved": round(achieved, 4), "peak": round(peak, 1),
            "unit": unit, "frac": round(achieved / peak, 5), "traffic": load_traffic(traffic_key or name),
            "algorithmic_work_per_launch": work, "avg_launch_us": round(avg_ms * 1e3, 3)}


def bench_decode(args, torch, Lb, cfg, nbuf, steps, warmup, with_dense, traffic_prefix="", flags=0,
                 with_mass=False):
    """Graph-replayed decode steps of one workload over nbuf buffer sets:
    step time, per-kernel durations and rooflines, the dense baseline, and
    optionally the attention coverage of the steps' selections."""
    from lisa_inputs import decode_inputs
    B, Lctx, M = cfg.B, (cfg.L or cfg.L_hi), cfg.M
    T = torch.bfloat16
    print(f"# decode: {cfg.name} B={B} L={Lctx} M={M} nbuf={nbuf}", file=sys.stderr, flush=True)
    inp = decode_inputs(cfg)

    def up(a, dt=T):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt).contiguous()

    base = {k: up(inp[k]) for k in ("q", "k_new", "v_new", "q_idx", "k_idx_new", "q_lin", "k_lin",
                                    "v_lin", "x", "w_gate", "k_cache", "v_cache", "k_idx_cache")}
    base["S"] = up(inp["S0"], torch.float32)
    base["z"] = up(inp["z0"], torch.float32)
    seq = torch.from_numpy(inp["seq_lens"].astype(np.int32)).cuda()
    w_idx = up(inp["w_idx"], torch.float32)
    sh = Lb.make_shape(B=B, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d, H_I=cfg.H_I, H_Ik=cfg.H_Ik,
                       d_I=cfg.d_I, hidden=cfg.hidden, M=M, cap=cfg.cap, max_len=Lctx, flags=flags)
    sets = []
    per_set = ("q", "k_new", "v_new", "q_idx", "k_idx_new", "q_lin", "k_lin", "v_lin", "x",
               "k_cache", "v_cache", "k_idx_cache", "S", "z")
    for i in range(nbuf):
        s = {k: base[k].clone() for k in per_set}
        s["out"] = torch.empty((B, cfg.H_q, cfg.d), dtype=T, device="cuda")
        s["out_dense"] = torch.empty((B, cfg.H_q, cfg.d), dtype=T, device="cuda")
        s["idx"] = torch.empty((B, M), dtype=torch.int32, device="cuda")
        s["ws"] = Lb.workspace(sh, Lb.LISA_OP_DECODE)
        s["ws_dense"] = Lb.workspace(sh, Lb.LISA_OP_DENSE_DECODE)
        sets.append(s)
    set_bytes = sum(t.numel() * t.element_size() for t in sets[0].values())
    print(f"# {nbuf} buffer sets of {set_bytes / 2**20:.1f} MiB", file=sys.stderr, flush=True)

    def step(s):
        Lb.lisa_decode_step(sh, seq, s["q"], s["k_new"], s["v_new"], s["q_idx"], s["k_idx_new"],
                            s["q_lin"], s["k_lin"], s["v_lin"], s["x"], base["w_gate"], w_idx,
                            s["k_cache"], s["v_cache"], s["k_idx_cache"], s["S"], s["z"], s["out"],
                            s["idx"], s["ws"])

    def dense_step(s):
        Lb.lisa_dense_decode(sh, seq, s["q"], s["k_cache"], s["v_cache"], s["out_dense"], s["ws_dense"])

    cap_stream = torch.cuda.Stream()

    def capture(fn):
        """HIP graph of one pass of fn over every buffer set."""
        with torch.cuda.stream(cap_stream):       # eager warm-up pass on the capture stream
            for s in sets:
                fn(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            for s in sets:
                fn(s)
        return g

    def run(g, n_steps):
        reps = max(1, (n_steps + len(sets) - 1) // len(sets))
        for _ in range(reps):
            g.replay()
        return reps * len(sets)

    def time_graph(g):
        """Mean step time over the timed replays, and the per-replay step
        times (an event pair around every replay) for the spread."""
        run(g, warmup)
        torch.cuda.synchronize()
        # at least 100 timed steps over at least 4 replays, whatever --steps says
        reps = max(4, (max(steps, 100) + len(sets) - 1) // len(sets))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            g.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) / len(sets) for i in range(reps)]
        time_graph.spread = per
        return ev[0].elapsed_time(ev[-1]) / (reps * len(sets)), reps * len(sets)

    def kernel_times(fn, kids):
        """Average duration of each kernel from HIP events recorded by the
        library around its launches, over eager (not graph) steps."""
        res = {}
        for kid in kids:
            st = [torch.cuda.Event(enable_timing=True) for _ in sets]
            sp = [torch.cuda.Event(enable_timing=True) for _ in sets]
            for e in st + sp:
                e.record()
            torch.cuda.synchronize()
            Lb.lisa_timing_enable(kid, st, sp)
            for s in sets:
                fn(s)
            torch.cuda.synchronize()
            cnt = Lb.lisa_timing_count()
            Lb.lisa_timing_enable(0)
            res[kid] = float(np.mean([a.elapsed_time(b) for a, b in zip(st[:cnt], sp[:cnt])])) if cnt else 0.0
        return res

    # ---------------- timed region: graph replays of whole decode steps
    g_main = capture(step)
    ms_step, done = time_graph(g_main)
    spread = np.array(time_graph.spread) * 1e3
    print(f"# timed {done} steps: {ms_step * 1e3:.2f} us/step", file=sys.stderr, flush=True)
    # ---------------- per-kernel durations (HIP events on the launch stream)
    dec_kids = (0, 1, 12, 2, 8)
    kt = kernel_times(step, dec_kids)
    dec_kids = tuple(k for k in dec_kids if kt[k] > 0)  # kernels this shape launches
    per_kernel_ms = {Lb.lisa_kernel_name(k): kt[k] for k in dec_kids}
    dom = max(dec_kids, key=lambda k: kt[k])
    dom_ms = kt[dom]
    print(f"# kernels (us): " + ", ".join(f"{k}={v * 1e3:.2f}" for k, v in per_kernel_ms.items()),
          file=sys.stderr, flush=True)

    # dense baseline over the same caches
    if with_dense:
        g_dense = capture(dense_step)
        ms_dense, _ = time_graph(g_dense)
        kd = kernel_times(dense_step, (2, 8))
        dense_kernel_us = {Lb.lisa_kernel_name(k): round(v * 1e3, 3) for k, v in kd.items()}
        del g_dense

    if with_mass:
        mass_leg = bench_mass(torch, Lb, cfg, sh, seq, sets, capture, time_graph, kernel_times,
                              inp["seq_lens"].astype(np.int64), traffic_prefix)

    lens = inp["seq_lens"].astype(np.int64)
    # no index-key stream in window mode; with a budget covering every
    # position the library skips the scan, so phase A's own work has none,
    # while the step's algorithmic bytes still count them
    window_mode = bool(flags & Lb.LISA_SLIDING_WINDOW)
    scans = not window_mode and M < Lctx
    work = {0: (phase_a_bytes(cfg, lens, B, scans), "hbm"),
            1: (SELECT_OPS_PER_KEY * int(lens.sum()), "alu"),
            12: (attention_bytes(cfg, lens, M, B), "hbm"),
            2: (attention_bytes(cfg, lens, M, B), "hbm"),
            8: (combine_bytes(cfg, B), "hbm")}
    roofs = {Lb.lisa_kernel_name(k): kernel_roofline(Lb.lisa_kernel_name(k), kt[k], *work[k],
                                                     traffic_key=traffic_prefix + Lb.lisa_kernel_name(k))
             for k in dec_kids}
    roof = roofs[Lb.lisa_kernel_name(dom)]
    step_bytes = decode_bytes(cfg, lens, M, B, not window_mode)
    extra = {
        "us_per_step": round(ms_step * 1e3, 3),
        "us_per_step_median_p10_p90": [round(float(np.median(spread)), 3), round(float(np.percentile(spread, 10)), 3),
                                       round(float(np.percentile(spread, 90)), 3)],
        "step_spread_note": f"per graph replay of {len(sets)} steps, {len(spread)} replays",
        "kernel_us": {k: round(v * 1e3, 3) for k, v in per_kernel_ms.items()},
        "kernel_timing": "hipExtLaunchKernel start/stop events on each kernel's dispatch, eager steps "
                         "over the same buffer sets right after the timed graph replays",
        "kernel_roofline": roofs,
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_roofline_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    if with_dense:
        extra.update({"dense_decode_us_per_step": round(ms_dense * 1e3, 3),
                      "dense_decode_kernel_us": dense_kernel_us,
                      "dense_decode_tok_s": round(B / (ms_dense * 1e-3), 1),
                      "speedup_vs_dense_decode": round(ms_dense / ms_step, 3)})
    if with_mass:
        extra["attention_mass"] = mass_leg
    del g_main
    sets.clear()
    torch.cuda.empty_cache()
    extra.update(inp=inp, ms_step=ms_step, steps=done, roofline=roof)
    return extra


def bench_mass(torch, Lb, cfg, sh, seq, sets, capture, time_graph, kernel_times, lens, traffic_prefix):
    """Attention coverage (mass and the per-head top-M bound) of every
    sequence's selection after the decode steps, over the same buffer sets:
    the call's time, its kernels and the logits kernel's roofline."""
    B = cfg.B
    for s in sets:
        s["mass"] = torch.empty((B, cfg.H_q), dtype=torch.float32, device="cuda")
        s["bound"] = torch.empty((B, cfg.H_q), dtype=torch.float32, device="cuda")
        s["ws_mass"] = Lb.workspace(sh, Lb.LISA_OP_MASS, B)

    def mass_call(s):
        Lb.lisa_attention_mass(sh, B, None, seq, s["q"], s["k_cache"], s["idx"], s["mass"], s["bound"],
                               s["ws_mass"])

    g = capture(mass_call)
    ms, _ = time_graph(g)
    del g
    kids = (14, 15, 16)
    kt = kernel_times(mass_call, kids)
    torch.cuda.synchronize()
    key_bytes = int(lens.sum()) * cfg.H_kv * cfg.d * 2
    logits_work = key_bytes + B * cfg.H_q * cfg.d * 2
    op_bytes = logits_work + B * cfg.M * 4 + 2 * B * cfg.H_q * 4
    m = sets[0]["mass"].cpu().numpy()
    bnd = sets[0]["bound"].cpu().numpy()
    for s in sets:
        for k in ("mass", "bound", "ws_mass"):
            del s[k]
    return {
        "what": "coverage of each sequence's selected M positions by the dense softmax weights, per query "
                "head, and the per-head top-M bound (LISA Section 4, Eq. 10); synthetic N(0,1) data, so the "
                "values are not comparable with trained-model figures",
        "us_per_call": round(ms * 1e3, 3),
        "kernel_us": {Lb.lisa_kernel_name(k): round(v * 1e3, 3) for k, v in kt.items()},
        "call_algorithmic_bytes": op_bytes,
        "call_hbm_roofline_frac": round(op_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_roofline": {"mass_logits": kernel_roofline("mass_logits", kt[14], logits_work, "hbm",
                                                           traffic_key=traffic_prefix + "mass_logits"),
                            "mass_select": kernel_roofline("mass_select", kt[15],
                                                           SELECT_OPS_PER_KEY * int(lens.sum()) * cfg.H_q, "alu",
                                                           traffic_key=traffic_prefix + "mass_select")},
        "mean_mass": round(float(m.mean()), 5),
        "mean_bound": round(float(bnd.mean()), 5),
    }


# ----------------------------------------------------------------------------
# Library kernels by symbol: (name the bench reports them under, source files
# whose hash ties a traffic record to the code it was taken on).
_COMMON = ["lisa_common.h", "lisa_kernels.h"]
TRAFFIC_KERNELS = {
    "decode": {
        "k_decode_phase_a": ("decode_phase_a", ["k_decode.hip", "lisa_attend.h", "lisa_mfma.h"] + _COMMON),
        "k_select_attend": ("select_attention", ["k_decode_fused.hip", "lisa_select.h", "lisa_attend.h",
                                                 "lisa_mfma.h"] + _COMMON),
        "k_attn_combine": ("attention_combine", ["k_decode.hip", "lisa_attend.h", "lisa_mfma.h"] + _COMMON),
    },
    "prefill": {
        "k_gate_transpose": ("prefill_gate_transpose", ["k_prefill_mfma.hip", "lisa_mfma.h", "lisa_prefill.h"] + _COMMON),
        "k_gate_mfma": ("prefill_gate", ["k_prefill_mfma.hip", "lisa_mfma.h", "lisa_prefill.h"] + _COMMON),
        "k_lin_seg_sums": ("prefill_linear_sums", ["k_linear_mfma.hip", "lisa_mfma.h", "lisa_prefill.h"] + _COMMON),
        "k_lin_seg_prefix": ("prefill_linear_prefix", ["k_linear_mfma.hip", "lisa_mfma.h", "lisa_prefill.h"] + _COMMON),
        "k_lin_chunks": ("prefill_linear", ["k_linear_mfma.hip", "lisa_mfma.h", "lisa_prefill.h"] + _COMMON),
        "k_index_scores_stream": ("prefill_index_scores", ["k_prefill_mfma.hip", "lisa_mfma.h", "lisa_prefill.h"] + _COMMON),
        "k_select_rows256": ("topm_select", ["k_select.hip", "lisa_select.h", "lisa_prefill.h"] + _COMMON),
        "k_mask_occupancy": ("prefill_tile_occupancy", ["k_select.hip", "lisa_select.h", "lisa_prefill.h"] + _COMMON),
        "k_attn_prefill_mfma": ("prefill_attention", ["k_attn_mfma.hip", "lisa_mfma.h", "lisa_prefill.h"] + _COMMON),
        "k_kl_mfma": ("indexer_kl", ["k_indexer_kl.hip", "lisa_mfma.h"] + _COMMON),
        "k_kl_loss": ("indexer_kl_loss", ["k_indexer_kl.hip", "lisa_mfma.h"] + _COMMON),
        "k_dropout_compact": ("candidate_dropout_compact", ["k_dropout.hip"] + _COMMON),
        "k_dropout_gather": ("candidate_dropout_gather", ["k_dropout.hip"] + _COMMON),
    },
    # (a key "symbol|<N" or "symbol|>=N" would take only the dispatches of
    # fewer / at least N work-items of a kernel that serves two steps)
    "batched": {
        "k_decode_phase_a": ("decode_phase_a", ["k_decode.hip", "lisa_attend.h", "lisa_mfma.h"] + _COMMON),
        "k_select_attend": ("select_attention", ["k_decode_fused.hip", "lisa_select.h", "lisa_attend.h",
                                                 "lisa_mfma.h"] + _COMMON),
        "k_attn_combine": ("attention_combine", ["k_decode.hip", "lisa_attend.h", "lisa_mfma.h"] + _COMMON),
        "k_mass_logits_mfma": ("mass_logits", ["k_mass.hip", "lisa_mfma.h"] + _COMMON),
        "k_select_rows256": ("mass_select", ["k_select.hip", "lisa_select.h", "lisa_prefill.h"] + _COMMON),
        "k_mass_reduce": ("mass_reduce", ["k_mass.hip", "lisa_mfma.h"] + _COMMON),
    },
}


TRAFFIC_WORKLOAD = {
    "decode": "decode step, Qwen-7B-shaped layer, batch 1, 16384 tokens, M = 2048",
    "prefill": "causal prefill, Qwen-7B-shaped layer, 16384 tokens, M = 2048",
    "batched": "decode step, Qwen-7B-shaped layer, batch 32, context lengths 4096..16384 (seeded), M = 2048",
}


def write_traffic(leg, fetch_csv, write_csv):
    """HBM bytes per launch of each library kernel of one leg from two
    rocprofv3 counter runs.  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are
    scaled by what they read for the calibration copies (an elementwise
    kernel that reads and writes 256 MiB), then averaged over the kernel's
    dispatches; the record carries the hash of the kernel's sources."""
    import csv
    import re

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"], int(r["Grid_Size"]))
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return vals

    def selected(sel, kernel, grid):
        sym, _, cond = sel.partition("|")
        if not re.search(r"lisa::%s\b" % sym, kernel):
            return False
        if cond.startswith(">="):
            return grid >= int(cond[2:])
        if cond.startswith("<"):
            return grid < int(cond[1:])
        return True

    want = 256 << 20
    out = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        vals = per_kernel(path, counter)
        # the calibration copies: torch.mul(src, 1.0, out=dst) on 64 Mi floats
        copies = [v for (d, k, _), v in vals.items() if "AUnaryFunctor<float, float, float" in k and v * 1024 > want / 4]
        if not copies:
            sys.exit(f"{path}: no calibration copy found (run with --copy-calibration)")
        factor = want / (1024.0 * float(np.median(copies)))
        for sym, (name, _) in TRAFFIC_KERNELS[leg].items():
            got = [v for (d, k, gs), v in vals.items() if selected(sym, k, gs)]
            if got:
                out.setdefault(name, {})[counter] = (float(np.mean(got)), factor, len(got))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    prefix = "" if leg == "decode" else leg + ":"
    for sym, (name, sources) in TRAFFIC_KERNELS[leg].items():
        c = out.get(name, {})
        if "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            continue
        (f_kib, f_fac, _), (w_kib, w_fac, _) = c["FETCH_SIZE"], c["WRITE_SIZE"]
        fb, wb = f_kib * 1024 * f_fac, w_kib * 1024 * w_fac
        rec[prefix + name] = {"bytes_per_launch": int(round(fb + wb)), "fetch_bytes": int(round(fb)),
                              "write_bytes": int(round(wb)), "fetch_kib_raw": round(f_kib, 2),
                              "write_kib_raw": round(w_kib, 2), "sources": sources,
                              "source_sha256": source_hash(sources), "workload": TRAFFIC_WORKLOAD[leg]}
        print(f"{prefix + name}: read {fb / 1e6:.3f} MB, written {wb / 1e6:.3f} MB per launch "
              f"(scale {f_fac:.3f} / {w_fac:.3f})")
    json.dump(rec, open(path, "w"), indent=1, sort_keys=False)


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer runs on a single "
              "MI355X and the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_attention_lightning_amd as Lb
    from lisa_inputs import QWEN7B_DECODE_16K, QWEN7B_RAGGED_DECODE, QWEN14B_DECODE_32K, prefill_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    Lb.library()
    cfg = QWEN7B_DECODE_16K
    B, Lctx, M = cfg.B, cfg.L, cfg.M
    T = torch.bfloat16
    print(f"# bench: {cfg.name} B={B} L={Lctx} M={M} nbuf={args.nbuf}", file=sys.stderr, flush=True)

    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):  # elementwise kernel: reads 256 MiB, writes 256 MiB
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.prefill_only:
        print(json.dumps(bench_prefill(args, torch, Lb, prefill_inputs)), flush=True)
        return
    if args.batched_only:
        cb = QWEN7B_RAGGED_DECODE
        db = bench_decode(args, torch, Lb, cb, 2, args.batched_steps, 8, not args.no_dense, "batched:",
                          with_mass=True)
        db.pop("inp")
        print(json.dumps({k: v for k, v in db.items()}), flush=True)
        return
    d = bench_decode(args, torch, Lb, cfg, args.nbuf, args.steps, args.warmup, not args.no_dense)
    inp = d.pop("inp")
    ms_step, done, roof = d.pop("ms_step"), d.pop("steps"), d.pop("roofline")
    tok_s = B / (ms_step * 1e-3)
    extra = d
    extra["pages_context"] = "about 50% end-to-end inference speedup at 16K context (other hardware, whole model)"
    if not args.no_batched:
        cb = QWEN7B_RAGGED_DECODE
        db = bench_decode(args, torch, Lb, cb, 2, args.batched_steps, 8, not args.no_dense, "batched:",
                          with_mass=True)
        db.pop("inp")
        bms = db.pop("ms_step")
        db.pop("steps")
        extra["batched_decode"] = dict(workload=cb.name, batch=cb.B, context=f"{cb.L_lo}..{cb.L_hi} (seeded uniform)",
                                       tok_s=round(cb.B / (bms * 1e-3), 1), **db)
        del db
        torch.cuda.empty_cache()
    if not args.no_window:
        dw = bench_decode(args, torch, Lb, cfg, 8, 160, 16, False, "window:", flags=Lb.LISA_SLIDING_WINDOW)
        dw.pop("inp")
        wms = dw.pop("ms_step")
        dw.pop("steps")
        extra["window_decode"] = dict(what="sliding-window mode (window M, no indexer or select), same workload",
                                      tok_s=round(B / (wms * 1e-3), 1), us_per_step=dw["us_per_step"],
                                      kernel_us=dw["kernel_us"], step_hbm_roofline_frac=dw["step_hbm_roofline_frac"])
        torch.cuda.empty_cache()
    if not args.no_sweep:
        q14 = QWEN14B_DECODE_32K
        sweep = {}
        for Mv in q14.M_sweep:
            cm = q14.replace(M=Mv)
            dm = bench_decode(args, torch, Lb, cm, 2, 32, 4, Mv == q14.M_sweep[0] and not args.no_dense,
                              f"sweep{Mv}:")
            dm.pop("inp")
            mms = dm.pop("ms_step")
            dm.pop("steps")
            keep = ("us_per_step", "us_per_step_median_p10_p90", "kernel_us", "step_algorithmic_bytes",
                    "step_hbm_roofline_frac", "dense_decode_us_per_step", "speedup_vs_dense_decode")
            sweep[str(Mv)] = dict(tok_s=round(cm.B / (mms * 1e-3), 1), **{k: v for k, v in dm.items() if k in keep})
            torch.cuda.empty_cache()
        dense_us = sweep[str(q14.M_sweep[0])].get("dense_decode_us_per_step")
        if dense_us:
            for v in sweep.values():
                v["speedup_vs_dense_decode"] = round(dense_us / v["us_per_step"], 3)
        extra["m_sweep_decode"] = dict(workload=q14.name, batch=q14.B, context=q14.L, dense_decode_us_per_step=dense_us,
                                       **sweep)

    if not args.no_kl:
        extra["segment_correct"] = bench_segment(torch, Lb, QWEN7B_RAGGED_DECODE)
    if not args.no_prefill:
        extra.update(bench_prefill(args, torch, Lb, prefill_inputs))

    cpu = None if args.no_cpu else cpu_baseline(args, inp, M)
    if not args.no_dense:
        peaks = achievable_peaks(torch)
        extra["achievable_peaks"] = peaks
        if roof["unit"] == "GB/s":
            roof["frac_of_achievable"] = round(roof["achieved"] / peaks["hbm_copy_GBs"], 5)

    rec = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tok/s", "n_gpus": 1,
        "steps": done, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 caches and activations; no trained weights)",
        "config": {"workload": cfg.name, "batch": B, "context": Lctx, "M": M, "H_q": cfg.H_q,
                   "H_kv": cfg.H_kv, "head_dim": cfg.d, "hidden": cfg.hidden,
                   "indexer": f"{cfg.H_I}x{cfg.d_I}", "buffer_sets": args.nbuf},
        "roofline": roof,
        "cpu_baseline": cpu,
        # every detail under "extra"; the headline figures at top level after it,
        # so that they also end the line (a reader that keeps only the end of
        # the output, or only top-level keys, still has them), the C1 step last
        "extra": extra,
        "m_sweep_decode": {k: summary_leg(v) for k, v in (extra.get("m_sweep_decode") or {}).items()
                           if isinstance(v, dict)} or None,
        "batched_decode": summary_leg(extra.get("batched_decode")),
        "prefill": summary_prefill(extra),
        "decode": summary_decode(extra),
    }
    print(json.dumps(rec), flush=True)


def summary_decode(e):
    """The headline decode step: timing spread, per-kernel times and
    rooflines, the step's roofline and the same-GPU dense baseline."""
    return {"us_per_step": e.get("us_per_step"), "median_p10_p90": e.get("us_per_step_median_p10_p90"),
            "timed": e.get("step_spread_note"), "kernel_us": e.get("kernel_us"),
            "kernel_frac": {k: v["frac"] for k, v in (e.get("kernel_roofline") or {}).items()},
            "step_algorithmic_bytes": e.get("step_algorithmic_bytes"),
            "step_hbm_roofline_frac": e.get("step_hbm_roofline_frac"),
            "dense_decode_us_per_step": e.get("dense_decode_us_per_step"),
            "speedup_vs_dense_decode": e.get("speedup_vs_dense_decode")}


def summary_prefill(e):
    if "prefill_ms" not in e:
        return None
    return {"workload": e.get("prefill_workload"), "ms": e.get("prefill_ms"),
            "median_p10_p90": e.get("prefill_ms_median_p10_p90"), "tok_s": e.get("prefill_tok_s"),
            "kernel_us": e.get("prefill_kernel_us"),
            "kernel_frac": {k: (v["frac"], v["bound"]) for k, v in (e.get("prefill_kernel_roofline") or {}).items()},
            "sdpa_causal_attention_ms": e.get("dense_causal_prefill_attention_ms")}


def summary_leg(d):
    if not d:
        return None
    keep = ("workload", "batch", "tok_s", "us_per_step", "us_per_step_median_p10_p90", "step_hbm_roofline_frac",
            "kernel_us", "dense_decode_us_per_step", "speedup_vs_dense_decode")
    return {k: d[k] for k in keep if k in d}


def load_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy kernel's reading), if
    they were taken on the kernel's current source files; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        ent = json.load(open(path)).get(kernel)
        if not ent or ent.get("source_sha256") != source_hash(ent.get("sources", [])):
            return None
        return ent.get("bytes_per_launch")
    except Exception:
        return None


def source_hash(files):
    """sha256 over the named files of the package's csrc directory, in order."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_attention_lightning_amd", "csrc")
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def bench_prefill(args, torch, Lb, prefill_inputs):
    from lisa_inputs import QWEN7B_PREFILL_16K
    cfg = QWEN7B_PREFILL_16K
    n, M = cfg.n, cfg.M
    T = torch.bfloat16
    print(f"# prefill: {cfg.name} n={n}", file=sys.stderr, flush=True)
    inp = prefill_inputs(cfg)

    def up(a, dt=T):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt).contiguous()

    sh = Lb.make_shape(B=1, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d, H_I=cfg.H_I, H_Ik=cfg.H_Ik,
                       d_I=cfg.d_I, hidden=cfg.hidden, M=M, cap=n)
    t = {k: up(inp[k]) for k in ("q", "k", "v", "k_idx", "q_idx", "q_lin", "k_lin", "v_lin", "x",
                                 "w_gate")}
    S = up(inp["S0"], torch.float32)
    z = up(inp["z0"], torch.float32)
    w_idx = up(inp["w_idx"], torch.float32)
    out = torch.empty((1, n, cfg.H_q, cfg.d), dtype=T, device="cuda")
    ws = Lb.workspace(sh, Lb.LISA_OP_PREFILL, n)

    def call():
        Lb.lisa_prefill(sh, n, t["q"], t["k"], t["v"], t["k_idx"], t["q_idx"], t["q_lin"], t["k_lin"],
                        t["v_lin"], t["x"], t["w_gate"], w_idx, S, z, out, None, ws)

    kern = {}
    call()
    torch.cuda.synchronize()
    for kid in (4, 9, 10, 5, 3, 1, 19, 6):  # one launch each per call
        st = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        sp = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for e in st + sp:
            e.record()
        Lb.lisa_timing_enable(kid, st, sp)
        call()
        torch.cuda.synchronize()
        cnt = Lb.lisa_timing_count()
        Lb.lisa_timing_enable(0)
        kern[Lb.lisa_kernel_name(kid)] = round(st[0].elapsed_time(sp[0]) * 1e3, 1) if cnt else 0.0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.prefill_iters + 1)]
    ev[0].record()
    for i in range(args.prefill_iters):
        call()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.prefill_iters
    per_call = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.prefill_iters)])
    # algorithmic work of each prefill kernel (rows t < M take every key and are not scored)
    r0 = min(M, n)
    scored_pairs = (n * (n + 1) - r0 * (r0 + 1)) // 2
    attn_pairs = sum(min(M, t + 1) for t in range(n))
    # q_L, k_L, v_L read once (352.3 MB at n = 16384); the fp32
    # branch output is the library's intermediate, not algorithmic traffic
    lin_bytes = 3 * n * cfg.H_L * cfg.d * 2
    pwork = {
        "prefill_index_scores": (2 * cfg.H_I * cfg.d_I * scored_pairs, "mfma"),
        "prefill_linear": (lin_bytes, "hbm"),
        "prefill_attention": (4 * cfg.H_q * cfg.d * attn_pairs, "mfma"),
        "prefill_gate": (n * cfg.hidden * 2 + cfg.hidden * cfg.H_q * 2 + n * cfg.H_q * 4, "hbm"),
        "topm_select": (SELECT_OPS_PER_KEY * scored_pairs, "alu"),
        # the key-tile occupancy reads the selection bitmask once
        "prefill_tile_occupancy": (cfg.B * n * (((n + 31) // 32 + 1) // 2 * 2) * 4, "hbm"),
    }
    proofs = {k: kernel_roofline(k, kern[k] * 1e-3, *pwork[k], traffic_key="prefill:" + k) for k in pwork if kern.get(k)}
    # the linear branch as a whole (segment sums + prefix + chunked outputs)
    lin_us = sum(kern.get(k, 0.0) for k in ("prefill_linear_sums", "prefill_linear_prefix", "prefill_linear"))
    lin_flops = 2 * cfg.H_L * (n * cfg.d * 64 + 2 * n * cfg.d * cfg.d)  # causal half of A, A V, phi(Q) S, phi(K)^T V
    proofs["prefill_linear_branch"] = kernel_roofline("prefill_linear_branch", lin_us * 1e-3, lin_bytes, "hbm")
    proofs["prefill_linear_branch_mfma"] = kernel_roofline("prefill_linear_branch", lin_us * 1e-3, lin_flops, "mfma")
    dense = dense_prefill_baseline(torch, t["q"], t["k"], t["v"], cfg, n, args.prefill_iters)
    # the same prefill in sliding-window mode (no indexer; each row attends to its M most recent keys)
    window = None if args.no_window else bench_window_prefill(args, torch, Lb, cfg, t, S, z, out, ws, n, M)
    indexer_kl = None if args.no_kl else bench_indexer_kl(args, torch, Lb, cfg, sh, t, n)
    del ws
    torch.cuda.empty_cache()
    dropout = None if args.no_kl else bench_dropout(torch, Lb, cfg, sh, t, w_idx, n, M)
    res = {"prefill_workload": cfg.name, "prefill_ms": round(ms, 3),
           "prefill_ms_median_p10_p90": [round(float(np.median(per_call)), 3),
                                         round(float(np.percentile(per_call, 10)), 3),
                                         round(float(np.percentile(per_call, 90)), 3)],
           "dense_causal_prefill_attention_ms": dense, "window_prefill": window,
           "prefill_tok_s": round(n / (ms * 1e-3), 1), "prefill_kernel_us": kern,
           "prefill_kernel_roofline": proofs, "indexer_kl": indexer_kl, "candidate_dropout": dropout}
    del t, out
    torch.cuda.empty_cache()
    return res


def bench_window_prefill(args, torch, Lb, cfg, t, S, z, out, ws, n, M):
    """The prefill in sliding-window mode: no indexer or select, each row
    attends to its M most recent keys."""
    shw = Lb.make_shape(B=1, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d, H_I=cfg.H_I, H_Ik=cfg.H_Ik,
                        d_I=cfg.d_I, hidden=cfg.hidden, M=M, cap=n, flags=Lb.LISA_SLIDING_WINDOW)

    def call_w():
        Lb.lisa_prefill(shw, n, t["q"], t["k"], t["v"], None, None, t["q_lin"], t["k_lin"],
                        t["v_lin"], t["x"], t["w_gate"], None, S, z, out, None, ws)

    call_w()
    st_w = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    sp_w = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in st_w + sp_w:
        e.record()
    torch.cuda.synchronize()
    Lb.lisa_timing_enable(6, st_w, sp_w)
    call_w()
    torch.cuda.synchronize()
    attn_w = round(st_w[0].elapsed_time(sp_w[0]) * 1e3, 1) if Lb.lisa_timing_count() else None
    Lb.lisa_timing_enable(0)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.prefill_iters):
        call_w()
    t1.record()
    torch.cuda.synchronize()
    ms_w = t0.elapsed_time(t1) / args.prefill_iters
    return {"ms": round(ms_w, 3), "tok_s": round(n / (ms_w * 1e-3), 1), "attention_us": attn_w,
            "what": "sliding-window mode, window M, no indexer or select"}


def bench_indexer_kl(args, torch, Lb, cfg, sh, t, n):
    """The indexer training objective over the same prefill: per-row,
    per-head KL against the grouped teacher attention and the loss."""
    kl = torch.empty((1, n, cfg.H_I), dtype=torch.float32, device="cuda")
    loss = torch.empty((1,), dtype=torch.float32, device="cuda")

    def call():
        Lb.lisa_indexer_kl(sh, n, t["q"], t["k"], t["q_idx"], t["k_idx"], kl, loss)

    call()
    torch.cuda.synchronize()
    st = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    sp = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for e in st + sp:
        e.record()
    torch.cuda.synchronize()
    Lb.lisa_timing_enable(17, st, sp)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    cnt = Lb.lisa_timing_count()
    Lb.lisa_timing_enable(0)
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(st[:cnt], sp[:cnt])]))
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    iters = max(1, args.prefill_iters // 2)
    t0.record()
    for _ in range(iters):
        call()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / iters
    pairs = n * (n + 1) // 2
    # logits of every causal pair: the teacher heads over d and the index heads over d_I
    flops = 2 * pairs * (cfg.H_q * cfg.d + cfg.H_I * cfg.d_I)
    roof = kernel_roofline("indexer_kl", k_ms, flops, "mfma", traffic_key="prefill:indexer_kl")
    return {"what": "indexer training objective forward (LISA Eq. 2): KL of each row's indexer softmax from the "
                    "mean of its 7 teacher heads' causal attention, all 16384 rows x 4 heads, and the loss",
            "ms_per_call": round(ms, 3), "kernel_us": round(k_ms * 1e3, 1),
            "note": "two passes over every causal pair (the row's teacher log-sum-exps first); the roofline counts "
                    "one pass of logits, so executed MFMA work is twice the algorithmic",
            "kernel_roofline": roof, "loss": round(float(loss.item()), 6)}


def bench_dropout(torch, Lb, cfg, sh, t, w_idx, n, M):
    """Candidate dropout over every row of the prefill: the indexer's own
    scores of the 16K tokens, uniform draws from torch, ceil(1.2 M)
    candidates and p = 0.2 (the paper's early-training setting)."""
    ld = (n + 3) // 4 * 4
    scores = torch.zeros((1, n, ld), dtype=torch.float32, device="cuda")
    idx0 = torch.empty((1, n, M), dtype=torch.int32, device="cuda")
    Lb.lisa_indexer_topk(sh, Lb.LISA_ROWS_PREFILL, n, None, t["q_idx"], t["k_idx"], w_idx, None, ld, scores, idx0,
                         None)
    del idx0
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    u = torch.rand((1, n, ld), dtype=torch.float32, device="cuda", generator=g)
    idx = torch.empty((1, n, M), dtype=torch.int32, device="cuda")
    ws = Lb.workspace(sh, Lb.LISA_OP_DROPOUT_PREFILL, n)
    n_cand = -(-6 * M // 5)

    def call():
        Lb.lisa_candidate_dropout(sh, Lb.LISA_ROWS_PREFILL, n, None, scores, u, ld, n_cand, 0.2, idx, ws)

    call()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    iters = 4
    t0.record()
    for _ in range(iters):
        call()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / iters
    kept = float((idx >= 0).sum(dim=2).float().mean().item())
    rows_len = n * (n + 1) // 2
    # two selections over every row (candidates, then survivors) plus the survivor mask pass
    work = 2 * SELECT_OPS_PER_KEY * rows_len
    res = {"what": "indexer candidate dropout over all 16384 prefill rows: top ceil(1.2 M) = %d candidates, "
                   "uniform draws, p = 0.2, the M best survivors" % n_cand,
           "ms_per_call": round(ms, 3), "mean_kept_per_row": round(kept, 1),
           "roofline": kernel_roofline("candidate_dropout", ms, work, "alu"),
           "note": "call time (two select launches, the survivor-score pass and the compaction); integer work "
                   "counted as for the top-M select"}
    del scores, u, idx, ws
    torch.cuda.empty_cache()
    return res


def achievable_peaks(torch):
    """What this GPU delivers to plain library work, next to the published
    peaks: a 1 GiB device-to-device copy (HBM read + write) and an 8192^3
    bf16 GEMM through torch (2-D, contiguous operands)."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * 4 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn((m, m), device="cuda").to(torch.bfloat16).contiguous()
    b = torch.randn((m, m), device="cuda").to(torch.bfloat16).contiguous()
    c = torch.empty((m, m), dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 2 * m ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_copy_GBs": round(copy_gbs, 1), "hbm_copy_frac_of_published": round(copy_gbs / HBM_PEAK_GBS, 3),
            "bf16_gemm_TFLOPs": round(gemm_tf, 1),
            "bf16_gemm_frac_of_published": round(gemm_tf / MFMA_BF16_PEAK_TFLOPS, 3),
            "what": "torch device copy of 1 GiB (read + write) and torch.matmul of two 8192 x 8192 bf16 matrices, "
                    "10 timed runs each"}


def bench_segment(torch, Lb, cfg):
    """Segment state correction of the linear state of a 32-sequence batch
    (elementwise over S and z: 24 bytes per state element)."""
    B = 32
    sh = Lb.make_shape(B=B, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d, H_I=cfg.H_I, H_Ik=cfg.H_Ik, d_I=cfg.d_I,
                       hidden=cfg.hidden, M=cfg.M, cap=cfg.cap, max_len=cfg.cap)
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    mk = lambda *shape: torch.randn(shape, dtype=torch.float32, device="cuda", generator=g)
    S, S0, mS = (mk(B, cfg.H_L, cfg.d, cfg.d) for _ in range(3))
    z, z0, mz = (mk(B, cfg.H_L, cfg.d) for _ in range(3))
    st = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    sp = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for e in st + sp:
        e.record()
    torch.cuda.synchronize()
    Lb.lisa_timing_enable(13, st, sp)
    for i in range(8):
        Lb.lisa_segment_correct(sh, S, z, S0, z0, mS, mz, i + 2, 0.3)
    torch.cuda.synchronize()
    cnt = Lb.lisa_timing_count()
    Lb.lisa_timing_enable(0)
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(st[:cnt], sp[:cnt])]))
    elems = B * cfg.H_L * cfg.d * (cfg.d + 1)
    res = {"what": "segment state correction (LISA Eqs. 6-9) of 32 sequences' 28 x 128 x 128 states and "
                   "normalisers", "kernel_us": round(k_ms * 1e3, 2),
           "roofline": kernel_roofline("segment_correct", k_ms, 24 * elems, "hbm")}
    del S, S0, mS, z, z0, mz
    torch.cuda.empty_cache()
    return res


def dense_prefill_baseline(torch, q, k, v, cfg, n, iters):
    """Dense causal attention over the same prefill q, k, v with torch's
    scaled_dot_product_attention (a library baseline on the same GPU; the
    fused flash / memory-efficient backends only, never the math path)."""
    try:
        import torch.nn.functional as F
        from torch.nn.attention import SDPBackend, sdpa_kernel
        G = cfg.H_q // cfg.H_kv
        qh = q.view(1, n, cfg.H_q, cfg.d).transpose(1, 2).contiguous()
        kh = k.view(1, n, cfg.H_kv, cfg.d).repeat_interleave(G, dim=2).transpose(1, 2).contiguous()
        vh = v.view(1, n, cfg.H_kv, cfg.d).repeat_interleave(G, dim=2).transpose(1, 2).contiguous()
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            F.scaled_dot_product_attention(qh, kh, vh, is_causal=True)
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(iters):
                F.scaled_dot_product_attention(qh, kh, vh, is_causal=True)
            t1.record()
            torch.cuda.synchronize()
        return {"ms": round(t0.elapsed_time(t1) / iters, 3), "what": "torch SDPA (flash/efficient backend), causal, "
                "K/V repeated to the query heads, attention only (no indexer, select, linear branch or gate)"}
    except Exception as e:  # no fused backend in this torch: not reported
        return {"ms": None, "error": str(e)[:200]}


def cpu_baseline(args, inp, M):
    """The fp64 oracle's decode step on the host, over a bounded sample."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = None
    cores = len(os.sched_getaffinity(0))
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode_step(inp, M)
        n += 1
        if time.perf_counter() - t0 > args.cpu_seconds:
            break
    dt = time.perf_counter() - t0
    B = len(inp["seq_lens"])
    res = {"value": round(n * B / dt, 3), "unit": "tok/s", "cores": blas or cores,
           "kind": "oracle", "sample": f"{n} decode steps of the same workload (fp64 NumPy), {dt:.1f} s",
           "affinity_cores": cores}
    try:  # the same oracle on one BLAS thread
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            n1 = 0
            t1 = time.perf_counter()
            while True:
                oracle.decode_step(inp, M)
                n1 += 1
                if time.perf_counter() - t1 > args.cpu_seconds / 3:
                    break
            d1 = time.perf_counter() - t1
        res["single_thread"] = {"value": round(n1 * B / d1, 3), "unit": "tok/s", "sample": f"{n1} steps, {d1:.1f} s"}
    except Exception as e:  # threadpoolctl missing: report without it
        res["single_thread"] = {"value": None, "error": str(e)[:200]}
    res["per_config"] = cpu_per_config(args)
    return res


def cpu_per_config(args):
    """The oracle on bounded samples of the other timed workloads (input
    generation excluded): 4 sequences of the ragged batch, one sequence of
    the 32K / 40-head decode at M = 2048 and, with --cpu-all, one row of the
    16K prefill."""
    import oracle
    from lisa_inputs import QWEN7B_RAGGED_DECODE, QWEN7B_PREFILL_16K, QWEN14B_DECODE_32K, decode_inputs, prefill_inputs
    budget = max(1.0, args.cpu_seconds / 3)
    out = {}

    def loop(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 > budget:
                return n, time.perf_counter() - t0

    ragged = QWEN7B_RAGGED_DECODE.replace(B=4)
    inp_ragged = decode_inputs(ragged)
    n, dt = loop(lambda: oracle.decode_step(inp_ragged, ragged.M))
    out[ragged.name] = {"value": round(n * ragged.B / dt, 3), "unit": "tok/s",
                        "sample": f"{n} steps of 4 sequences, lengths {inp_ragged['seq_lens'].tolist()}, {dt:.1f} s"}
    del inp_ragged
    if args.cpu_all:  # about half a minute: the oracle's prefill builds the whole sequence's linear state
        pre = QWEN7B_PREFILL_16K
        inp_pre = prefill_inputs(pre)
        rows = [8191]
        n, dt = loop(lambda: oracle.prefill_rows(inp_pre, pre.M, rows))
        out[pre.name] = {"value": round(n * len(rows) / dt, 4), "unit": "rows/s",
                         "sample": f"{n} call(s) of the output of prefill row {rows[0]}, which includes the linear "
                                   f"state over the whole 16384-token sequence, {dt:.1f} s"}
        del inp_pre
    q14 = QWEN14B_DECODE_32K.replace(B=1)
    inp_q14 = decode_inputs(q14)
    n, dt = loop(lambda: oracle.decode_step(inp_q14, 2048))
    out[q14.name] = {"value": round(n / dt, 3), "unit": "tok/s",
                    "sample": f"{n} steps of one 32768-token sequence, M = 2048, {dt:.1f} s"}
    return out


if __name__ == "__main__":
    main()
