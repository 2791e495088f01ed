"""The allocation-free decode step (lisa_decode_step_noalloc) against the
workspace entry point lisa_decode_step on the same inputs: the same kernels
run, so outputs, index lists, caches and states must agree bit for bit.
Two calls in a row share the library's static scratch, the second with a
smaller shape; a shape that needs more than the scratch is rejected."""
import numpy as np
import pytest
import torch

import long_context_attention_lightning_amd as L
from lisa_inputs import QWEN7B_DECODE_16K, QWEN7B_RAGGED_DECODE, decode_inputs
from gpu_helpers import dev, host, shape_of, tdtype

pytestmark = pytest.mark.gpu


def _step(cfg, inp, noalloc):
    T = tdtype(cfg)
    seq = inp["seq_lens"]
    sh = shape_of(cfg, max_len=int(seq.max()), cap=inp["k_cache"].shape[1], B=len(seq))
    t = {k: dev(inp[k], T) for k in ("q", "k_new", "v_new", "q_idx", "k_idx_new", "q_lin", "k_lin", "v_lin",
                                     "x", "w_gate", "k_cache", "v_cache", "k_idx_cache")}
    S, z = dev(inp["S0"], torch.float32), dev(inp["z0"], torch.float32)
    out = torch.empty((len(seq), cfg.H_q, cfg.d), dtype=T, device="cuda")
    idx = torch.full((len(seq), cfg.M), -7, dtype=torch.int32, device="cuda")
    args = (sh, torch.from_numpy(seq.astype(np.int32)).cuda(), t["q"], t["k_new"], t["v_new"], t["q_idx"],
            t["k_idx_new"], t["q_lin"], t["k_lin"], t["v_lin"], t["x"], t["w_gate"],
            dev(inp["w_idx"], torch.float32), t["k_cache"], t["v_cache"], t["k_idx_cache"], S, z, out, idx)
    if noalloc:
        L.lisa_decode_step_noalloc(*args)
    else:
        L.lisa_decode_step(*args, L.workspace(sh, L.LISA_OP_DECODE))
    torch.cuda.synchronize()
    return {"out": host(out), "idx": host(idx), "S": host(S), "z": host(z),
            "k_cache": host(t["k_cache"]), "k_idx_cache": host(t["k_idx_cache"])}


def _same(a, b, label):
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{label}: {k} differs"
    print(f"[{label}] bit-identical: {', '.join(a)}", flush=True)


def test_noalloc_matches_workspace_step_twice_then_smaller():
    big = QWEN7B_DECODE_16K                                     # batch 1, 16384 tokens, M = 2048
    small = QWEN7B_RAGGED_DECODE.replace(B=3, L_lo=100, L_hi=3000, cap=3000, M=256)
    for label, cfg in (("16K batch 1", big), ("again, batch 3 up to 3000 tokens, M = 256", small)):
        inp = decode_inputs(cfg)
        _same(_step(cfg, inp, True), _step(cfg, inp, False), label)


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    cfg = QWEN7B_RAGGED_DECODE  # batch 32 at up to 32K tokens: its score rows alone take 4 MiB
    sh = shape_of(cfg, max_len=32768, cap=32768, B=32)
    assert L.lisa_workspace_bytes(sh, L.LISA_OP_DECODE, 0) > L.LISA_DECODE_SCRATCH_BYTES
    import ctypes
    lib = L.library()  # the size check comes before any pointer is looked at
    rc = lib.lisa_decode_step_noalloc(ctypes.byref(sh), *([None] * 19), None)
    err = L.lisa_last_error()
    print(f"[too large] status {rc}: {err}", flush=True)
    assert rc == -3 and "allocation-free" in err
