"""Segment state correction ("LISA", arXiv 2607.19358v1, Section 3.3, Eqs.
6-9) of the HIP path against the fp64 oracle, through the C ABI, over a run
of segments of a real linear-branch state."""
import numpy as np
import pytest
import torch

import long_context_attention_lightning_amd as L
import oracle
from lisa_inputs import QWEN7B_PREFILL_16K, prefill_inputs
from gpu_helpers import dev, host, shape_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("alpha", [0.0, 0.3, 1.0])
def test_segment_correction_run_matches_oracle(alpha):
    """Six segments of 64 tokens: each segment's tokens enter the state
    (lisa_linear_state_update), then the segment is corrected; the GPU state,
    start state and mean direction track the oracle's."""
    cfg = QWEN7B_PREFILL_16K.replace(B=2, n=384, cap=384, H_q=4, H_kv=1, H_L=4, d=128, hidden=64)
    inp = prefill_inputs(cfg, n=384, salt=11)
    sh = shape_of(cfg, M=64, cap=384, B=2)
    T = torch.bfloat16
    S = dev(inp["S0"], torch.float32)
    z = dev(inp["z0"], torch.float32)
    S_start, z_start = S.clone(), z.clone()
    mS = torch.full_like(S, float("nan"))  # not read for the first segment
    mz = torch.full_like(z, float("nan"))
    rS, rz = inp["S0"].astype(np.float64), inp["z0"].astype(np.float64)
    rS0, rz0 = rS.copy(), rz.copy()
    rmS, rmz = np.zeros_like(rS), np.zeros_like(rz)
    k = 64
    for t in range(1, 7):
        lo, hi = (t - 1) * k, t * k
        L.lisa_linear_state_update(sh, k, dev(inp["k_lin"][:, lo:hi], T), dev(inp["v_lin"][:, lo:hi], T), S, z)
        L.lisa_segment_correct(sh, S, z, S_start, z_start, mS, mz, t, alpha)
        torch.cuda.synchronize()
        # oracle: the same tokens (bf16 values) enter the fp64 state, then the correction
        for b in range(2):
            rS[b], rz[b] = oracle.linear_state_update(inp["k_lin"][b, lo:hi], inp["v_lin"][b, lo:hi], rS[b], rz[b])
        rS, rz, rmS, rmz = oracle.segment_correct(rS, rz, rS0, rz0, rmS, rmz, t, alpha)
        rS0, rz0 = rS.copy(), rz.copy()
        for name, g, r in (("S", S, rS), ("z", z, rz), ("S_start", S_start, rS0), ("mean_S", mS, rmS),
                           ("mean_z", mz, rmz)):
            err = np.max(np.abs(host(g) - r)) / max(np.max(np.abs(r)), 1e-30)
            print(f"[alpha={alpha} t={t}] {name} rel={err:.3e}", flush=True)
            assert err <= 1e-4, (name, t, err)
