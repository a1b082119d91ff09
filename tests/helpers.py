"""Shared test helpers: build the oracle and the GPU model from the same seeded draws,
and the tolerance metrics used by every parity test.

Tolerances (floating point):
  * layer / stack outputs: range-relative error max|y - y_ref| / max|y_ref| <= 1e-3 per
    compared tensor (one decode step's output for all sequences);
  * recurrent state: max |S - S_ref| <= 2e-3 elementwise.
The GPU path computes in fp32 with fp32 accumulation against an fp64 oracle; both sides
use the same quantised / rounded weights (checked bit-exact separately).
"""
from __future__ import annotations

import numpy as np

import synth
from oracle import kda as ok

OUT_RTOL = 1e-3
STATE_ATOL = 2e-3


def range_rel(y, ref) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(y - ref).max() / max(np.abs(ref).max(), 1e-30))


def oracle_layers(run: synth.RunInputs):
    w = run.workload
    d = w.dims
    return [ok.prepare_layer(dr, w.wtype, d.n_heads, d.d_k, d.d_v, w.norm_eps, w.l2_eps,
                             gate=d.gate, gate_lb=w.gate_lb)
            for dr in run.layers]


def gpu_model(run: synth.RunInputs):
    import linear_attention_decode_amd as kda
    w = run.workload
    d = w.dims
    return kda.KdaModel(run.layers, n_heads=d.n_heads, d_k=d.d_k, d_v=d.d_v, wtype=w.wtype,
                        prenorm_residual=w.prenorm_residual, norm_eps=w.norm_eps,
                        l2_eps=w.l2_eps, gate=d.gate, gate_lb=w.gate_lb)


def gpu_decode(model, run: synth.RunInputs, steps: int, snapshot_every: int = 0,
               graph: bool = True, persistent: bool = True):
    """Decode `steps` tokens on the GPU from S0 / zero window.  Returns (y [steps][B][D],
    S, window, snapshots)."""
    import torch
    w = run.workload
    B = w.batch
    st = model.new_state(B)
    st.S.copy_(torch.from_numpy(run.s0))
    ws = model.workspace(0, B)
    model.set_option(0, 1 if graph else 0)
    model.set_option(2, 1 if persistent else 0)
    x_all = torch.from_numpy(np.ascontiguousarray(run.x[:steps, :, 0, :])).cuda()
    y = torch.empty((B, model.d_model), dtype=torch.float32, device="cuda")
    ys = torch.empty((steps, B, model.d_model), dtype=torch.float32, device="cuda")
    snaps = {}
    for t in range(steps):
        xt = x_all[t].contiguous()
        model.decode_step(xt, y, st, ws)
        ys[t].copy_(y)
        if snapshot_every and (t + 1) % snapshot_every == 0:
            snaps[t + 1] = st.S.detach().cpu().numpy().copy()
    torch.cuda.synchronize()
    model.status()
    return ys.cpu().numpy(), st.S.cpu().numpy(), st.conv.cpu().numpy(), snaps
