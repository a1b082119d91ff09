"""GPU test of kda_decode_step_static (the decode step for callers that cannot allocate:
its workspace is the library's static device array) against kda_decode_step with a
caller workspace, through the C ABI: the same model, state and inputs give the same
outputs and states bit for bit (the same kernels in the same order), on two calls in a
row, the second with a smaller batch; and a batch too large for the array is refused
before anything is enqueued."""
import sys

import numpy as np
import pytest

import synth
from tests.helpers import gpu_model

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _step_pair(model, run, B, steps, torch, kda):
    """`steps` tokens through both entry points from the same state; returns the max
    difference of outputs and states (must be 0)."""
    st_a = model.new_state(B)
    st_a.S.copy_(torch.from_numpy(run.s0[:, :B]))
    st_b = st_a.clone()
    ws = model.workspace(kda.KDA_OP_DECODE, B)
    ya = torch.empty((B, model.d_model), dtype=torch.float32, device="cuda")
    yb = torch.empty_like(ya)
    diff = 0.0
    for t in range(steps):
        x = torch.from_numpy(np.ascontiguousarray(run.x[t, :B, 0, :])).cuda()
        kda.kda_decode_step(model.handle, x, ya, st_a, ws)
        kda.kda_decode_step_static(model.handle, x, yb, st_b)
        torch.cuda.synchronize()
        diff = max(diff, float((ya - yb).abs().max()), float((st_a.S - st_b.S).abs().max()),
                   float((st_a.conv - st_b.conv).abs().max()))
    return diff


def test_static_scratch_decode_matches_workspace_decode():
    import torch
    import linear_attention_decode_amd as kda
    w = synth.scaled(synth.WORKLOADS["stack"], n_layers=2, batch=4, steps=3, seed=111)
    run = synth.draw_run(w)
    model = gpu_model(run)
    _say("static-scratch decode: B=4 then B=2, 2-layer Q8_0 stack (per-layer kernels)")
    assert _step_pair(model, run, 4, 3, torch, kda) == 0.0
    assert _step_pair(model, run, 2, 3, torch, kda) == 0.0
    _say("  B=1 one-launch (no scratch use) and B=1 per-layer")
    assert _step_pair(model, run, 1, 2, torch, kda) == 0.0
    model.set_option(kda.KDA_OPT_PERSISTENT, 0)
    assert _step_pair(model, run, 1, 2, torch, kda) == 0.0
    # a batch whose workspace exceeds the array is refused up front
    big = model.new_state(200)
    assert kda.kda_workspace_bytes(model.handle, kda.KDA_OP_DECODE, 200, 1) > (8 << 20)
    x = torch.zeros((200, model.d_model), dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(kda.KdaError) as ei:
        kda.kda_decode_step_static(model.handle, x, y, big)
    assert ei.value.status == kda._lib.KDA_E_WORKSPACE
    model.close()


def test_static_scratch_shared_across_models():
    """Two models on one GPU take turns on the same array (serialised calls): each keeps
    matching its own workspace path."""
    import torch
    import linear_attention_decode_amd as kda
    d = synth.LayerDims(d_model=256, n_heads=2, d_k=64, d_v=64, rank_f=32, rank_g=32)
    w1 = synth.scaled(synth.WORKLOADS["tiny"], dims=d, wtype="bf16", batch=3, steps=3, s0_std=0.1, seed=112)
    w2 = synth.scaled(synth.WORKLOADS["stack"], n_layers=1, batch=3, steps=3, seed=113)
    r1, r2 = synth.draw_run(w1), synth.draw_run(w2)
    m1, m2 = gpu_model(r1), gpu_model(r2)
    _say("static-scratch decode: two models alternating")
    for _ in range(2):
        assert _step_pair(m1, r1, 3, 3, torch, kda) == 0.0
        assert _step_pair(m2, r2, 3, 3, torch, kda) == 0.0
    m1.close()
    m2.close()
