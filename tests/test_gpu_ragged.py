"""GPU parity of batched decode with ragged / left-padded sequences (kda_decode_step_masked).

Each sequence b takes tokens only at its own steps [start_b, start_b + len_b) of the batch's
step loop (left padding before, ragged end after); at every other step its mask entry is 0
and its state and window must stay exactly as they were.  Each sequence is compared with
the oracle run on that sequence's own tokens alone: every output of an active step, the
final state, and the final window.  A step's inputs for masked rows are garbage on purpose
(large values), which must not reach any state.
"""
import sys

import numpy as np
import pytest

import synth
from oracle import kda as ok
from tests.helpers import OUT_RTOL, STATE_ATOL, gpu_model, oracle_layers, range_rel

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _ragged(w, starts, lens, graph=True):
    import torch
    run = synth.draw_run(w)
    layers = oracle_layers(run)
    model = gpu_model(run)
    B, steps = w.batch, w.steps
    mask = np.zeros((steps, B), np.int32)
    for b in range(B):
        mask[starts[b]:starts[b] + lens[b], b] = 1
    x = run.x[:, :, 0, :].copy()
    rng = np.random.default_rng(7)
    x[mask == 0] = rng.standard_normal((int((mask == 0).sum()), x.shape[-1])).astype(np.float32) * 50
    st = model.new_state(B)
    st.S.copy_(torch.from_numpy(run.s0))
    ws = model.workspace(0, B)
    model.set_option(0, 1 if graph else 0)
    xs = torch.from_numpy(x).cuda()
    ms = torch.from_numpy(mask).cuda()
    y = torch.empty((B, model.d_model), dtype=torch.float32, device="cuda")
    ys = torch.empty((steps, B, model.d_model), dtype=torch.float32, device="cuda")
    for t in range(steps):
        before = (st.S.clone(), st.conv.clone())
        model.decode_step_masked(xs[t].contiguous(), y, st, ms[t].contiguous(), ws)
        ys[t].copy_(y)
        for b in range(B):
            if mask[t, b] == 0:
                assert torch.equal(st.S[:, b], before[0][:, b]), f"step {t}: masked seq {b} state moved"
                assert torch.equal(st.conv[:, b], before[1][:, b]), f"step {t}: masked seq {b} window moved"
    torch.cuda.synchronize()
    ys = ys.cpu().numpy()
    S, Z = st.S.cpu().numpy(), st.conv.cpu().numpy()
    worst = 0.0
    for b in range(B):
        steps_b = np.nonzero(mask[:, b])[0]
        xb = run.x[steps_b, b:b + 1]                      # [len][1][1][D]
        ry, rS, rZ, _ = ok.decode_run(layers, xb, run.s0[:, b:b + 1], w.prenorm_residual)
        for i, t in enumerate(steps_b):
            e = range_rel(ys[t, b], ry[i, 0])
            worst = max(worst, e)
            assert e <= OUT_RTOL, f"seq {b} step {t}: output error {e:.3e}"
        assert np.abs(S[:, b] - rS[:, 0]).max() <= STATE_ATOL, f"seq {b}: state"
        assert range_rel(Z[:, b], rZ[:, 0]) <= OUT_RTOL, f"seq {b}: window"
    model.close()
    return worst


def test_ragged_q8_0_stack_b5():
    """B=5 sequences of lengths 6, 3, 5, 1, 4 starting at steps 0, 2, 1, 5, 0 over 6 steps
    (left padding and ragged ends), a 2-layer Q8_0 stack at D=2048 (vector projections)."""
    w = synth.scaled(synth.WORKLOADS["stack"], n_layers=2, batch=5, steps=6, seed=91)
    _say("ragged decode q8_0 2 layers D=2048 B=5")
    e = _ragged(w, starts=[0, 2, 1, 5, 0], lens=[6, 3, 5, 1, 4])
    _say(f"  worst output error {e:.2e}")


def test_ragged_q8_0_stack_b12_matrix_cores():
    """B=12 (the projections on the matrix cores, whose epilogue rolls the windows)."""
    w = synth.scaled(synth.WORKLOADS["stack"], n_layers=2, batch=12, steps=5, seed=92)
    starts = [0, 1, 2, 3, 4, 0, 0, 1, 2, 0, 3, 4]
    lens = [5, 4, 3, 2, 1, 2, 3, 1, 2, 5, 1, 1]
    _say("ragged decode q8_0 2 layers D=2048 B=12 (MFMA projections)")
    _ragged(w, starts, lens)


@pytest.mark.parametrize("wtype", ["f32", "bf16"])
def test_ragged_single_layer_eager(wtype):
    """A single layer (no residual), eager launches (no graph), F32 and BF16 weights."""
    d = synth.LayerDims(d_model=256, n_heads=2, d_k=64, d_v=64, rank_f=32, rank_g=32)
    w = synth.scaled(synth.WORKLOADS["tiny"], dims=d, wtype=wtype, batch=4, steps=5,
                     s0_std=0.1, seed=93)
    _say(f"ragged decode single layer {wtype} B=4, eager")
    _ragged(w, starts=[0, 1, 3, 0], lens=[5, 2, 2, 3], graph=False)
