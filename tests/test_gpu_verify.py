"""GPU parity of multi-token verify + commit against the oracle.

Verify runs T tokens per sequence through every layer from the committed state without
changing it and records a replay log; commit advances the state to the one reached after
the accepted prefix.  Compared per step: every token's output (accepted or not), and the
committed state and conv window.
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


def gpu_verify(model, run, steps, accept=None, snap_every=1):
    """Verify + commit for `steps` steps.  Returns the outputs of every step and the
    committed (S, window) after every `snap_every`-th step.  After every commit the window
    roll is checked bit for bit: with a accepted tokens, rows [0, 3 - a) of the new window
    are rows [a, 3) of the previous one."""
    import torch
    w = run.workload
    B, T = w.batch, w.tokens
    st = model.new_state(B)
    st.S.copy_(torch.from_numpy(run.s0))
    ws = model.workspace(1, B, T)
    log = model.verify_log(B, T)
    acc = run.accept if accept is None else accept
    xs = torch.from_numpy(np.ascontiguousarray(run.x[:steps])).cuda()
    ys = torch.empty((steps, B, T, model.d_model), dtype=torch.float32, device="cuda")
    accs = torch.from_numpy(np.ascontiguousarray(acc[:steps]).astype(np.int32)).cuda()
    states = {}
    for t in range(steps):
        prev = st.conv.clone()
        model.verify_steps(xs[t].contiguous(), T, ys[t], st, log, ws)
        model.verify_commit(st, log, T, accs[t].contiguous())
        for b in range(B):
            a = int(min(max(acc[t, b], 1), T))
            if a < 3:
                assert torch.equal(st.conv[:, b, :3 - a].view(torch.int32),
                                   prev[:, b, a:].view(torch.int32)), f"step {t} seq {b}: window roll"
        if (t + 1) % snap_every == 0:
            states[t] = (st.S.cpu().numpy().copy(), st.conv.cpu().numpy().copy())
    torch.cuda.synchronize()
    return ys.cpu().numpy(), states


def _check(w, steps, accept=None, snap_every=1):
    run = synth.draw_run(w)
    layers = oracle_layers(run)
    model = gpu_model(run)
    acc = run.accept if accept is None else accept
    y, states = gpu_verify(model, run, steps, acc, snap_every)
    worst = 0.0
    # oracle step by step (verify_run's commit semantics), recording each committed state
    ry_all = np.empty((steps,) + run.x.shape[1:3] + (run.x.shape[3],))
    S = [[np.array(run.s0[l, b], np.float64) for b in range(w.batch)] for l in range(w.n_layers)]
    Z = [[np.zeros((3, w.dims.conv_channels)) for _ in range(w.batch)] for _ in range(w.n_layers)]
    for t in range(steps):
        for b in range(w.batch):
            yb, s_new, z_new = ok.stack_step(layers, run.x[t, b].astype(np.float64),
                                             [S[l][b] for l in range(w.n_layers)],
                                             [Z[l][b] for l in range(w.n_layers)],
                                             keep_after=int(min(max(acc[t, b], 1), w.tokens)))
            ry_all[t, b] = yb
            for l in range(w.n_layers):
                S[l][b], Z[l][b] = s_new[l], z_new[l]
        e = range_rel(y[t], ry_all[t])
        worst = max(worst, e)
        assert e <= OUT_RTOL, f"step {t}: output range-rel error {e:.3e}"
        if t not in states:
            continue
        gS, gZ = states[t]
        rS = np.array([[S[l][b] for b in range(w.batch)] for l in range(w.n_layers)])
        rZ = np.array([[Z[l][b] for b in range(w.batch)] for l in range(w.n_layers)])
        serr = np.abs(gS - rS).max()
        assert serr <= STATE_ATOL, f"step {t}: committed state error {serr:.3e}"
        assert range_rel(gZ, rZ) <= OUT_RTOL
    model.close()
    return worst


def test_verify_small_stack():
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=2, batch=3, steps=4, seed=31)
    _say("verify 2 layers B=3 T=4 D=2048 q8_0, 4 steps")
    _check(w, w.steps)


def test_verify_ragged_columns_matrix_cores():
    """B=5 x T=3 = 15 token positions at D=2048: MFMA projections with a padded column tile."""
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=2, batch=5, tokens=3, steps=3, seed=35)
    _say("verify 2 layers B=5 T=3 D=2048 q8_0, 3 steps (MFMA projections)")
    _check(w, w.steps)


@pytest.mark.parametrize("T", [1, 2, 3])
def test_verify_token_counts(T):
    d = synth.LayerDims(d_model=96, n_heads=3, d_k=64, d_v=64, rank_f=32, rank_g=32)
    w = synth.scaled(synth.WORKLOADS["verify"], dims=d, n_layers=2, batch=2, steps=3, tokens=T,
                     seed=40 + T)
    _say(f"verify ragged dims T={T}")
    _check(w, w.steps)


@pytest.mark.parametrize("D,rank", [(1024, 32), (2048, 64)])
def test_verify_low_rank_gates_matrix_cores(D, rank):
    """Verify of a model with the one-launch copies at ranks 32 and 64: the many-column gates
    on the matrix cores with lane groups past rank / 32 empty, 12 columns (a full and a
    partial group of 8); D = 1024 also takes the vector projections and the separate conv."""
    d = synth.LayerDims(d_model=D, n_heads=D // 128, d_k=128, d_v=128, rank_f=rank, rank_g=rank)
    w = synth.scaled(synth.WORKLOADS["verify"], dims=d, n_layers=2, batch=3, steps=3,
                     seed=80 + rank)
    _say(f"verify D={D} rank={rank} 2 layers B=3 T=4, 3 steps")
    _check(w, w.steps)


def test_verify_accept_clamped():
    """Accept lengths outside 1..T are clamped: 0 commits one token, 9 commits T."""
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=1, batch=2, steps=2, seed=50)
    acc = np.array([[0, 9], [9, 0]], np.int32)
    _say("verify accept clamping")
    _check(w, w.steps, accept=acc)


@pytest.mark.timeout(1200)
def test_verify_full_run_64_steps():
    """The verify workload as configured: 34 Q8_0 layers, B=8 sequences, T=4 tokens, all 64
    verify + commit steps with the seeded accept lengths; every output, the committed state
    every 16 steps, the window roll after every commit."""
    w = synth.WORKLOADS["verify"]
    _say(f"verify full size: 34 layers B=8 T=4 q8_0, all {w.steps} steps")
    e = _check(w, w.steps, snap_every=16)
    _say(f"  worst output error {e:.2e}")


def test_verify_commit_rejects_short_log():
    """A log smaller than a verify of the state's batch and T is refused before anything is
    enqueued (the replay would read past its end)."""
    import torch
    import linear_attention_decode_amd as kda
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=1, batch=2, steps=1, seed=52)
    run = synth.draw_run(w)
    model = gpu_model(run)
    st = model.new_state(2)
    small = model.verify_log(2, 3)
    acc = torch.ones(2, dtype=torch.int32, device="cuda")
    with pytest.raises(kda.KdaError) as ei:
        model.verify_commit(st, small, 4, acc)
    assert ei.value.status == kda._lib.KDA_E_WORKSPACE
    model.close()


def test_verify_commit_graph_replays_equal_eager():
    """Verify and commit captured as hipGraphs and replayed from fixed buffers (inputs and
    accept lengths copied in by the program between replays, with synchronisations) give
    bit for bit what the eager launches give, on every step."""
    import torch
    import linear_attention_decode_amd as kda
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=2, batch=3, steps=4, seed=53)
    run = synth.draw_run(w)
    model = gpu_model(run)
    B, T = w.batch, w.tokens
    _say("verify + commit: graph replays vs eager, 2 layers B=3 T=4, 4 steps")
    outs = {}
    for graph in (True, False):
        model.set_option(kda.KDA_OPT_GRAPH, 1 if graph else 0)
        st = model.new_state(B)
        st.S.copy_(torch.from_numpy(run.s0))
        ws = model.workspace(kda.KDA_OP_VERIFY, B, T)
        log = model.verify_log(B, T)
        xin = torch.empty((B, T, model.d_model), dtype=torch.float32, device="cuda")
        ain = torch.empty((B,), dtype=torch.int32, device="cuda")
        y = torch.empty_like(xin)
        rec = []
        for t in range(w.steps):
            xin.copy_(torch.from_numpy(np.ascontiguousarray(run.x[t])))
            ain.copy_(torch.from_numpy(run.accept[t].copy()))
            model.verify_steps(xin, T, y, st, log, ws)
            model.verify_commit(st, log, T, ain)
            torch.cuda.synchronize()
            rec.append((y.cpu().numpy().copy(), st.S.cpu().numpy().copy(), st.conv.cpu().numpy().copy()))
        outs[graph] = rec
    for (ya, Sa, Za), (yb, Sb, Zb) in zip(outs[True], outs[False]):
        np.testing.assert_array_equal(ya, yb)
        np.testing.assert_array_equal(Sa, Sb)
        np.testing.assert_array_equal(Za, Zb)
    model.close()
