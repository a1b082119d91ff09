"""GPU parity of multi-token verify + commit against the oracle.

Verify runs T tokens per sequence through every layer from the committed state and records
a replay log; commit records the accepted prefix, which the next verify on the state folds
in (replayed inside its own kernels) or kda_state_flush applies.  Compared per step: every
token's output (accepted or not), and the committed state and conv window.
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


def gpu_verify(model, run, steps, accept=None, snap_every=1, fold=True):
    """Verify + commit for `steps` steps.  Returns the outputs of every step and the
    committed (S, window) after every `snap_every`-th step.

    fold=True: each commit is folded into the next verify; the state after commit t is
    read right after verify t + 1 (a verify leaves no commit pending, so st's buffers hold
    the last committed state), the last one after kda_state_flush.  fold=False: every
    commit is applied at once by kda_state_flush and read after it.

    After every commit the window roll is checked bit for bit: with a accepted tokens, rows
    [0, 3 - a) of the new window are rows [a, 3) of the previous one."""
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
    prev = [st.conv.clone()]

    def committed(t):
        # st holds the state after commit t: check the roll, keep a snapshot if due
        for b in range(B):
            a = int(min(max(acc[t, b], 1), T))
            if a < 3:
                assert torch.equal(st.conv[:, b, :3 - a].view(torch.int32),
                                   prev[0][:, b, a:].view(torch.int32)), f"step {t} seq {b}: window roll"
        prev[0] = st.conv.clone()
        if (t + 1) % snap_every == 0 or t == steps - 1:
            states[t] = (st.S.cpu().numpy().copy(), st.conv.cpu().numpy().copy())

    for t in range(steps):
        model.verify_steps(xs[t].contiguous(), T, ys[t], st, log, ws)
        if fold and t > 0:
            committed(t - 1)
        model.verify_commit(st, log, T, accs[t].contiguous())
        if not fold:
            model.flush(st)
            committed(t)
    if fold:
        model.flush(st)
        committed(steps - 1)
    torch.cuda.synchronize()
    return ys.cpu().numpy(), states


def _check(w, steps, accept=None, snap_every=1, fold=True):
    run = synth.draw_run(w)
    layers = oracle_layers(run)
    model = gpu_model(run)
    acc = run.accept if accept is None else accept
    y, states = gpu_verify(model, run, steps, acc, snap_every, fold)
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


@pytest.mark.parametrize("fold", [True, False])
def test_verify_small_stack(fold):
    """Commits folded into the next verify, or applied at once by kda_state_flush."""
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=2, batch=3, steps=4, seed=31)
    _say(f"verify 2 layers B=3 T=4 D=2048 q8_0, 4 steps, fold={fold}")
    _check(w, w.steps, fold=fold)


def test_verify_ragged_columns_matrix_cores():
    """B=5 x T=3 = 15 token positions at D=2048: MFMA projections with a padded column tile."""
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=2, batch=5, tokens=3, steps=3, seed=35)
    _say("verify 2 layers B=5 T=3 D=2048 q8_0, 3 steps (MFMA projections)")
    _check(w, w.steps)


def test_verify_bf16_matrix_cores():
    """A BF16 stack: B=3 x T=4 = 12 token positions at D=2048 on the BF16 MFMA products."""
    w = synth.scaled(synth.WORKLOADS["verify"], wtype="bf16", n_layers=2, batch=3, steps=3, seed=37)
    _say("verify 2 layers B=3 T=4 D=2048 bf16, 3 steps (MFMA projections)")
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


@pytest.mark.parametrize("fold", [True, False])
def test_verify_accept_clamped(fold):
    """Accept lengths outside 1..T are clamped: 0 commits one token, 9 commits T."""
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=1, batch=2, steps=3, seed=50)
    acc = np.array([[0, 9], [9, 0], [0, 9]], np.int32)
    _say(f"verify accept clamping, fold={fold}")
    _check(w, w.steps, accept=acc, fold=fold)


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
    bit for bit what the eager launches give, on every step: the outputs, and the state
    each verify leaves (the previous step's commit folded in); the last commit flushed.
    Consecutive verifies alternate between the log's halves (two captured graphs)."""
    import torch
    import linear_attention_decode_amd as kda
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=2, batch=3, steps=5, seed=53)
    run = synth.draw_run(w)
    model = gpu_model(run)
    B, T = w.batch, w.tokens
    _say("verify + commit: graph replays vs eager, 2 layers B=3 T=4, 5 steps")
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
            model.verify_steps(xin, T, y, st, log, ws)
            torch.cuda.synchronize()
            rec.append((y.cpu().numpy().copy(), st.S.cpu().numpy().copy(), st.conv.cpu().numpy().copy()))
            ain.copy_(torch.from_numpy(run.accept[t].copy()))
            model.verify_commit(st, log, T, ain)
        model.flush(st)
        torch.cuda.synchronize()
        rec.append((None, st.S.cpu().numpy().copy(), st.conv.cpu().numpy().copy()))
        outs[graph] = rec
    for (ya, Sa, Za), (yb, Sb, Zb) in zip(outs[True], outs[False]):
        if ya is not None:
            np.testing.assert_array_equal(ya, yb)
        np.testing.assert_array_equal(Sa, Sb)
        np.testing.assert_array_equal(Za, Zb)
    model.close()


def test_verify_fold_equals_flush_bit_exact():
    """A commit folded into the next verify (replayed inside its head and projection
    kernels) and the same commit applied by kda_state_flush before it give the same bits:
    every output, and every committed state and window."""
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=2, batch=3, steps=4, seed=54)
    run = synth.draw_run(w)
    _say("verify fold vs flush, bit for bit, 2 layers B=3 T=4, 4 steps")
    res = {}
    for fold in (True, False):
        model = gpu_model(run)
        res[fold] = gpu_verify(model, run, w.steps, run.accept, 1, fold)
        model.close()
    np.testing.assert_array_equal(res[True][0], res[False][0])
    assert sorted(res[True][1]) == sorted(res[False][1])
    for t in res[True][1]:
        np.testing.assert_array_equal(res[True][1][t][0], res[False][1][t][0])
        np.testing.assert_array_equal(res[True][1][t][1], res[False][1][t][1])


def _oracle_state(layers, run, w, S, Z, t, acc):
    """Advance the oracle's per-sequence (S, Z) lists by verify step t with accept acc[b]."""
    ys = np.empty(run.x.shape[2:])
    out = []
    for b in range(w.batch):
        yb, s_new, z_new = ok.stack_step(layers, run.x[t, b].astype(np.float64),
                                         [S[l][b] for l in range(w.n_layers)],
                                         [Z[l][b] for l in range(w.n_layers)],
                                         keep_after=int(acc[b]))
        out.append(yb)
        for l in range(w.n_layers):
            S[l][b], Z[l][b] = s_new[l], z_new[l]
    return np.array(out)


def test_pending_commit_applied_by_other_calls():
    """A recorded commit is applied by whatever touches the state next: a decode step, a
    verify with a different T (a log sized for 4 serves 2), a verify through a second log,
    and the canonical window read.  Each result against the oracle."""
    import torch
    import linear_attention_decode_amd as kda
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=2, batch=2, tokens=4, steps=5, seed=55)
    run = synth.draw_run(w)
    layers = oracle_layers(run)
    model = gpu_model(run)
    B, T = w.batch, w.tokens
    _say("pending commit applied by decode / verify T=2 / second log / window read")
    st = model.new_state(B)
    st.S.copy_(torch.from_numpy(run.s0))
    S = [[np.array(run.s0[l, b], np.float64) for b in range(B)] for l in range(w.n_layers)]
    Z = [[np.zeros((3, w.dims.conv_channels)) for _ in range(B)] for _ in range(w.n_layers)]
    logA = model.verify_log(B, T)
    logB = model.verify_log(B, T)
    wsv = model.workspace(kda.KDA_OP_VERIFY, B, T)
    acc = torch.tensor([3, 1], dtype=torch.int32, device="cuda")

    def verify(t, log, Tt, a):
        x = torch.from_numpy(np.ascontiguousarray(run.x[t][:, :Tt])).cuda()
        y = torch.empty_like(x)
        model.verify_steps(x, Tt, y, st, log, wsv)
        ry = _oracle_state(layers, _sub(run, Tt), w, S, Z, t, a)
        assert range_rel(y.cpu().numpy(), ry) <= OUT_RTOL

    def check_state(what):
        model.flush(st)
        torch.cuda.synchronize()
        rS = np.array([[S[l][b] for b in range(B)] for l in range(w.n_layers)])
        rZ = np.array([[Z[l][b] for b in range(B)] for l in range(w.n_layers)])
        assert np.abs(st.S.cpu().numpy() - rS).max() <= STATE_ATOL, what
        assert range_rel(st.conv.cpu().numpy(), rZ) <= OUT_RTOL, what

    # verify (T=4) + commit 3 / 1, then a decode step applies it
    verify(0, logA, T, [3, 1])
    model.verify_commit(st, logA, T, acc)
    x = torch.from_numpy(np.ascontiguousarray(run.x[1][:, 0])).cuda()
    y = torch.empty_like(x)
    model.decode_step(x, y, st, model.workspace(kda.KDA_OP_DECODE, B, 1))
    ry = _oracle_state(layers, _sub(run, 1), w, S, Z, 1, [1, 1])
    assert range_rel(y.cpu().numpy(), ry[:, 0]) <= OUT_RTOL
    check_state("after decode")
    # verify T=4 + commit, then verify T=2 on the same log folds it in; commit 2 / 1
    verify(2, logA, T, [3, 1])
    model.verify_commit(st, logA, T, acc)
    verify(3, logA, 2, [2, 1])
    model.verify_commit(st, logA, 2, torch.tensor([2, 1], dtype=torch.int32, device="cuda"))
    # a verify through the second log applies the first log's commit before it runs
    verify(4, logB, T, [1, 3])
    model.verify_commit(st, logB, T, torch.tensor([1, 3], dtype=torch.int32, device="cuda"))
    # the canonical window read applies the pending commit
    z = model.conv_window(st)
    torch.cuda.synchronize()
    rZ = np.array([[Z[l][b] for b in range(B)] for l in range(w.n_layers)])
    assert range_rel(z.cpu().numpy(), rZ) <= OUT_RTOL
    check_state("after the second log")
    model.close()


def _sub(run, Tt):
    """The run with each step's tokens cut to the first Tt (for the oracle helper)."""
    return synth.RunInputs(run.workload, run.layers, run.s0,
                           np.ascontiguousarray(run.x[:, :, :Tt]), run.x_bits, run.accept)


def test_commit_misuse_refused():
    """A commit with no verify to commit, a second commit of one verify, a commit of a
    verify retired by a decode step, and a commit with another T are refused (KDA_E_ARG)
    before anything is enqueued; the state is unchanged by each."""
    import torch
    import linear_attention_decode_amd as kda
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=1, batch=2, steps=2, seed=56)
    run = synth.draw_run(w)
    model = gpu_model(run)
    B, T = w.batch, w.tokens
    _say("commit misuse: none, twice, retired, other T")
    st = model.new_state(B)
    st.S.copy_(torch.from_numpy(run.s0))
    log = model.verify_log(B, T)
    ws = model.workspace(kda.KDA_OP_VERIFY, B, T)
    acc = torch.full((B,), 2, dtype=torch.int32, device="cuda")

    def refused(Tc=T):
        with pytest.raises(kda.KdaError) as ei:
            model.verify_commit(st, log, Tc, acc)
        assert ei.value.status == kda._lib.KDA_E_ARG

    refused()
    x = torch.from_numpy(np.ascontiguousarray(run.x[0])).cuda()
    y = torch.empty_like(x)
    model.verify_steps(x, T, y, st, log, ws)
    refused(T - 1)
    model.verify_commit(st, log, T, acc)
    refused()
    model.flush(st)
    model.verify_steps(x, T, y, st, log, ws)
    S0 = st.S.clone()
    model.decode_step(x[:, 0].contiguous(), y[:, 0].contiguous(), st,
                      model.workspace(kda.KDA_OP_DECODE, B, 1))
    S1 = st.S.clone()
    refused()
    model.flush(st)
    assert torch.equal(st.S, S1) and not torch.equal(S0, S1)
    model.close()


def test_two_states_sharing_one_log():
    """Two independent states verified through one log in turn: the second state's verify
    applies the commit the first one left pending in that log before overwriting it, so
    both committed states match the oracle."""
    import torch
    import linear_attention_decode_amd as kda
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=2, batch=2, steps=2, seed=57)
    run = synth.draw_run(w)
    layers = oracle_layers(run)
    model = gpu_model(run)
    B, T = w.batch, w.tokens
    _say("two states, one log")
    log = model.verify_log(B, T)
    ws = model.workspace(kda.KDA_OP_VERIFY, B, T)
    sts, refs = [], []
    for i in range(2):
        st = model.new_state(B)
        st.S.copy_(torch.from_numpy(run.s0))
        sts.append(st)
        refs.append(([[np.array(run.s0[l, b], np.float64) for b in range(B)] for l in range(2)],
                     [[np.zeros((3, w.dims.conv_channels)) for _ in range(B)] for _ in range(2)]))
    for t in range(w.steps):
        for i in range(2):
            x = torch.from_numpy(np.ascontiguousarray(run.x[t] * (1.0 + 0.5 * i))).float().cuda()
            y = torch.empty_like(x)
            model.verify_steps(x, T, y, sts[i], log, ws)
            acc = run.accept[t] if i == 0 else run.accept[t][::-1].copy()
            model.verify_commit(sts[i], log, T, torch.from_numpy(acc.astype(np.int32)).cuda())
            S, Z = refs[i]
            yy = y.cpu().numpy()
            for b in range(B):
                ry, s2, z2 = ok.stack_step(layers, (run.x[t, b] * (1.0 + 0.5 * i)).astype(np.float64),
                                           [S[l][b] for l in range(2)], [Z[l][b] for l in range(2)],
                                           keep_after=int(acc[b]))
                assert range_rel(yy[b], ry) <= OUT_RTOL, f"step {t} state {i} seq {b}"
                for l in range(2):
                    S[l][b], Z[l][b] = s2[l], z2[l]
    for i in range(2):
        model.flush(sts[i])
        torch.cuda.synchronize()
        S, Z = refs[i]
        rS = np.array([[S[l][b] for b in range(B)] for l in range(2)])
        rZ = np.array([[Z[l][b] for b in range(B)] for l in range(2)])
        assert np.abs(sts[i].S.cpu().numpy() - rS).max() <= STATE_ATOL, f"state {i}"
        assert range_rel(sts[i].conv.cpu().numpy(), rZ) <= OUT_RTOL
    model.close()
