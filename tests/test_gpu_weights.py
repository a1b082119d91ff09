"""A model that owns its weights: for a stack eligible for the one-launch decode,
kda_model_create copies every packed matrix into its matrix-core order and every kernel
reads only that copy.  Here the caller's packed buffers are overwritten with garbage right
after the model is made; every call shape (one-launch decode, batched per-layer decode
below and above 64 columns, masked decode, verify + commit, sequential-scan prefill) must
still match the oracle, which it would not if any kernel read a caller buffer."""
import sys

import numpy as np
import pytest

import synth
from oracle import kda as ok
from tests.helpers import OUT_RTOL, STATE_ATOL, gpu_decode, gpu_model, oracle_layers, range_rel

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _dims(D, rank):
    return synth.LayerDims(d_model=D, n_heads=D // 128, d_k=128, d_v=128, rank_f=rank, rank_g=rank)


def _owned_model(run):
    import torch
    model = gpu_model(run)
    assert model.persistent_blocks() > 0 and model.owns_weights()
    for buf in model._packed.values():
        buf.fill_(0xA5)                   # any read of a caller buffer now gives garbage
    torch.cuda.synchronize()
    return model


def _check_decode(run, y, S, Z, steps):
    ry, rS, rZ, _ = ok.decode_run(oracle_layers(run), run.x, run.s0, True, steps=steps)
    e = max(range_rel(y[t], ry[t]) for t in range(steps))
    assert e <= OUT_RTOL, f"output error {e:.3e}"
    assert np.abs(S - rS).max() <= STATE_ATOL
    assert range_rel(Z, rZ) <= OUT_RTOL


@pytest.mark.parametrize("D,rank,B", [(1024, 32, 1), (1024, 32, 3), (2048, 128, 5), (1024, 32, 70)])
def test_owned_copy_decode(D, rank, B):
    """B = 1 runs the one-launch kernel and (persistent path off) the per-layer kernels;
    B = 3, 5 the per-layer kernels on the copy; B = 70 the products in two launches of at
    most 64 columns."""
    w = synth.scaled(synth.WORKLOADS["stack"], dims=_dims(D, rank), n_layers=2, batch=B, steps=3,
                     seed=170 + B)
    _say(f"owned copy: decode D={D} rank={rank} B={B}, caller buffers overwritten")
    run = synth.draw_run(w)
    model = _owned_model(run)
    for persistent in ((True, False) if B == 1 else (False,)):
        y, S, Z, _ = gpu_decode(model, run, w.steps, persistent=persistent)
        _check_decode(run, y, S, Z, w.steps)
    assert model.release_packed()
    y, S, Z, _ = gpu_decode(model, run, w.steps, persistent=False)
    _check_decode(run, y, S, Z, w.steps)
    model.close()


def test_owned_copy_masked_verify_scan():
    """Masked decode (B = 2, one row masked), verify + commit (B = 3, T = 4, 12 columns) with
    the commit flushed, then a 10-token scan prefill, on a model whose caller buffers hold
    garbage."""
    import torch
    import linear_attention_decode_amd as kda
    w = synth.scaled(synth.WORKLOADS["verify"], dims=_dims(1024, 32), n_layers=2, batch=3,
                     steps=2, seed=175)
    _say("owned copy: masked decode, verify + commit, scan prefill")
    run = synth.draw_run(w)
    layers = oracle_layers(run)
    model = _owned_model(run)
    B, T = w.batch, w.tokens
    st = model.new_state(B)
    st.S.copy_(torch.from_numpy(run.s0))
    S = [[run.s0[l, b].astype(np.float64) for b in range(B)] for l in range(2)]
    Z = [[np.zeros((3, w.dims.conv_channels)) for _ in range(B)] for _ in range(2)]
    # masked decode: sequence 1 takes no token
    x = torch.from_numpy(np.ascontiguousarray(run.x[0][:, 0])).cuda()
    y = torch.empty_like(x)
    active = torch.tensor([1, 0, 1], dtype=torch.int32, device="cuda")
    model.decode_step_masked(x, y, st, active, model.workspace(kda.KDA_OP_DECODE, B))
    yy = y.cpu().numpy()
    for b in (0, 2):
        ry, s2, z2 = ok.stack_step(layers, run.x[0, b, 0].astype(np.float64)[None, :],
                                   [S[l][b] for l in range(2)], [Z[l][b] for l in range(2)])
        assert range_rel(yy[b], ry[0]) <= OUT_RTOL
        for l in range(2):
            S[l][b], Z[l][b] = s2[l], z2[l]
    # verify + commit, flushed
    ws = model.workspace(kda.KDA_OP_VERIFY, B, T)
    log = model.verify_log(B, T)
    xv = torch.from_numpy(np.ascontiguousarray(run.x[1])).cuda()
    yv = torch.empty_like(xv)
    model.verify_steps(xv, T, yv, st, log, ws)
    model.verify_commit(st, log, T, torch.from_numpy(run.accept[1].copy()).cuda())
    model.flush(st)
    yy = yv.cpu().numpy()
    for b in range(B):
        ry, s2, z2 = ok.stack_step(layers, run.x[1, b].astype(np.float64), [S[l][b] for l in range(2)],
                                   [Z[l][b] for l in range(2)], keep_after=int(run.accept[1, b]))
        assert range_rel(yy[b], ry) <= OUT_RTOL
        for l in range(2):
            S[l][b], Z[l][b] = s2[l], z2[l]
    # scan prefill of 10 tokens from there
    xs = np.random.default_rng(176).standard_normal((B, 10, w.dims.d_model)).astype(np.float32)
    ys = torch.empty((B, 10, w.dims.d_model), dtype=torch.float32, device="cuda")
    model.prefill_scan(torch.from_numpy(xs).cuda(), 10, ys, st, model.workspace(kda.KDA_OP_SCAN, B, 10))
    yy = ys.cpu().numpy()
    for b in range(B):
        for t in range(10):
            ry, s2, z2 = ok.stack_step(layers, xs[b, t].astype(np.float64)[None, :],
                                       [S[l][b] for l in range(2)], [Z[l][b] for l in range(2)])
            assert range_rel(yy[b, t], ry[0]) <= OUT_RTOL, f"scan seq {b} token {t}"
            for l in range(2):
                S[l][b], Z[l][b] = s2[l], z2[l]
    rS = np.array([[S[l][b] for b in range(B)] for l in range(2)])
    assert np.abs(st.S.cpu().numpy() - rS).max() <= STATE_ATOL
    model.close()


def test_caller_buffers_read_without_copy():
    """A model that is not one-launch eligible (a single BF16 layer) owns no copy and says
    so; releasing its packed buffers is refused by the binding."""
    w = synth.scaled(synth.WORKLOADS["layer"], steps=1)
    run = synth.draw_run(w)
    model = gpu_model(run)
    assert not model.owns_weights() and not model.release_packed()
    model.close()
