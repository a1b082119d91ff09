"""GPU parity of the forget-gate forms other than KDA's per-channel softplus gate: the
lower-bounded ("safe") gate and the per-head scalar gate of the gated delta rule, through
decode (per-layer kernels), verify + commit and chunked prefill, against the oracle; and
decode's two ways of computing the gates (inside the head kernel for up to 8 sequences, a
gates launch above that) against each other."""
import sys

import numpy as np
import pytest

import synth
from oracle import kda as ok
from tests.helpers import OUT_RTOL, STATE_ATOL, gpu_decode, gpu_model, oracle_layers, range_rel

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _dims(gate, D=256, H=2, dk=64, rank=32):
    return synth.LayerDims(d_model=D, n_heads=H, d_k=dk, d_v=dk, rank_f=rank, rank_g=rank, gate=gate)


def _safe_params(run, seed):
    """The safe gate's per-head factor a (used as given) spread over (0.2, 3)."""
    rng = np.random.default_rng(seed)
    for dr in run.layers:
        dr["a_log"] = rng.uniform(0.2, 3.0, dr["a_log"].shape).astype(np.float32)


@pytest.mark.parametrize("gate", ["safe", "scalar"])
@pytest.mark.parametrize("wtype", ["f32", "bf16", "q8_0"])
def test_gate_forms_decode(gate, wtype):
    """A 2-layer pre-norm stack, B=2, 12 steps; the state every 4 steps."""
    w = synth.scaled(synth.WORKLOADS["tiny"], dims=_dims(gate), wtype=wtype, n_layers=2,
                     prenorm_residual=True, batch=2, steps=12, s0_std=0.1, seed=101)
    _say(f"decode gate={gate} {wtype} 2 layers B=2 12 steps")
    run = synth.draw_run(w)
    if gate == "safe":
        _safe_params(run, 102)
    layers = oracle_layers(run)
    model = gpu_model(run)
    assert model.persistent_blocks() == 0
    y, S, Z, snaps = gpu_decode(model, run, w.steps, 4)
    ry, rS, rZ, rsnaps = ok.decode_run(layers, run.x, run.s0, True, check_every=4)
    e = max(range_rel(y[t], ry[t]) for t in range(w.steps))
    assert e <= OUT_RTOL, e
    assert np.abs(S - rS).max() <= STATE_ATOL
    for k in snaps:
        assert np.abs(snaps[k] - rsnaps[k]).max() <= STATE_ATOL
    assert range_rel(Z, rZ) <= OUT_RTOL
    model.close()
    _say(f"  out {e:.2e}")


@pytest.mark.parametrize("gate,B", [("safe", 1), ("scalar", 1), ("safe", 12), ("scalar", 12)])
def test_gate_forms_full_size_stack(gate, B):
    """D=2048, 16 heads, Q8_0, 3 layers, 6 steps.  The per-layer kernels read the caller's
    row-major weights: B = 1 has the head kernel compute the gates, B = 12 runs the gates
    kernel and takes the matrix-core projections with two 16-row tiles a block.  B = 1 also
    runs the one-launch kernel: the safe gate's formula is one of its two, the scalar gate
    takes its per-head F_b row and dt_bias repeated over the head's channels."""
    d = synth.LayerDims(d_model=2048, n_heads=16, d_k=128, d_v=128, rank_f=128, rank_g=128, gate=gate)
    w = synth.scaled(synth.WORKLOADS["stack"], dims=d, n_layers=3, steps=6, batch=B, seed=103)
    _say(f"decode gate={gate} q8_0 D=2048 3 layers 6 steps B={B}")
    run = synth.draw_run(w)
    if gate == "safe":
        _safe_params(run, 104)
    layers = oracle_layers(run)
    model = gpu_model(run)
    assert model.persistent_blocks() > 0 and not model.owns_weights()
    ry, rS, rZ, _ = ok.decode_run(layers, run.x, run.s0, True)
    for persistent in ((True, False) if B == 1 else (False,)):
        y, S, Z, _ = gpu_decode(model, run, w.steps, persistent=persistent)
        e = max(range_rel(y[t], ry[t]) for t in range(w.steps))
        assert e <= OUT_RTOL, e
        assert np.abs(S - rS).max() <= STATE_ATOL
        _say(f"  {'one launch' if persistent and B == 1 else 'per layer'}: out {e:.2e}")
    model.close()


@pytest.mark.parametrize("gate", ["safe", "scalar"])
def test_gate_forms_verify_commit(gate):
    """Verify + commit (T=3) of a 2-layer Q8_0 stack, B=3, 3 steps."""
    import torch
    w = synth.scaled(synth.WORKLOADS["verify"], dims=_dims(gate, D=256, H=2, dk=64, rank=32),
                     n_layers=2, batch=3, tokens=3, steps=3, seed=105)
    _say(f"verify gate={gate} 2 layers B=3 T=3")
    run = synth.draw_run(w)
    if gate == "safe":
        _safe_params(run, 106)
    layers = oracle_layers(run)
    model = gpu_model(run)
    B, T = w.batch, w.tokens
    st = model.new_state(B)
    st.S.copy_(torch.from_numpy(run.s0))
    ws = model.workspace(1, B, T)
    log = model.verify_log(B, T)
    S = [[run.s0[l, b].astype(np.float64) for b in range(B)] for l in range(2)]
    Z = [[np.zeros((3, w.dims.conv_channels)) for _ in range(B)] for _ in range(2)]
    y = torch.empty((B, T, model.d_model), dtype=torch.float32, device="cuda")
    for t in range(w.steps):
        model.verify_steps(torch.from_numpy(np.ascontiguousarray(run.x[t])).cuda(), T, y, st, log, ws)
        model.verify_commit(st, log, T, torch.from_numpy(run.accept[t].copy()).cuda())
        yy = y.cpu().numpy()
        Sprev = [list(r) for r in S]
        for b in range(B):
            ry, s2, z2 = ok.stack_step(layers, run.x[t, b].astype(np.float64), [S[l][b] for l in range(2)],
                                       [Z[l][b] for l in range(2)], keep_after=int(run.accept[t, b]))
            assert range_rel(yy[b], ry) <= OUT_RTOL
            for l in range(2):
                S[l][b], Z[l][b] = s2[l], z2[l]
        if t == w.steps - 1:
            model.flush(st)
        gS = st.S.cpu().numpy()      # the state after the previous commit until the flush
        ref = S if t == w.steps - 1 else Sprev
        assert np.abs(gS - np.array([[ref[l][b] for b in range(B)] for l in range(2)])).max() <= STATE_ATOL
    model.close()


@pytest.mark.parametrize("gate", ["safe", "scalar"])
def test_gate_forms_prefill(gate):
    """Chunked prefill, BF16, B=2, L=150 (a ragged last chunk), S0 != 0."""
    import torch
    import linear_attention_decode_amd as kda
    w = synth.scaled(synth.WORKLOADS["prefill"], dims=_dims(gate, rank=64), batch=2, tokens=150,
                     s0_std=0.1, seed=107)
    _say(f"prefill gate={gate} D=256 B=2 L=150")
    run = synth.draw_run(w)
    if gate == "safe":
        _safe_params(run, 108)
    layer = oracle_layers(run)[0]
    model = gpu_model(run)
    st = model.new_state(w.batch)
    st.S.copy_(torch.from_numpy(run.s0))
    x = torch.from_numpy(np.ascontiguousarray(run.x_bits[0]).view(np.int16)).cuda()
    y = torch.empty((2, 150, w.dims.d_model), dtype=torch.float32, device="cuda")
    model.prefill_chunked(x, kda.KDA_BF16, 150, 64, y, st, model.workspace(kda.KDA_OP_PREFILL, 2, 150))
    torch.cuda.synchronize()
    ry, rS, rZ = ok.prefill_run(layer, run.x[0], run.s0[0])
    yy = y.cpu().numpy()
    e = max(range_rel(yy[b, t], ry[b, t]) for b in range(2) for t in range(150))
    assert e <= OUT_RTOL, e
    assert np.abs(st.S.cpu().numpy()[0] - rS).max() <= STATE_ATOL
    model.close()


@pytest.mark.parametrize("gate,wtype", [("kda", "bf16"), ("safe", "q8_0"), ("scalar", "f32"),
                                        ("kda", "mxfp4")])
def test_fused_and_separate_gates_agree(gate, wtype):
    """The same 8 sequences decoded as a batch of 8 (gates inside the head kernel) and as
    the first 8 rows of a batch of 9 (gates kernel): outputs and states agree to fp32
    rounding (the two sum each gate row's dot in a different order), 4 steps, 2 layers."""
    import torch
    d = synth.LayerDims(d_model=512, n_heads=4, d_k=128, d_v=128, rank_f=64, rank_g=64, gate=gate)
    w9 = synth.scaled(synth.WORKLOADS["stack"], dims=d, wtype=wtype, n_layers=2, batch=9, steps=4,
                      seed=107)
    _say(f"fused vs separate gates: gate={gate} {wtype} B=8 vs B=9, 2 layers, 4 steps")
    run = synth.draw_run(w9)
    if gate == "safe":
        _safe_params(run, 108)
    model = gpu_model(run)
    model.set_option(2, 0)
    res = {}
    for B in (8, 9):
        st = model.new_state(B)
        st.S.copy_(torch.from_numpy(np.ascontiguousarray(run.s0[:, :B])))
        ws = model.workspace(0, B)
        ys = []
        for t in range(w9.steps):
            x = torch.from_numpy(np.ascontiguousarray(run.x[t, :B, 0, :])).cuda()
            y = torch.empty_like(x)
            model.decode_step(x, y, st, ws)
            ys.append(y.cpu().numpy())
        torch.cuda.synchronize()
        res[B] = (np.array(ys), st.S.cpu().numpy(), st.conv.cpu().numpy())
    y8, S8, Z8 = res[8]
    y9, S9, Z9 = res[9]
    ey = max(range_rel(y8[t], y9[t, :8]) for t in range(w9.steps))
    es = np.abs(S8 - S9[:, :8]).max()
    _say(f"  out {ey:.2e} state {es:.2e}")
    assert ey <= 1e-5, ey
    assert es <= 1e-5, es
    assert range_rel(Z8, Z9[:, :8]) <= 1e-5
    model.close()


def test_matrix_core_gates_in_head_bit_exact():
    """A model with its own gate-tile-order copy computes the gates inside the head kernel on
    the matrix cores for up to 16 decode sequences, and with the separate gates launch above
    that; both take the same arithmetic in the same order, so 16 sequences decoded alone and
    as the first 16 rows of a batch of 17 agree bit for bit (2 layers, 3 steps)."""
    import torch
    w = synth.scaled(synth.WORKLOADS["stack"], n_layers=2, batch=17, steps=3, seed=109)
    _say("matrix-core gates in the head kernel vs the gates launch: B=16 vs B=17, bit for bit")
    run = synth.draw_run(w)
    model = gpu_model(run)
    assert model.owns_weights()
    model.set_option(2, 0)
    res = {}
    for B in (16, 17):
        st = model.new_state(B)
        st.S.copy_(torch.from_numpy(np.ascontiguousarray(run.s0[:, :B])))
        ws = model.workspace(0, B)
        ys = []
        for t in range(w.steps):
            x = torch.from_numpy(np.ascontiguousarray(run.x[t, :B, 0, :])).cuda()
            y = torch.empty_like(x)
            model.decode_step(x, y, st, ws)
            ys.append(y.cpu().numpy())
        torch.cuda.synchronize()
        res[B] = (np.array(ys), st.S.cpu().numpy(), st.conv.cpu().numpy())
    y16, S16, Z16 = res[16]
    y17, S17, Z17 = res[17]
    assert np.array_equal(y16, y17[:, :16])
    assert np.array_equal(S16, S17[:, :16])
    assert np.array_equal(Z16, Z17[:, :16])
    model.close()
