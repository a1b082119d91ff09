"""GPU parity of the chunked (WY/UT) prefill against the sequential token-by-token oracle.

The GPU runs the projections as BF16 GEMMs on matrix cores, the delta rule in 64-token
chunks with an fp32 state carried across chunks; the oracle runs the recurrence one token
at a time in float64.  Compared: every output token, the final state and the conv window.
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


SMALL = synth.LayerDims(d_model=256, n_heads=2, d_k=64, d_v=64, rank_f=64, rank_g=64)


def _small(L, B=2, seed=60, s0_std=0.1):
    return synth.scaled(synth.WORKLOADS["prefill"], dims=SMALL, batch=B, tokens=L, s0_std=s0_std,
                        seed=seed)


def gpu_prefill(model, x_f32, x_bits, st, use_f32=False):
    import torch
    import linear_attention_decode_amd as kda
    B, L, D = x_f32.shape
    if use_f32:
        x = torch.from_numpy(np.ascontiguousarray(x_f32)).cuda()
        dt = kda.KDA_F32
    else:
        x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()
        dt = kda.KDA_BF16
    y = torch.empty((B, L, D), dtype=torch.float32, device="cuda")
    ws = model.workspace(kda.KDA_OP_PREFILL, B, L)
    model.prefill_chunked(x, dt, L, 64, y, st, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _compare(y, ry, S, rS, Z, rZ):
    errs = [range_rel(y[b, t], ry[b, t]) for b in range(y.shape[0]) for t in range(y.shape[1])]
    e = max(errs)
    assert e <= OUT_RTOL, f"output range-rel error {e:.3e}"
    serr = np.abs(S - rS).max()
    assert serr <= STATE_ATOL, f"state error {serr:.3e}"
    zerr = range_rel(Z, rZ)
    assert zerr <= OUT_RTOL, f"window error {zerr:.3e}"
    return e, serr


@pytest.mark.parametrize("L", [1, 2, 3, 5, 64, 150])
def test_prefill_small(L):
    import torch
    w = _small(L)
    _say(f"prefill small D=256 H=2 dk=64 B=2 L={L}")
    run = synth.draw_run(w)
    layer = oracle_layers(run)[0]
    model = gpu_model(run)
    st = model.new_state(w.batch)
    st.S.copy_(torch.from_numpy(run.s0))
    y = gpu_prefill(model, run.x[0], run.x_bits[0], st)
    ry, rS, rZ = ok.prefill_run(layer, run.x[0], run.s0[0])
    _compare(y, ry, st.S.cpu().numpy()[0], rS, st.conv.cpu().numpy()[0], rZ)
    model.close()


def test_prefill_continuation_and_f32_input():
    """Two prefill calls (130 then 77 tokens) from S0 != 0: the second starts from the
    state and window the first left; F32 inputs take the split-BF16 GEMM path."""
    import torch
    w = _small(207, seed=61)
    _say("prefill continuation 130 + 77 tokens, f32 input")
    run = synth.draw_run(w)
    rng = np.random.default_rng(5)
    x32 = rng.standard_normal(run.x[0].shape).astype(np.float32)    # not BF16-representable
    layer = oracle_layers(run)[0]
    model = gpu_model(run)
    st = model.new_state(w.batch)
    st.S.copy_(torch.from_numpy(run.s0))
    y1 = gpu_prefill(model, x32[:, :130], None, st, use_f32=True)
    y2 = gpu_prefill(model, np.ascontiguousarray(x32[:, 130:]), None, st, use_f32=True)
    y = np.concatenate([y1, y2], axis=1)
    ry, rS, rZ = ok.prefill_run(layer, x32, run.s0[0])
    _compare(y, ry, st.S.cpu().numpy()[0], rS, st.conv.cpu().numpy()[0], rZ)
    model.close()


def test_prefill_matches_decode_on_gpu():
    """Chunked prefill and token-by-token decode of the same tokens agree."""
    import torch
    from tests.helpers import gpu_decode
    w = _small(70, B=1, seed=62)
    _say("prefill vs decode, 70 tokens")
    run = synth.draw_run(w)
    model = gpu_model(run)
    st = model.new_state(1)
    st.S.copy_(torch.from_numpy(run.s0))
    y = gpu_prefill(model, run.x[0], run.x_bits[0], st)
    dec_run = synth.RunInputs(synth.scaled(w, steps=70, tokens=1), run.layers, run.s0,
                              run.x[0].transpose(1, 0, 2)[:, :, None, :].copy(), None, None)
    yd, Sd, Zd, _ = gpu_decode(model, dec_run, 70)
    assert max(range_rel(y[0, t], yd[t, 0]) for t in range(70)) <= OUT_RTOL
    assert np.abs(st.S.cpu().numpy() - Sd).max() <= STATE_ATOL
    model.close()


def test_prefill_full_size():
    """B=4 sequences of 8192 tokens, D=2048, 16 heads, BF16 weights, chunk 64, S0 = 0."""
    import torch
    w = synth.WORKLOADS["prefill"]
    _say("prefill full size B=4 L=8192 D=2048 H=16")
    run = synth.draw_run(w)
    layer = oracle_layers(run)[0]
    model = gpu_model(run)
    st = model.new_state(w.batch)
    y = gpu_prefill(model, run.x[0], run.x_bits[0], st)
    S = st.S.cpu().numpy()[0]
    Z = st.conv.cpu().numpy()[0]
    for b in range(w.batch):
        ry, rS, rZ = ok.prefill_run(layer, run.x[0], run.s0[0], seqs=[b])
        e, se = _compare(y[b:b + 1], ry, S[b:b + 1], rS, Z[b:b + 1], rZ)
        _say(f"  seq {b}: out {e:.2e} state {se:.2e}")
    model.close()


def test_prefill_strong_decay_blocks():
    """Forget gates strong enough that a 16-token block's decay range passes 2^64 on some
    channels (head 0: those diagonal blocks take the pairwise path) next to a head whose
    blocks are factored with decay factors up to ~2^50 (head 1); 150 tokens (ragged)."""
    import torch
    w = _small(150, seed=63)
    _say("prefill strong decay, 150 tokens, a_log = [3.0, 0.5]")
    run = synth.draw_run(w)
    run.layers[0]["a_log"] = np.array([3.0, 0.5], np.float32)
    layer = oracle_layers(run)[0]
    model = gpu_model(run)
    st = model.new_state(w.batch)
    st.S.copy_(torch.from_numpy(run.s0))
    y = gpu_prefill(model, run.x[0], run.x_bits[0], st)
    ry, rS, rZ = ok.prefill_run(layer, run.x[0], run.s0[0])
    _compare(y, ry, st.S.cpu().numpy()[0], rS, st.conv.cpu().numpy()[0], rZ)
    model.close()


def _slow_gates(run, seed):
    """Per-channel decay rates from nearly 1 to fast: A_log per head in U(-6, -1), dt_bias
    per key channel in U(-6, 2), so many channels keep alpha > 0.999 per token and carry
    the state across chunk boundaries (a slow channel stays slow on every token)."""
    rng = np.random.default_rng(seed)
    for dr in run.layers:
        dr["a_log"] = rng.uniform(-6.0, -1.0, dr["a_log"].shape).astype(np.float32)
        dr["dt_bias"] = rng.uniform(-6.0, 2.0, dr["dt_bias"].shape).astype(np.float32)


@pytest.mark.parametrize("dims", ["small", "full"])
def test_prefill_slow_gates_carry_state(dims):
    """Slow per-channel gates, S0 != 0, 200 tokens (four chunks, a ragged last one): the
    state carried across each chunk end (each key row decayed by its own channel's
    end-of-chunk factor) dominates the outputs and the final state."""
    import torch
    if dims == "small":
        w = _small(200, seed=64)
    else:
        w = synth.scaled(synth.WORKLOADS["prefill"], batch=1, tokens=200, s0_std=0.1, seed=65)
    _say(f"prefill slow gates {dims} D={w.dims.d_model} L=200, S0 != 0")
    run = synth.draw_run(w)
    _slow_gates(run, 66)
    layer = oracle_layers(run)[0]
    # a quarter of the channels keep more than half their state across a 64-token chunk
    # from the bias alone (the low-rank term is small)
    slow = np.exp(-np.exp(layer.a_log)[:, None] * ok.softplus(layer.dt_bias.reshape(len(layer.a_log), -1)))
    assert (slow ** 64 > 0.5).mean() > 0.25
    model = gpu_model(run)
    st = model.new_state(w.batch)
    st.S.copy_(torch.from_numpy(run.s0))
    y = gpu_prefill(model, run.x[0], run.x_bits[0], st)
    ry, rS, rZ = ok.prefill_run(layer, run.x[0], run.s0[0])
    e, se = _compare(y, ry, st.S.cpu().numpy()[0], rS, st.conv.cpu().numpy()[0], rZ)
    _say(f"  out {e:.2e} state {se:.2e}")
    model.close()


def test_prefill_window_roll_bit_exact():
    """The window a prefill leaves holds the last three pre-conv projections, oldest first:
    prefills of 200 and 201 tokens of the same sequence leave windows shifted by one row,
    bit for bit (a token's projection does not depend on the call's length); prefills of 1
    and 2 tokens from a random window keep its newest rows, bit for bit."""
    import torch
    w = _small(201, B=2, seed=67)
    run = synth.draw_run(w)
    model = gpu_model(run)
    _say("prefill window roll: L=200 vs 201, and L=1, 2 from a random window")
    wins = {}
    for L in (200, 201):
        st = model.new_state(w.batch)
        st.S.copy_(torch.from_numpy(run.s0))
        gpu_prefill(model, np.ascontiguousarray(run.x[0][:, :L]), np.ascontiguousarray(run.x_bits[0][:, :L]), st)
        wins[L] = st.conv.cpu().numpy()[0].copy()
    np.testing.assert_array_equal(wins[201][:, :2].view(np.uint32), wins[200][:, 1:].view(np.uint32))
    rng = np.random.default_rng(68)
    z0 = rng.standard_normal((1, w.batch, 3, w.dims.conv_channels)).astype(np.float32)
    for L in (1, 2):
        st = model.new_state(w.batch)
        st.S.copy_(torch.from_numpy(run.s0))
        st.conv.copy_(torch.from_numpy(z0))
        gpu_prefill(model, np.ascontiguousarray(run.x[0][:, :L]), np.ascontiguousarray(run.x_bits[0][:, :L]), st)
        z = st.conv.cpu().numpy()[0]
        np.testing.assert_array_equal(z[:, :3 - L].view(np.uint32), z0[0][:, L:].view(np.uint32))
    model.close()
