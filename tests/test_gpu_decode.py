"""GPU parity of the decode path (pack, one layer, the 34-layer stack) against the oracle.

Every case prints its name before running so a fault names it.  Tolerances are stated in
tests/helpers.py (range-relative 1e-3 on outputs, 2e-3 absolute on the state); packing
and conv-window indexing are compared bit for bit.
"""
import sys

import numpy as np
import pytest

import synth
from oracle import kda as ok
from tests.helpers import OUT_RTOL, STATE_ATOL, gpu_decode, gpu_model, oracle_layers, range_rel

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


# ----------------------------------------------------------------------------------------
# packing: bit-exact against the oracle's quantiser / rounding
# ----------------------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 32), (7, 96), (64, 2048), (2048, 128), (13, 4096)])
def test_pack_q8_0_bit_exact(torch, shape):
    import linear_attention_decode_amd as kda
    _say(f"pack q8_0 {shape}")
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    w[0, :32] = 0.0                                    # an all-zero block
    if shape[1] >= 64:
        w[-1, 32:64] *= 1e4                            # a large-scale block
        w[-1, 33] = 0.5 * float(np.float32(w[-1, 32:64].__abs__().max()))
    src = torch.from_numpy(w).cuda()
    nb = kda.kda_packed_bytes(kda.KDA_Q8_0, *shape)
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    kda.kda_pack_device(kda.KDA_Q8_0, src, buf)
    d16, qs = kda.kda_unpack_q8_0_device(buf, *shape)
    torch.cuda.synchronize()
    rd16, rq = ok.q8_0_quantize(w)
    np.testing.assert_array_equal(d16.cpu().numpy().view(np.uint16), rd16.view(np.uint16))
    np.testing.assert_array_equal(qs.cpu().numpy(), rq)
    # the host-source pack and the host-side canonical view: the same bytes
    buf2 = torch.empty(nb, dtype=torch.uint8, device="cuda")
    kda.kda_pack(kda.KDA_Q8_0, w, buf2)
    hd16, hqs = kda.kda_unpack_q8_0(buf2, *shape)
    np.testing.assert_array_equal(hd16, rd16.view(np.uint16))
    np.testing.assert_array_equal(hqs, rq)
    # the two byte planes (the padding between them is not written by the device kernel)
    n, so = shape[0] * shape[1], -(-shape[0] * shape[1] // 256) * 256
    a, b = buf2.cpu().numpy(), buf.cpu().numpy()
    np.testing.assert_array_equal(a[:n], b[:n])
    np.testing.assert_array_equal(a[so:so + n // 16], b[so:so + n // 16])


def test_pack_q8_0_ties_bit_exact(torch):
    import linear_attention_decode_amd as kda
    _say("pack q8_0 ties")
    x = np.zeros((2, 32), np.float32)
    x[0, :8] = [127, 2.5, -2.5, 0.5, -0.5, 3.5, -3.5, 1.5]
    x[0, 31] = -126.5
    x[1] = np.arange(32) / 31.0
    rd16, rq = ok.q8_0_quantize(x)
    for host in (False, True):
        buf = torch.empty(kda.kda_packed_bytes(kda.KDA_Q8_0, 2, 32), dtype=torch.uint8, device="cuda")
        if host:
            kda.kda_pack(kda.KDA_Q8_0, x, buf)
        else:
            kda.kda_pack_device(kda.KDA_Q8_0, torch.from_numpy(x).cuda(), buf)
        d16, qs = kda.kda_unpack_q8_0(buf, 2, 32)
        np.testing.assert_array_equal(d16, rd16.view(np.uint16))
        np.testing.assert_array_equal(qs, rq)


@pytest.mark.parametrize("shape", [(3, 5), (128, 2048)])
def test_pack_bf16_bit_exact(torch, shape):
    import linear_attention_decode_amd as kda
    _say(f"pack bf16 {shape}")
    rng = np.random.default_rng(5)
    w = (rng.standard_normal(shape) * rng.uniform(1e-3, 1e3, shape)).astype(np.float32)
    for host in (False, True):
        buf = torch.empty(kda.kda_packed_bytes(kda.KDA_BF16, *shape), dtype=torch.uint8, device="cuda")
        if host:
            kda.kda_pack(kda.KDA_BF16, w, buf)
        else:
            kda.kda_pack_device(kda.KDA_BF16, torch.from_numpy(w).cuda(), buf)
        bits = buf.cpu().numpy().view(np.uint16).reshape(shape)
        got = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        np.testing.assert_array_equal(got, ok.bf16_round(w))


# ----------------------------------------------------------------------------------------
# decode parity
# ----------------------------------------------------------------------------------------
def _decode_parity(w, steps, snap_every=0, graph=True, persistent=True, expect_persistent=None):
    run = synth.draw_run(w)
    layers = oracle_layers(run)
    model = gpu_model(run)
    if expect_persistent is not None:
        assert (model.persistent_blocks() > 0) == expect_persistent
    y, S, Z, snaps = gpu_decode(model, run, steps, snap_every, graph, persistent)
    ry, rS, rZ, rsnaps = ok.decode_run(layers, run.x, run.s0, w.prenorm_residual, steps=steps,
                                       check_every=snap_every)
    errs = [range_rel(y[t], ry[t]) for t in range(steps)]
    assert max(errs) <= OUT_RTOL, f"output range-rel error {max(errs):.3e} at step {int(np.argmax(errs))}"
    serr = np.abs(S - rS).max()
    assert serr <= STATE_ATOL, f"state error {serr:.3e}"
    for k, v in snaps.items():
        assert np.abs(v - rsnaps[k]).max() <= STATE_ATOL, f"state error at step {k}"
    assert range_rel(Z, rZ) <= OUT_RTOL
    model.close()
    return max(errs), serr


def test_decode_tiny_layer(torch):
    w = synth.WORKLOADS["tiny"]
    _say(f"decode tiny D={w.dims.d_model} H={w.dims.n_heads} dk={w.dims.d_k} steps={w.steps}")
    e, s = _decode_parity(w, w.steps)
    _say(f"  tiny: out {e:.2e} state {s:.2e}")


def test_decode_layer_bf16_256_steps(torch):
    w = synth.WORKLOADS["layer"]
    _say(f"decode layer bf16 D=2048 H=16 steps={w.steps}")
    e, s = _decode_parity(w, w.steps, snap_every=32)
    _say(f"  layer: out {e:.2e} state {s:.2e}")


@pytest.mark.parametrize("wtype", ["f32", "bf16", "q8_0"])
def test_decode_ragged_batch(torch, wtype):
    """B=3 sequences, H=3 heads (row tiles end mid-block), a 2-layer residual stack."""
    d = synth.LayerDims(d_model=96, n_heads=3, d_k=64, d_v=64, rank_f=32, rank_g=32)
    base = synth.WORKLOADS["tiny"]
    w = synth.scaled(base, dims=d, wtype=wtype, n_layers=2, prenorm_residual=True, batch=3,
                     steps=6, s0_std=0.1, seed=21)
    _say(f"decode ragged {wtype} B=3 H=3 L=2")
    _decode_parity(w, w.steps, snap_every=3)


@pytest.mark.parametrize("persistent", [True, False], ids=["one-launch", "per-layer"])
def test_decode_stack_q8_0_full_size(torch, persistent):
    w = synth.scaled(synth.WORKLOADS["stack"], steps=8)
    _say(f"decode stack q8_0 34 layers D=2048 steps=8 persistent={persistent}")
    e, s = _decode_parity(w, w.steps, persistent=persistent, expect_persistent=True)
    _say(f"  stack: out {e:.2e} state {s:.2e}")


@pytest.mark.parametrize("B", [9, 12, 33])
def test_decode_batched_q8_0_matrix_cores(torch, B):
    """B > 8 sequences of Q8_0 decode take the MFMA projections (column count not a
    multiple of 16 for 9 and 33; the conv epilogue runs per sequence)."""
    w = synth.scaled(synth.WORKLOADS["stack"], n_layers=2, batch=B, steps=4, seed=60 + B)
    _say(f"decode batched q8_0 B={B} 2 layers D=2048 4 steps (MFMA projections)")
    e, s = _decode_parity(w, w.steps, snap_every=2)
    _say(f"  B={B}: out {e:.2e} state {s:.2e}")


@pytest.mark.parametrize("B", [5, 9, 33])
def test_decode_batched_bf16_matrix_cores(torch, B):
    """BF16 weights with 5..64 columns take the MFMA products (BF16 weights against x as two
    BF16 terms): a 2-layer D=2048 BF16 stack, 4 steps."""
    w = synth.scaled(synth.WORKLOADS["stack"], wtype="bf16", n_layers=2, batch=B, steps=4, seed=70 + B)
    _say(f"decode batched bf16 B={B} 2 layers D=2048 4 steps (MFMA projections)")
    e, s = _decode_parity(w, w.steps, snap_every=2, expect_persistent=False)
    _say(f"  B={B}: out {e:.2e} state {s:.2e}")


def test_decode_layer_bf16_batched(torch):
    """The BF16 layer workload (no pre-norm, no residual) at B=6: MFMA products."""
    w = synth.scaled(synth.WORKLOADS["layer"], batch=6, steps=6)
    _say("decode layer bf16 B=6 6 steps (MFMA projections)")
    e, s = _decode_parity(w, w.steps, snap_every=3)
    _say(f"  out {e:.2e} state {s:.2e}")


@pytest.mark.timeout(900)
def test_decode_stack_full_run_128_steps(torch):
    """The stack workload as configured: 34 Q8_0 layers, B=1, all 128 decode steps through
    the one-launch kernel, every step's output and the state every 32 steps against the
    oracle (error growth over the whole run)."""
    w = synth.WORKLOADS["stack"]
    _say(f"decode stack q8_0 34 layers D=2048 all {w.steps} steps, one launch, state every 32")
    e, s = _decode_parity(w, w.steps, snap_every=32, expect_persistent=True)
    _say(f"  stack 128 steps: out {e:.2e} state {s:.2e}")


def test_one_launch_window_roll_bit_exact(torch):
    """The one-launch kernel rolls each layer's window in place: after every step rows 0-1
    are bit-for-bit rows 1-2 of the step before, and row 2 is this token's projection
    (against the oracle's, to the output tolerance: the dots round differently)."""
    w = synth.scaled(synth.WORKLOADS["stack"], n_layers=3, steps=6, seed=45)
    run = synth.draw_run(w)
    layers = oracle_layers(run)
    model = gpu_model(run)
    assert model.persistent_blocks() > 0
    _say("one-launch window roll, 3 layers, 6 steps")
    st = model.new_state(1)
    st.S.copy_(torch.from_numpy(run.s0))
    ws = model.workspace(0, 1)
    y = torch.empty((1, model.d_model), dtype=torch.float32, device="cuda")
    S = [run.s0[l, 0].astype(np.float64) for l in range(w.n_layers)]
    Z = [np.zeros((3, w.dims.conv_channels)) for _ in range(w.n_layers)]
    prev = st.conv.cpu().numpy().copy()
    for t in range(w.steps):
        model.decode_step(torch.from_numpy(np.ascontiguousarray(run.x[t, :, 0, :])).cuda(), y, st, ws)
        cur = st.conv.cpu().numpy().copy()
        _, S, Z = ok.stack_step(layers, run.x[t, 0, 0].astype(np.float64)[None, :], S, Z)
        np.testing.assert_array_equal(cur[:, 0, :2].view(np.uint32), prev[:, 0, 1:].view(np.uint32))
        for l in range(w.n_layers):
            assert range_rel(cur[l, 0, 2], Z[l][2]) <= OUT_RTOL
        prev = cur
    model.status()
    model.close()


def test_decode_stack_one_launch_three_layers_32_steps(torch):
    """The one-launch decode over 32 consecutive tokens (tags advance every token), with
    the state checked every 8 steps."""
    w = synth.scaled(synth.WORKLOADS["stack"], n_layers=3, steps=32, seed=23)
    _say("decode one-launch stack 3 layers 32 steps")
    _decode_parity(w, w.steps, snap_every=8, expect_persistent=True)


@pytest.mark.parametrize("D,rank", [(1024, 32), (1024, 128), (2048, 64)])
def test_decode_one_launch_other_shapes(torch, D, rank):
    """The one-launch decode at its other compiled shapes: D = 1024 (8 heads, two input runs
    per wave) and low ranks 32 and 64, whose gate tiles leave lane groups past rank / 32
    empty; two layers, 6 tokens, the state checked every 3."""
    d = synth.LayerDims(d_model=D, n_heads=D // 128, d_k=128, d_v=128, rank_f=rank, rank_g=rank)
    w = synth.scaled(synth.WORKLOADS["stack"], dims=d, n_layers=2, steps=6, seed=70 + rank + D // 1024)
    _say(f"decode one-launch D={D} H={D // 128} rank={rank} 2 layers 6 steps")
    e, s = _decode_parity(w, w.steps, snap_every=3, expect_persistent=True)
    _say(f"  D={D} rank={rank}: out {e:.2e} state {s:.2e}")


def test_graph_replay_equals_eager(torch):
    """The captured hipGraph replays exactly the eager launches (deterministic kernels)."""
    w = synth.scaled(synth.WORKLOADS["layer"], steps=5)
    _say("graph vs eager, layer bf16, 5 steps")
    run = synth.draw_run(w)
    model = gpu_model(run)
    ya, Sa, Za, _ = gpu_decode(model, run, 5, graph=True)
    yb, Sb, Zb, _ = gpu_decode(model, run, 5, graph=False)
    np.testing.assert_array_equal(ya, yb)
    np.testing.assert_array_equal(Sa, Sb)
    np.testing.assert_array_equal(Za, Zb)
    model.close()


def test_conv_window_canonical(torch):
    """kda_conv_window_canonical returns [n_layers][B][3][C], oldest token first: after a
    few steps of the one-launch stack its rows equal the window the oracle holds (to the
    output tolerance: the projections differ by rounding) and the state buffer's own bytes."""
    w = synth.scaled(synth.WORKLOADS["stack"], n_layers=2, steps=5, seed=44)
    run = synth.draw_run(w)
    model = gpu_model(run)
    _say("conv window canonical view, 2-layer one-launch stack, 5 steps")
    st = model.new_state(1)
    st.S.copy_(torch.from_numpy(run.s0))
    ws = model.workspace(0, 1)
    y = torch.empty((1, model.d_model), dtype=torch.float32, device="cuda")
    for t in range(w.steps):
        model.decode_step(torch.from_numpy(np.ascontiguousarray(run.x[t, :, 0, :])).cuda(), y, st, ws)
    out = model.conv_window(st)
    torch.cuda.synchronize()
    model.status()
    assert tuple(out.shape) == (2, 1, 3, model.channels)
    assert torch.equal(out, st.conv)
    _, _, rZ, _ = ok.decode_run(oracle_layers(run), run.x, run.s0, True, steps=w.steps)
    assert range_rel(out.cpu().numpy(), rZ) <= OUT_RTOL
    model.close()


def test_conv_window_indexing_bit_exact(torch):
    """Integer-valued weights and inputs make every projection exact in fp32, so the
    window (copies of the last three projections, oldest first) must match bit for bit."""
    w = synth.scaled(synth.WORKLOADS["tiny"], steps=5, seed=9)
    run = synth.draw_run(w)
    rng = np.random.default_rng(9)
    for dr in run.layers:
        for k in ("wq", "wk", "wv"):
            dr[k] = rng.integers(-2, 3, size=dr[k].shape).astype(np.float32)
    run.x[:] = rng.integers(-3, 4, size=run.x.shape).astype(np.float32)
    _say("conv window bit-exact, tiny, 5 steps")
    layers = oracle_layers(run)
    model = gpu_model(run)
    _, _, Z, _ = gpu_decode(model, run, 5)
    _, _, rZ, _ = ok.decode_run(layers, run.x, run.s0, False, steps=5)
    np.testing.assert_array_equal(Z.astype(np.float64), rZ)
    model.close()


def test_one_launch_wait_limit_times_out_and_recovers(torch):
    """A one-launch step whose waits between blocks run out ends through the kernel's own
    bound: with a 1 us limit set from the host the output blocks give up on the head flags
    at the first layer, every other wait then ends through its own bound, and
    kda_model_status reports the step.  With the default limit restored the model decodes
    the same tokens correctly from a fresh state."""
    import linear_attention_decode_amd as kda
    w = synth.scaled(synth.WORKLOADS["stack"], n_layers=2, steps=3, seed=37)
    run = synth.draw_run(w)
    model = gpu_model(run)
    assert model.persistent_blocks() > 0
    _say("one-launch decode with a 1 us wait limit: one step, expect a reported timeout")
    model.set_option(kda.KDA_OPT_WAIT_US, 1)
    st = model.new_state(1)
    ws = model.workspace(0, 1)
    x = torch.from_numpy(np.ascontiguousarray(run.x[0, :, 0, :])).cuda()
    y = torch.empty((1, model.d_model), dtype=torch.float32, device="cuda")
    model.decode_step(x, y, st, ws)
    torch.cuda.synchronize()
    S_after, Z_after = st.S.clone(), st.conv.clone()
    _say("  a second step before the status call: refused, nothing enqueued")
    with pytest.raises(kda.KdaError) as ei:
        model.decode_step(x, y, st, ws)
    assert ei.value.status == kda._lib.KDA_E_HIP
    with pytest.raises(kda.KdaError):
        model.conv_window(st)
    torch.cuda.synchronize()
    assert torch.equal(st.S, S_after) and torch.equal(st.conv, Z_after)
    with pytest.raises(kda.KdaError):
        model.status()
    model.status()                      # reported once; the exchange words were reset
    _say("  default limit again: 3 steps against the oracle")
    model.set_option(kda.KDA_OPT_WAIT_US, 0)
    ys, S, _, _ = gpu_decode(model, run, w.steps)
    ry, rS, _, _ = ok.decode_run(oracle_layers(run), run.x, run.s0, w.prenorm_residual, steps=w.steps)
    assert max(range_rel(ys[t], ry[t]) for t in range(w.steps)) <= OUT_RTOL
    assert np.abs(S - rS).max() <= STATE_ATOL
    model.close()


def test_one_launch_cooperative_launch(torch):
    """The one-launch decode through the cooperative launch (KDA_OPT_COOPERATIVE = 1) gives
    the same results as the default plain launch, both within the oracle's bounds."""
    import linear_attention_decode_amd as kda
    w = synth.scaled(synth.WORKLOADS["stack"], n_layers=2, steps=4, seed=43)
    run = synth.draw_run(w)
    model = gpu_model(run)
    assert model.persistent_blocks() > 0
    _say("one-launch decode, plain vs cooperative launch, 2 layers 4 steps")
    ya, Sa, Za, _ = gpu_decode(model, run, w.steps)
    model.set_option(kda.KDA_OPT_COOPERATIVE, 1)
    yb, Sb, Zb, _ = gpu_decode(model, run, w.steps)
    model.set_option(kda.KDA_OPT_COOPERATIVE, 0)
    ry, rS, _, _ = ok.decode_run(oracle_layers(run), run.x, run.s0, w.prenorm_residual, steps=w.steps)
    for ys, S in ((ya, Sa), (yb, Sb)):
        assert max(range_rel(ys[t], ry[t]) for t in range(w.steps)) <= OUT_RTOL
        assert np.abs(S - rS).max() <= STATE_ATOL
    np.testing.assert_array_equal(ya, yb)
    np.testing.assert_array_equal(Sa, Sb)
    model.close()
