"""GPU parity of the MXFP4 weight format: packing bit for bit against the oracle's
quantiser (device kernel and host packer), and decode / verify / scan prefill through the
per-layer kernels against the oracle run on the same dequantised weights."""
import sys

import numpy as np
import pytest

import synth
from oracle import kda as ok
from tests.helpers import OUT_RTOL, STATE_ATOL, gpu_decode, gpu_model, oracle_layers, range_rel

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


@pytest.mark.parametrize("shape", [(1, 32), (7, 96), (64, 2048), (2048, 128), (5, 4096)])
def test_pack_mxfp4_bit_exact(shape):
    import torch
    import linear_attention_decode_amd as kda
    _say(f"pack mxfp4 {shape}")
    rng = np.random.default_rng(shape[0] * 3 + shape[1])
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    w[0, :32] = 0.0                                    # a block of zeros
    if shape[1] >= 64:
        w[-1, 32:64] *= 1e4                            # a large-scale block
        # values on the midpoints of the grid (ties) at the block's scale
        X = 2.0 ** (np.floor(np.log2(np.abs(w[-1, 32:64]).max())) - 2)
        w[-1, 33:40] = (np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * X).astype(np.float32)
    re, rc = ok.mxfp4_quantize(w)
    nb = kda.kda_packed_bytes(kda.KDA_MXFP4, *shape)
    for host in (False, True):
        buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
        if host:
            kda.kda_pack(kda.KDA_MXFP4, w, buf)
        else:
            kda.kda_pack_device(kda.KDA_MXFP4, torch.from_numpy(w).cuda(), buf)
        e, c = kda.kda_unpack_mxfp4(buf, *shape)
        np.testing.assert_array_equal(e, re)
        np.testing.assert_array_equal(c, rc)


@pytest.mark.parametrize("gate", ["kda", "scalar"])
def test_decode_mxfp4_small_stack(gate):
    d = synth.LayerDims(d_model=256, n_heads=2, d_k=64, d_v=64, rank_f=64, rank_g=64, gate=gate)
    w = synth.scaled(synth.WORKLOADS["tiny"], dims=d, wtype="mxfp4", n_layers=2, prenorm_residual=True,
                     batch=3, steps=8, s0_std=0.1, seed=161)
    _say(f"decode mxfp4 gate={gate} 2 layers D=256 B=3 8 steps")
    run = synth.draw_run(w)
    layers = oracle_layers(run)
    model = gpu_model(run)
    y, S, Z, snaps = gpu_decode(model, run, w.steps, 4)
    ry, rS, rZ, rsn = ok.decode_run(layers, run.x, run.s0, True, check_every=4)
    e = max(range_rel(y[t], ry[t]) for t in range(w.steps))
    assert e <= OUT_RTOL, e
    assert np.abs(S - rS).max() <= STATE_ATOL
    for k in snaps:
        assert np.abs(snaps[k] - rsn[k]).max() <= STATE_ATOL
    assert range_rel(Z, rZ) <= OUT_RTOL
    model.close()
    _say(f"  out {e:.2e}")


def test_decode_mxfp4_stack_d2048():
    """The stack workload's shapes (D=2048, 16 heads, rank 128) with MXFP4 projections,
    4 layers, 6 steps: B = 1 through the one-launch kernel (on the exact int8 expansion of
    the codes) and through the per-layer kernels (vector dots), B = 4 and 9 per layer
    (matrix cores: the codes converted to BF16 by gfx950's scaled FP4 conversion).  The
    per-layer kernels read the caller's 4-bit buffers, so the model owns no copy."""
    for B in (1, 4, 9):
        w = synth.scaled(synth.WORKLOADS["stack"], wtype="mxfp4", n_layers=4, batch=B, steps=6, seed=162 + B)
        _say(f"decode mxfp4 D=2048 4 layers B={B} 6 steps")
        run = synth.draw_run(w)
        model = gpu_model(run)
        assert model.persistent_blocks() > 0 and not model.owns_weights()
        ry, rS, rZ, _ = ok.decode_run(oracle_layers(run), run.x, run.s0, True)
        for persistent in ((True, False) if B == 1 else (False,)):
            y, S, Z, _ = gpu_decode(model, run, w.steps, persistent=persistent)
            e = max(range_rel(y[t], ry[t]) for t in range(w.steps))
            assert e <= OUT_RTOL, e
            assert np.abs(S - rS).max() <= STATE_ATOL
            _say(f"  B={B} {'one launch' if persistent and B == 1 else 'per layer'}: out {e:.2e}")
        model.close()


@pytest.mark.parametrize("case", ["zero_block", "scale_beyond_fp16"])
def test_mxfp4_one_launch_eligibility(case):
    """An MXFP4 stack runs the one-launch decode when every nonzero block's scale has an fp16
    power of two: a block of zeros (E8M0 exponent -127) does not stop it; W_q scaled by
    2^-30 (exponents far below fp16's) keeps the stack on the per-layer kernels.  Either way
    B = 1 matches the oracle (2 layers, 4 steps)."""
    w = synth.scaled(synth.WORKLOADS["stack"], wtype="mxfp4", n_layers=2, batch=1, steps=4, seed=168)
    _say(f"mxfp4 one-launch eligibility: {case}")
    run = synth.draw_run(w)
    if case == "zero_block":
        run.layers[1]["wo"][5, 64:96] = 0.0
    else:
        run.layers[0]["wq"] *= np.float32(2.0 ** -30)
    model = gpu_model(run)
    assert (model.persistent_blocks() > 0) == (case == "zero_block")
    y, S, Z, _ = gpu_decode(model, run, w.steps)
    ry, rS, rZ, _ = ok.decode_run(oracle_layers(run), run.x, run.s0, True)
    e = max(range_rel(y[t], ry[t]) for t in range(w.steps))
    assert e <= OUT_RTOL, e
    assert np.abs(S - rS).max() <= STATE_ATOL
    model.close()
    _say(f"  out {e:.2e}")


def test_verify_and_scan_mxfp4():
    """Verify + commit (B=2, T=4) and a 10-token scan prefill on a 2-layer MXFP4 stack."""
    import torch
    import linear_attention_decode_amd as kda
    d = synth.LayerDims(d_model=256, n_heads=2, d_k=64, d_v=64, rank_f=32, rank_g=32)
    w = synth.scaled(synth.WORKLOADS["verify"], dims=d, wtype="mxfp4", n_layers=2, batch=2, tokens=4,
                     steps=2, seed=165)
    _say("verify + commit mxfp4 2 layers B=2 T=4, 2 steps")
    run = synth.draw_run(w)
    layers = oracle_layers(run)
    model = gpu_model(run)
    st = model.new_state(2)
    st.S.copy_(torch.from_numpy(run.s0))
    ws = model.workspace(kda.KDA_OP_VERIFY, 2, 4)
    log = model.verify_log(2, 4)
    y = torch.empty((2, 4, 256), dtype=torch.float32, device="cuda")
    S = [[run.s0[l, b].astype(np.float64) for b in range(2)] for l in range(2)]
    Z = [[np.zeros((3, d.conv_channels)) for _ in range(2)] for _ in range(2)]
    for t in range(w.steps):
        model.verify_steps(torch.from_numpy(np.ascontiguousarray(run.x[t])).cuda(), 4, y, st, log, ws)
        model.verify_commit(st, log, 4, torch.from_numpy(run.accept[t].copy()).cuda())
        yy = y.cpu().numpy()
        for b in range(2):
            ry, s2, z2 = ok.stack_step(layers, run.x[t, b].astype(np.float64), [S[l][b] for l in range(2)],
                                       [Z[l][b] for l in range(2)], keep_after=int(run.accept[t, b]))
            assert range_rel(yy[b], ry) <= OUT_RTOL
            for l in range(2):
                S[l][b], Z[l][b] = s2[l], z2[l]
    model.flush(st)
    assert np.abs(st.S.cpu().numpy() - np.array([[S[l][b] for b in range(2)] for l in range(2)])).max() <= STATE_ATOL
    # then a scan prefill of 10 tokens from the committed state
    _say("  scan prefill 10 tokens from the committed state")
    x = np.random.default_rng(166).standard_normal((2, 10, 256)).astype(np.float32)
    ys = torch.empty((2, 10, 256), dtype=torch.float32, device="cuda")
    model.prefill_scan(torch.from_numpy(x).cuda(), 10, ys, st, model.workspace(kda.KDA_OP_SCAN, 2, 10))
    yy = ys.cpu().numpy()
    for b in range(2):
        for t in range(10):
            ry, s2, z2 = ok.stack_step(layers, x[b, t].astype(np.float64)[None, :], [S[l][b] for l in range(2)],
                                       [Z[l][b] for l in range(2)])
            for l in range(2):
                S[l][b], Z[l][b] = s2[l], z2[l]
            assert range_rel(yy[b, t], ry[0]) <= OUT_RTOL
    assert np.abs(st.S.cpu().numpy() - np.array([[S[l][b] for b in range(2)] for l in range(2)])).max() <= STATE_ATOL
    model.close()
