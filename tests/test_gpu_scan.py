"""GPU parity of the sequential-scan prefill (kda_prefill_scan) against the oracle run token
by token: every output, the final state and the final window, for single layers and
pre-norm stacks, every weight format and gate form, token blocks that fill the matrix-core
projections, ragged last blocks, one-token blocks (wide batches) and the vector path."""
import sys

import numpy as np
import pytest

import synth
from oracle import kda as ok
from tests.helpers import OUT_RTOL, STATE_ATOL, gpu_model, oracle_layers, range_rel

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _scan_case(w, L, z0=None):
    import torch
    import linear_attention_decode_amd as kda
    run = synth.draw_run(synth.scaled(w, steps=L, tokens=1))
    layers = oracle_layers(run)
    model = gpu_model(run)
    B = w.batch
    st = model.new_state(B)
    st.S.copy_(torch.from_numpy(run.s0))
    if z0 is not None:
        st.conv.copy_(torch.from_numpy(z0))
    x = np.ascontiguousarray(run.x[:, :, 0, :].transpose(1, 0, 2))        # [B][L][D]
    y = torch.empty((B, L, model.d_model), dtype=torch.float32, device="cuda")
    ws = model.workspace(kda.KDA_OP_SCAN, B, L)
    model.prefill_scan(torch.from_numpy(x).cuda(), L, y, st, ws)
    torch.cuda.synchronize()
    yy, S, Z = y.cpu().numpy(), st.S.cpu().numpy(), st.conv.cpu().numpy()
    # oracle: token by token through the whole stack (the same recurrence per layer)
    n_l = w.n_layers
    Ss = [[run.s0[l, b].astype(np.float64) for b in range(B)] for l in range(n_l)]
    Zs = [[(z0[l, b].astype(np.float64) if z0 is not None else np.zeros((3, w.dims.conv_channels)))
           for b in range(B)] for l in range(n_l)]
    worst = 0.0
    for b in range(B):
        for t in range(L):
            xt = run.x[t, b, 0].astype(np.float64)[None, :]
            if w.prenorm_residual:
                ry, s2, z2 = ok.stack_step(layers, xt, [Ss[l][b] for l in range(n_l)], [Zs[l][b] for l in range(n_l)])
            else:
                ry, s1, z1 = ok.layer_forward(layers[0], xt, Ss[0][b], Zs[0][b])
                s2, z2 = [s1], [z1]
            for l in range(n_l):
                Ss[l][b], Zs[l][b] = s2[l], z2[l]
            e = range_rel(yy[b, t], ry[0])
            worst = max(worst, e)
            assert e <= OUT_RTOL, f"seq {b} token {t}: output error {e:.3e}"
    rS = np.array([[Ss[l][b] for b in range(B)] for l in range(n_l)])
    rZ = np.array([[Zs[l][b] for b in range(B)] for l in range(n_l)])
    assert np.abs(S - rS).max() <= STATE_ATOL
    assert range_rel(Z, rZ) <= OUT_RTOL
    model.close()
    return worst, Z


TINY = synth.LayerDims(d_model=256, n_heads=2, d_k=64, d_v=64, rank_f=32, rank_g=32)


@pytest.mark.parametrize("wtype,B,L", [("f32", 2, 20), ("f32", 1, 70), ("bf16", 3, 25), ("q8_0", 2, 9)])
def test_scan_single_layer(wtype, B, L):
    w = synth.scaled(synth.WORKLOADS["tiny"], dims=TINY, wtype=wtype, batch=B, s0_std=0.1, seed=120 + L)
    _say(f"scan single layer {wtype} B={B} L={L}")
    e, _ = _scan_case(w, L)
    _say(f"  worst {e:.2e}")


@pytest.mark.parametrize("B,L", [(3, 40), (40, 3), (70, 2)])
def test_scan_stack_q8_0_d2048(B, L):
    """2-layer Q8_0 stack at D=2048: blocks of 21 tokens x 3 sequences on the matrix-core
    projections (a ragged second block), one-token blocks of 40 sequences (matrix cores)
    and of 70 (vector projections, column passes)."""
    w = synth.scaled(synth.WORKLOADS["stack"], n_layers=2, batch=B, seed=130 + B)
    _say(f"scan stack q8_0 D=2048 2 layers B={B} L={L}")
    e, _ = _scan_case(w, L)
    _say(f"  worst {e:.2e}")


@pytest.mark.parametrize("gate", ["safe", "scalar"])
def test_scan_gate_forms(gate):
    d = synth.LayerDims(d_model=256, n_heads=2, d_k=64, d_v=64, rank_f=32, rank_g=32, gate=gate)
    w = synth.scaled(synth.WORKLOADS["tiny"], dims=d, wtype="bf16", n_layers=2, prenorm_residual=True,
                     batch=2, s0_std=0.1, seed=140)
    _say(f"scan gate={gate} bf16 2-layer stack B=2 L=12")
    _scan_case(w, 12)


@pytest.mark.parametrize("L", [1, 2])
def test_scan_short_keeps_window_rows(L):
    """L = 1 or 2 tokens from a random window: the window's newest 3 - L rows move to the
    front bit for bit."""
    w = synth.scaled(synth.WORKLOADS["tiny"], dims=TINY, wtype="f32", batch=2, s0_std=0.1, seed=150 + L)
    rng = np.random.default_rng(151)
    z0 = rng.standard_normal((1, 2, 3, TINY.conv_channels)).astype(np.float32)
    _say(f"scan L={L} from a random window")
    _, Z = _scan_case(w, L, z0)
    np.testing.assert_array_equal(Z[:, :, :3 - L].view(np.uint32), z0[:, :, L:].view(np.uint32))
