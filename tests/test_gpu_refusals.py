"""GPU: calls the library refuses (a state batch of 0, T outside 1..8, L = 0, a chunk other
than 64, a weight or input dtype the path does not take, an unaligned pointer, a workspace
or verify log one byte short) return their status before anything is launched, and leave
the state and the conv window bit for bit as they were; the model keeps working afterwards
(a valid call then gives the same bits as on a model that never saw the refused calls)."""
import sys

import numpy as np
import pytest

import synth
from tests.helpers import gpu_model

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _snapshot(st):
    import torch
    torch.cuda.synchronize()
    return st.S.cpu().numpy().copy(), st.conv.cpu().numpy().copy()


def _refused(fn, status):
    import linear_attention_decode_amd as kda
    with pytest.raises(kda.KdaError) as ei:
        fn()
    assert ei.value.status == status, (ei.value.status, status)


def _unaligned_like(t):
    """A tensor of t's shape whose data pointer is 4 bytes past a 16-byte boundary."""
    import torch
    buf = torch.empty(t.numel() + 4, dtype=t.dtype, device=t.device)
    return buf[1:1 + t.numel()].view(t.shape)


def _decode_model(seed):
    d = synth.LayerDims(d_model=256, n_heads=2, d_k=64, d_v=64, rank_f=32, rank_g=32)
    w = synth.scaled(synth.WORKLOADS["tiny"], dims=d, wtype="q8_0", n_layers=2,
                     prenorm_residual=True, batch=2, steps=2, s0_std=0.1, seed=seed)
    return w, synth.draw_run(w)


def test_decode_and_verify_refusals_leave_state_untouched():
    import torch
    import linear_attention_decode_amd as kda
    from linear_attention_decode_amd import _lib
    _say("refused decode / verify / prefill calls on a 2-layer Q8_0 stack, B=2")
    w, run = _decode_model(120)
    model = gpu_model(run)
    st = model.new_state(2)
    st.S.copy_(torch.from_numpy(run.s0))
    st.conv.copy_(torch.randn_like(st.conv))      # a window that is not all zeros
    S0, Z0 = _snapshot(st)
    x = torch.from_numpy(np.ascontiguousarray(run.x[0, :, 0, :])).cuda()
    y = torch.empty_like(x)
    ws = model.workspace(_lib.KDA_OP_DECODE, 2)
    need = kda.kda_workspace_bytes(model.handle, _lib.KDA_OP_DECODE, 2, 1)

    bad = model.new_state(2)
    bad.S.copy_(st.S)
    bad.conv.copy_(st.conv)
    bad.batch = 0
    _refused(lambda: model.decode_step(x, y, bad, ws), _lib.KDA_E_SHAPE)
    _refused(lambda: model.decode_step(x, y, st, ws[:need - 1]), _lib.KDA_E_WORKSPACE)
    _refused(lambda: model.decode_step(x, _unaligned_like(y), st, ws), _lib.KDA_E_ALIGN)

    T = 4
    xv = torch.randn((2, T, w.dims.d_model), device="cuda")
    yv = torch.empty_like(xv)
    log = model.verify_log(2, T)
    wsv = model.workspace(_lib.KDA_OP_VERIFY, 2, T)
    for t_bad in (0, 9):
        _refused(lambda: model.verify_steps(xv, t_bad, yv, st, log, wsv), _lib.KDA_E_SHAPE)
    _refused(lambda: model.verify_steps(xv, T, yv, st, log[:256], wsv), _lib.KDA_E_WORKSPACE)
    # the chunked prefill takes a single BF16 layer without the pre-norm residual
    _refused(lambda: model.prefill_chunked(xv, _lib.KDA_F32, T, 64, yv, st, wsv),
             _lib.KDA_E_UNSUPPORTED)
    _refused(lambda: model.prefill_scan(xv, 0, yv, st, wsv), _lib.KDA_E_SHAPE)

    S1, Z1 = _snapshot(st)
    assert np.array_equal(S1, S0) and np.array_equal(Z1, Z0)

    # a valid step now gives the bits of a model that never saw the refused calls
    model.decode_step(x, y, st, ws)
    fresh = gpu_model(run)
    st2 = fresh.new_state(2)
    st2.S.copy_(torch.from_numpy(S0))
    st2.conv.copy_(torch.from_numpy(Z0))
    y2 = torch.empty_like(x)
    fresh.decode_step(x, y2, st2, fresh.workspace(_lib.KDA_OP_DECODE, 2))
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert torch.equal(st.S, st2.S) and torch.equal(st.conv, st2.conv)
    fresh.close()
    model.close()


def test_prefill_refusals_leave_state_untouched():
    import torch
    from linear_attention_decode_amd import _lib
    d = synth.LayerDims(d_model=256, n_heads=2, d_k=64, d_v=64, rank_f=64, rank_g=64)
    L = 70
    w = synth.scaled(synth.WORKLOADS["prefill"], dims=d, batch=2, tokens=L, s0_std=0.1, seed=121)
    _say(f"refused chunked-prefill calls: BF16 D=256 B=2 L={L}")
    run = synth.draw_run(w)
    model = gpu_model(run)
    st = model.new_state(2)
    st.S.copy_(torch.from_numpy(run.s0))
    st.conv.copy_(torch.randn_like(st.conv))
    S0, Z0 = _snapshot(st)
    x = torch.from_numpy(np.ascontiguousarray(run.x_bits[0]).view(np.int16)).cuda()
    y = torch.empty((2, L, d.d_model), dtype=torch.float32, device="cuda")
    ws = model.workspace(_lib.KDA_OP_PREFILL, 2, L)

    _refused(lambda: model.prefill_chunked(x, _lib.KDA_BF16, 0, 64, y, st, ws), _lib.KDA_E_SHAPE)
    _refused(lambda: model.prefill_chunked(x, _lib.KDA_BF16, L, 32, y, st, ws), _lib.KDA_E_SHAPE)
    _refused(lambda: model.prefill_chunked(x, _lib.KDA_Q8_0, L, 64, y, st, ws), _lib.KDA_E_DTYPE)
    _refused(lambda: model.prefill_chunked(x, _lib.KDA_BF16, L, 64, _unaligned_like(y), st, ws),
             _lib.KDA_E_ALIGN)
    _refused(lambda: model.prefill_chunked(x, _lib.KDA_BF16, L, 64, y, st, ws[:ws.numel() // 2]),
             _lib.KDA_E_WORKSPACE)

    S1, Z1 = _snapshot(st)
    assert np.array_equal(S1, S0) and np.array_equal(Z1, Z0)

    model.prefill_chunked(x, _lib.KDA_BF16, L, 64, y, st, ws)
    fresh = gpu_model(run)
    st2 = fresh.new_state(2)
    st2.S.copy_(torch.from_numpy(S0))
    st2.conv.copy_(torch.from_numpy(Z0))
    y2 = torch.empty_like(y)
    fresh.prefill_chunked(x, _lib.KDA_BF16, L, 64, y2, st2, fresh.workspace(_lib.KDA_OP_PREFILL, 2, L))
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert torch.equal(st.S, st2.S) and torch.equal(st.conv, st2.conv)
    fresh.close()
    model.close()
