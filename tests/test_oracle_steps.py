"""Pins of the oracle's per-token steps and of the layer / stack wiring.

Every pin is checked against something other than the oracle's own formula: closed forms
of special cases, invariants the pages or the mathematics fix, and a brute-force product
form of the recurrence.  Each pin is also run against a planted mistake (a mutant of the
oracle function, on the CPU) to show that it bites.
"""
import math

import numpy as np
import pytest

import synth
from oracle import kda as ok

RNG = np.random.default_rng


# ----------------------------------------------------------------------------------------
# conv + SiLU + window roll
# ----------------------------------------------------------------------------------------
def pin_conv(conv_fn) -> bool:
    rng = RNG(1)
    C = 12
    p_seq = rng.standard_normal((6, C))
    # identity kernel: a = SiLU(p), whatever the window holds
    w_id = np.zeros((C, 4)); w_id[:, 3] = 1.0
    Z = rng.standard_normal((3, C))
    a, Z2 = conv_fn(Z, p_seq[0], w_id)
    ok1 = np.allclose(a, p_seq[0] / (1 + np.exp(-p_seq[0])), rtol=1e-15, atol=0)
    ok2 = np.array_equal(Z2, np.concatenate([Z[1:], p_seq[:1]]))
    # impulse at t=0 then zeros: outputs walk back through the taps 3, 2, 1, 0
    w = rng.standard_normal((C, 4))
    Z = np.zeros((3, C))
    imp = rng.standard_normal(C)
    outs = []
    for t in range(4):
        a, Z = conv_fn(Z, imp if t == 0 else np.zeros(C), w)
        outs.append(a)
    ok3 = all(np.allclose(outs[t], ok.silu(w[:, 3 - t] * imp), rtol=1e-14, atol=1e-300)
              for t in range(4))
    return ok1 and ok2 and ok3


def test_conv_pins():
    assert pin_conv(ok.conv_silu)


def test_conv_mutant_reversed_taps():
    def mutant(Z, p, w):
        return ok.conv_silu(Z, p, w[:, ::-1])
    assert not pin_conv(mutant)


def test_conv_mutant_window_not_rolled():
    def mutant(Z, p, w):
        a, _ = ok.conv_silu(Z, p, w)
        return a, np.concatenate([p[None, :], Z[:-1]])
    assert not pin_conv(mutant)


# ----------------------------------------------------------------------------------------
# head split + L2 norms
# ----------------------------------------------------------------------------------------
def pin_split(split_fn) -> bool:
    rng = RNG(2)
    H, dk, dv = 3, 8, 5
    a = rng.standard_normal(2 * H * dk + H * dv) * 3
    q, k, v = split_fn(a, H, dk, dv, 0.0)
    good = np.allclose(np.linalg.norm(k, axis=1), 1.0, rtol=1e-14)
    good &= np.allclose(np.linalg.norm(q, axis=1), dk ** -0.5, rtol=1e-14)
    # q of head 1 is parallel to channels [dk, 2dk), k of head 0 to [H dk, H dk + dk)
    good &= np.allclose(q[1] / np.linalg.norm(q[1]), a[dk:2 * dk] / np.linalg.norm(a[dk:2 * dk]))
    good &= np.allclose(k[0] / np.linalg.norm(k[0]), a[H * dk:H * dk + dk] / np.linalg.norm(a[H * dk:H * dk + dk]))
    good &= np.array_equal(v[2], a[2 * H * dk + 2 * dv: 2 * H * dk + 3 * dv])
    return bool(good)


def test_split_pins():
    assert pin_split(ok.split_heads)


def test_split_mutant_scale_on_k():
    def mutant(a, H, dk, dv, eps):
        q, k, v = ok.split_heads(a, H, dk, dv, eps)
        return q / dk ** -0.5, k * dk ** -0.5, v
    assert not pin_split(mutant)


# ----------------------------------------------------------------------------------------
# forget gate
# ----------------------------------------------------------------------------------------
def pin_gate(gate_fn) -> bool:
    # softplus(0) = ln 2 and exp(A_log=0) = 1  =>  alpha = exp(-ln 2) = 1/2
    a = gate_fn(np.zeros((2, 3)), np.zeros(2))
    good = np.allclose(a, 0.5, rtol=1e-15)
    # large positive f: softplus(f) -> f, alpha -> exp(-e^{A_log} f)
    f = np.full((1, 2), 40.0)
    good &= np.allclose(gate_fn(f, np.array([math.log(0.25)])), math.exp(-10.0), rtol=1e-12)
    # large negative f: softplus(f) -> e^f, alpha -> 1 - e^{A_log} e^f
    f = np.full((1, 1), -30.0)
    good &= np.allclose(gate_fn(f, np.array([0.0])), math.exp(-math.exp(-30.0)), rtol=1e-15)
    # alpha in (0, 1], and A_log -> -inf gives exactly 1
    rng = RNG(3)
    al = gate_fn(rng.standard_normal((4, 16)) * 3, rng.uniform(-1, 0, 4))
    good &= bool(np.all((al > 0) & (al < 1)))
    good &= np.array_equal(gate_fn(rng.standard_normal((2, 4)), np.array([-np.inf, -np.inf])),
                           np.ones((2, 4)))
    return bool(good)


def test_gate_pins():
    assert pin_gate(ok.forget_gate)


def test_gate_mutant_softplus_sign():
    def mutant(f, a_log):
        return np.exp(-np.exp(a_log)[:, None] * ok.softplus(-f))
    assert not pin_gate(mutant)


def test_sigmoid_softplus_closed_forms():
    assert ok.sigmoid(0.0) == 0.5
    assert abs(ok.softplus(0.0) - math.log(2.0)) < 1e-16
    z = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(ok.softplus(z), np.log1p(np.exp(z)), rtol=1e-14)
    np.testing.assert_allclose(ok.sigmoid(z) + ok.sigmoid(-z), 1.0, rtol=1e-15)


# ----------------------------------------------------------------------------------------
# delta rule
# ----------------------------------------------------------------------------------------
def _unit(v):
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def brute_force_states(S0, k, v, alpha, beta):
    """S_T = (prod_t A_t) S0 + sum_s (prod_{t>s} A_t) beta_s k_s v_s^T with
    A_t = (I - beta_t k_t k_t^T) diag(alpha_t), recomputed from S0 for every T."""
    T, dk = k.shape
    out = []
    for Tn in range(1, T + 1):
        S = np.zeros_like(S0)
        for s in range(-1, Tn):
            P = np.eye(dk)
            for t in range(s + 1, Tn):
                A_t = (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(alpha[t])
                P = A_t @ P
            S = S + (P @ S0 if s < 0 else P @ (beta[s] * np.outer(k[s], v[s])))
        out.append(S)
    return out


def pin_delta(step_fn) -> bool:
    rng = RNG(4)
    H, dk, dv = 2, 6, 5
    good = True
    # beta = 1, unit k: the updated state maps k exactly onto v
    S = rng.standard_normal((H, dk, dv))
    k = _unit(rng.standard_normal((H, dk)))
    v = rng.standard_normal((H, dv))
    q = rng.standard_normal((H, dk))
    alpha = rng.uniform(0.2, 1.0, (H, dk))
    S2, _ = step_fn(S, q, k, v, alpha, np.ones(H))
    good &= np.allclose(np.einsum("hij,hi->hj", S2, k), v, rtol=0, atol=1e-13)
    # alpha = 1, beta = 0: unchanged
    S2, _ = step_fn(S, q, k, v, np.ones((H, dk)), np.zeros(H))
    good &= np.array_equal(S2, S)
    # S0 = 0, one token: S = beta k v^T, o = beta (k.q) v
    beta = rng.uniform(0.1, 1.0, H)
    S2, o = step_fn(np.zeros((H, dk, dv)), q, k, v, alpha, beta)
    good &= np.allclose(S2, beta[:, None, None] * k[:, :, None] * v[:, None, :], atol=1e-15)
    good &= np.allclose(o, (beta * np.sum(k * q, 1))[:, None] * v, atol=1e-15)
    # beta = 0 for T tokens: S_T = diag(prod alpha) S0
    T = 5
    al = rng.uniform(0.3, 1.0, (T, H, dk))
    S2 = S
    for t in range(T):
        S2, _ = step_fn(S2, q, k, v, al[t], np.zeros(H))
    good &= np.allclose(S2, np.prod(al, 0)[:, :, None] * S, rtol=1e-14)
    # brute force over T tokens from S0 (rectangular dk != dv catches transposes)
    T = 6
    ks = _unit(rng.standard_normal((T, H, dk)))
    vs = rng.standard_normal((T, H, dv))
    qs = rng.standard_normal((T, H, dk))
    als = rng.uniform(0.3, 1.0, (T, H, dk))
    bs = rng.uniform(0.0, 1.0, (T, H))
    S2 = S
    for t in range(T):
        S2, o = step_fn(S2, qs[t], ks[t], vs[t], als[t], bs[t])
        for h in range(H):
            ref = brute_force_states(S[h], ks[:t + 1, h], vs[:t + 1, h], als[:t + 1, h], bs[:t + 1, h])[-1]
            good &= np.allclose(S2[h], ref, rtol=1e-12, atol=1e-12)
            good &= np.allclose(o[h], ref.T @ qs[t, h], rtol=1e-12, atol=1e-12)
    return bool(good)


def test_delta_rule_pins():
    assert pin_delta(ok.delta_rule_step)


@pytest.mark.parametrize("which", ["read_before_update", "decay_on_values", "no_decay_in_error",
                                   "transposed_readout"])
def test_delta_rule_mutants(which):
    def mutant(S, q, k, v, alpha, beta):
        if which == "read_before_update":
            S1 = alpha[:, :, None] * S
            S_new, _ = ok.delta_rule_step(S, q, k, v, alpha, beta)
            return S_new, np.einsum("hij,hi->hj", S1, q)
        if which == "decay_on_values":
            if S.shape[1] != S.shape[2]:
                alpha = np.resize(alpha, (S.shape[0], S.shape[2]))
            S1 = S * alpha[:, None, :]
        else:
            S1 = alpha[:, :, None] * S
        base = S if which == "no_decay_in_error" else S1
        e = np.einsum("hij,hi->hj", base, k)
        delta = beta[:, None] * (v - e)
        S_new = S1 + k[:, :, None] * delta[:, None, :]
        if which == "transposed_readout":
            n = min(S.shape[1], S.shape[2])
            o = np.einsum("hij,hj->hi", S_new[:, :n, :n], q[:, :n])
            o = np.resize(o, (S.shape[0], S.shape[2]))
        else:
            o = np.einsum("hij,hi->hj", S_new, q)
        return S_new, o
    assert not pin_delta(mutant)


# ----------------------------------------------------------------------------------------
# gated norm and RMSNorm
# ----------------------------------------------------------------------------------------
def test_gated_norm_rms_is_one():
    rng = RNG(5)
    o = rng.standard_normal((4, 32)) * 3
    n = ok.gated_norm(o, np.ones((4, 32)), np.ones(32), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, axis=1)), 1.0, rtol=1e-14)
    g = rng.uniform(0.1, 1, (4, 32))
    n2 = ok.gated_norm(o, g, np.ones(32), 0.0)
    np.testing.assert_allclose(n2 / g, n, rtol=1e-14)
    # per head: scaling one head does not change another
    o2 = o.copy(); o2[0] *= 100
    np.testing.assert_allclose(ok.gated_norm(o2, g, np.ones(32), 0.0)[1:], n2[1:], rtol=1e-14)


# ----------------------------------------------------------------------------------------
# layer and stack wiring
# ----------------------------------------------------------------------------------------
def _tiny_layer(seed=7, **over):
    w = synth.WORKLOADS["tiny"]
    run = synth.draw_run(synth.scaled(w, seed=seed, steps=2))
    L = ok.prepare_layer(run.layers[0], "f32", w.dims.n_heads, w.dims.d_k, w.dims.d_v)
    for k, v in over.items():
        setattr(L, k, v)
    return L, run


def pin_single_token(layer_fn) -> bool:
    """S0 = 0, empty window, one token, RMSNorm eps 0:
    o_h = beta_h (k_h . q_h) v_h, so n_h = sign(k_h . q_h) v_h / rms(v_h) * gate_h and
    out = W_o n, independent of alpha and of |beta|."""
    L, run = _tiny_layer(norm_eps=0.0)
    H, dk, dv = L.n_heads, L.d_k, L.d_v
    u = run.x[0, 0, 0].astype(np.float64)
    out, _, _ = layer_fn(L, u[None, :], np.zeros((H, dk, dv)), np.zeros((3, L.channels)))
    w3 = L.conv_w[:, 3]
    K = H * dk
    sl = lambda y: y / (1 + np.exp(-y))
    qa = sl(w3[:K] * (L.wq @ u)).reshape(H, dk)
    ka = sl(w3[K:2 * K] * (L.wk @ u)).reshape(H, dk)
    va = sl(w3[2 * K:] * (L.wv @ u)).reshape(H, dv)
    gate = 1 / (1 + np.exp(-(L.gb @ (L.ga @ u)))).reshape(H, dv)
    sgn = np.sign(np.sum(qa * ka, axis=1))
    n = sgn[:, None] * va / np.sqrt(np.mean(va * va, axis=1, keepdims=True)) * gate
    return bool(np.allclose(out[0], L.wo @ n.reshape(-1), rtol=1e-10, atol=1e-12))


def pin_two_tokens_projection(layer_fn) -> bool:
    """alpha = 1 (A_log = -inf), beta = 1 (huge beta logits), identity conv, S0 = 0:
    S_2 = (I - k2 k2^T) k1 v1^T + k2 v2^T, o_2 = v1 (k1.q2 - (k1.k2)(k2.q2)) + v2 (k2.q2).
    Distinguishes the q and k slots (unlike the single-token form)."""
    L, run = _tiny_layer(seed=8, norm_eps=0.0, l2_eps=0.0)
    H, dk, dv = L.n_heads, L.d_k, L.d_v
    L.a_log = np.full(H, -np.inf)
    L.wbeta = np.abs(L.wbeta) * 1e4          # logits >> 40: sigmoid == 1 in float64
    cw = np.zeros_like(L.conv_w); cw[:, 3] = 1.0
    L.conv_w = cw
    U = np.abs(run.x[:2, 0, 0].astype(np.float64))
    out, S_end, _ = layer_fn(L, U, np.zeros((H, dk, dv)), np.zeros((3, L.channels)))
    K = H * dk
    sl = lambda y: y / (1 + np.exp(-y))
    good = True
    for t in range(2):
        assert np.all(L.wbeta @ U[t] > 40)
    qs = [sl(L.wq @ U[t]).reshape(H, dk) for t in range(2)]
    ks = [sl(L.wk @ U[t]).reshape(H, dk) for t in range(2)]
    vs = [sl(L.wv @ U[t]).reshape(H, dv) for t in range(2)]
    qs = [q / np.linalg.norm(q, axis=1, keepdims=True) * dk ** -0.5 for q in qs]
    ks = [k / np.linalg.norm(k, axis=1, keepdims=True) for k in ks]
    gate = 1 / (1 + np.exp(-(L.gb @ (L.ga @ U[1])))).reshape(H, dv)
    o2 = np.empty((H, dv))
    for h in range(H):
        k1, k2, q2, v1, v2 = ks[0][h], ks[1][h], qs[1][h], vs[0][h], vs[1][h]
        o2[h] = v1 * (k1 @ q2 - (k1 @ k2) * (k2 @ q2)) + v2 * (k2 @ q2)
        S2 = np.outer(k1, v1) - np.outer(k2, (k2 @ k1) * v1) + np.outer(k2, v2)
        good &= np.allclose(S_end[h], S2, rtol=1e-9, atol=1e-9)
    n = o2 / np.sqrt(np.mean(o2 * o2, axis=1, keepdims=True)) * gate
    good &= np.allclose(out[1], L.wo @ n.reshape(-1), rtol=1e-8, atol=1e-10)
    return bool(good)


def test_layer_single_token_closed_form():
    assert pin_single_token(ok.layer_forward)


def test_layer_two_token_projection_form():
    assert pin_two_tokens_projection(ok.layer_forward)


@pytest.mark.parametrize("which", ["qk_swapped", "v_from_k", "wo_rows_permuted", "gate_on_o"])
def test_layer_wiring_mutants(monkeypatch, which):
    real_split = ok.split_heads
    real_norm = ok.gated_norm
    real = ok.layer_forward
    if which == "qk_swapped":
        def split(a, H, dk, dv, eps):
            K = H * dk
            b = np.concatenate([a[K:2 * K], a[:K], a[2 * K:]])
            return real_split(b, H, dk, dv, eps)
        monkeypatch.setattr(ok, "split_heads", split)
    elif which == "v_from_k":
        def split(a, H, dk, dv, eps):
            q, k, v = real_split(a, H, dk, dv, eps)
            K = H * dk
            return q, k, a[K:K + H * dv].reshape(H, dv)
        monkeypatch.setattr(ok, "split_heads", split)
    elif which == "gate_on_o":
        def norm(o, gate, w, eps):
            return real_norm(o * gate, np.ones_like(gate), w, eps)
        monkeypatch.setattr(ok, "gated_norm", norm)

    def layer(L, U, S, Z, **kw):
        if which == "wo_rows_permuted":
            L = ok.OracleLayer(**{**L.__dict__, "wo": L.wo[::-1].copy()})
        return real(L, U, S, Z, **kw)
    assert not (pin_single_token(layer) and pin_two_tokens_projection(layer))


def test_stack_zero_output_projection_is_identity():
    w = synth.scaled(synth.WORKLOADS["tiny"], n_layers=3, prenorm_residual=True, steps=3)
    run = synth.draw_run(w)
    d = w.dims
    layers = [ok.prepare_layer(dr, "f32", d.n_heads, d.d_k, d.d_v) for dr in run.layers]
    for L in layers:
        L.wo = np.zeros_like(L.wo)
    X = run.x[:, 0, 0].astype(np.float64)
    y, S, Z = ok.stack_step(layers, X, [np.zeros((d.n_heads, d.d_k, d.d_v))] * 3,
                            [np.zeros((3, d.conv_channels))] * 3)
    np.testing.assert_array_equal(y, X)
    assert all(np.abs(s).max() > 0 for s in S)


def test_rms_norm_has_unit_rms():
    x = RNG(6).standard_normal((5, 100)) * 7
    y = ok.rms_norm(x, 1.0, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)


def test_verify_commit_semantics():
    """Accepting all T tokens every step equals plain decode of the flattened token
    stream; accepting a < T commits exactly the state after the first a tokens."""
    base = synth.scaled(synth.WORKLOADS["tiny"], n_layers=2, prenorm_residual=True,
                        batch=2, steps=3, tokens=3, s0_std=0.1)
    run = synth.draw_run(base)
    d = base.dims
    layers = [ok.prepare_layer(dr, "f32", d.n_heads, d.d_k, d.d_v) for dr in run.layers]
    full = np.full((3, 2), 3, np.int32)
    y, S, Z = ok.verify_run(layers, run.x, run.s0, full)
    xflat = run.x.transpose(1, 0, 2, 3).reshape(2, 9, -1).transpose(1, 0, 2)[:, :, None, :]
    y2, S2, Z2, _ = ok.decode_run(layers, xflat, run.s0, True)
    np.testing.assert_allclose(y.transpose(1, 0, 2, 3).reshape(2, 9, -1),
                               y2.transpose(1, 0, 2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S2, rtol=1e-12, atol=1e-12)
    # windows hold projections, computed by BLAS over blocks of different widths
    np.testing.assert_allclose(Z, Z2, rtol=1e-12, atol=1e-14)
    # one step, accept 2 of 3: state == decode of the first 2 tokens
    acc = np.array([[2, 1]], np.int32)
    _, S3, Z3 = ok.verify_run(layers, run.x[:1], run.s0, acc)
    for b, a in enumerate([2, 1]):
        xb = run.x[0, b, :a][:, None, None, :]
        _, S4, Z4, _ = ok.decode_run(layers, xb, run.s0[:, b:b + 1], True)
        np.testing.assert_allclose(S3[:, b], S4[:, 0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Z3[:, b], Z4[:, 0], rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------------------
# wiring of the pre-norm, the forget gate's inputs and beta's heads
# ----------------------------------------------------------------------------------------
def _single_token_out(L, u):
    """Closed form of one token from S0 = 0 and an empty window, RMSNorm eps 0 (see
    pin_single_token): out = W_o n with n_h = sign(k_h . q_h) v_h / rms(v_h) * gate_h."""
    H, dk, dv = L.n_heads, L.d_k, L.d_v
    K = H * dk
    w3 = L.conv_w[:, 3]
    sl = lambda y: y / (1 + np.exp(-y))
    qa = sl(w3[:K] * (L.wq @ u)).reshape(H, dk)
    ka = sl(w3[K:2 * K] * (L.wk @ u)).reshape(H, dk)
    va = sl(w3[2 * K:] * (L.wv @ u)).reshape(H, dv)
    gate = 1 / (1 + np.exp(-(L.gb @ (L.ga @ u)))).reshape(H, dv)
    sgn = np.sign(np.sum(qa * ka, axis=1))
    n = sgn[:, None] * va / np.sqrt(np.mean(va * va, axis=1, keepdims=True)) * gate
    return L.wo @ n.reshape(-1)


def pin_stack_prenorm(stack_fn) -> bool:
    """One layer of the pre-norm residual stack from S0 = 0 and an empty window:
    (a) RMSNorm makes the layer's input scale-free, so x1(10 x) - 10 x = x1(x) - x;
    (b) x1 - x is the single-token closed form at u = x / sqrt(mean(x^2)) (the RMS of the
    residual stream, weight ones, eps 0), which fixes the mean (not the sum) of squares."""
    L, run = _tiny_layer(seed=11, norm_eps=0.0)
    H, dk, dv = L.n_heads, L.d_k, L.d_v
    x = run.x[0, 0, 0].astype(np.float64) * 3.0
    S0 = [np.zeros((H, dk, dv))]
    Z0 = [np.zeros((3, L.channels))]
    y1, _, _ = stack_fn([L], x[None, :], S0, Z0, eps=0.0)
    y10, _, _ = stack_fn([L], 10.0 * x[None, :], S0, Z0, eps=0.0)
    good = np.allclose(y10[0] - 10.0 * x, y1[0] - x, rtol=1e-9, atol=1e-11)
    u = x / np.sqrt(np.mean(x * x))
    good &= np.allclose(y1[0] - x, _single_token_out(L, u), rtol=1e-10, atol=1e-12)
    return bool(good)


def test_stack_prenorm_wiring():
    assert pin_stack_prenorm(ok.stack_step)


def test_stack_prenorm_mutant_no_norm():
    def mutant(layers, X, S, Z, keep_after=None, eps=1e-6):
        X = np.array(np.atleast_2d(X), np.float64, copy=True)
        for l, L in enumerate(layers):
            out, _, _ = ok.layer_forward(L, X, S[l], Z[l], keep_after=keep_after)
            X = X + out
        return X, None, None
    assert not pin_stack_prenorm(mutant)


def test_stack_prenorm_mutant_l2_norm():
    def mutant(layers, X, S, Z, keep_after=None, eps=1e-6):
        X = np.array(np.atleast_2d(X), np.float64, copy=True)
        for l, L in enumerate(layers):
            h = X / np.sqrt(np.sum(X * X, axis=-1, keepdims=True) + eps)
            out, _, _ = ok.layer_forward(L, h, S[l], Z[l], keep_after=keep_after)
            X = X + out
        return X, None, None
    assert not pin_stack_prenorm(mutant)


def pin_forget_gate_wiring(layer_fn) -> bool:
    """F_a = 0 makes the forget-gate input f = dt_bias exactly.  Token 1 has beta = 1 and
    token 2 = -token 1 has beta = 0 (huge beta logits of opposite signs), so from S0 = 0
    the delta rule reduces to S1 = k1 v1^T and S2 = diag(alpha) S1 with
    alpha_{h,i} = exp(-exp(A_log[h]) softplus(dt_bias[h dk + i])) (the workload's gate
    formula), evaluated here with libm scalars; the A_log values of the heads differ, so a
    head mix-up shows.  A second case with dt_bias = 0 and F_a, F_b random checks the
    low-rank term f = F_b (F_a u) the same way."""
    L, run = _tiny_layer(seed=12, norm_eps=0.0)
    H, dk, dv = L.n_heads, L.d_k, L.d_v
    u1 = run.x[0, 0, 0].astype(np.float64)
    # beta logits of several thousand: rows aligned with u1 so that W_beta u1 >> 0
    L.wbeta = np.tile(u1 / np.linalg.norm(u1), (H, 1)) * np.linspace(3e3, 5e3, H)[:, None]
    L.a_log = np.linspace(-0.9, 0.4, H)
    U = np.stack([u1, -u1])
    good = True
    for case in ("bias", "lowrank"):
        if case == "bias":
            L.fa = np.zeros_like(L.fa)
        else:
            rng = RNG(13)
            L.fa = rng.standard_normal(L.fa.shape) * 0.2
            L.fb = rng.standard_normal(L.fb.shape) * 0.5
            L.dt_bias = np.zeros_like(L.dt_bias)
        _, S1, _ = layer_fn(L, U[:1], np.zeros((H, dk, dv)), np.zeros((3, L.channels)))
        _, S2, _ = layer_fn(L, U, np.zeros((H, dk, dv)), np.zeros((3, L.channels)))
        f = L.dt_bias if case == "bias" else L.fb @ (L.fa @ U[1])
        for h in range(H):
            for i in range(dk):
                z = float(f[h * dk + i])
                sp = max(z, 0.0) + math.log1p(math.exp(-abs(z)))
                a = math.exp(-math.exp(float(L.a_log[h])) * sp)
                good &= np.allclose(S2[h, i], a * S1[h, i], rtol=1e-12, atol=1e-15)
    return bool(good)


def test_forget_gate_wiring():
    assert pin_forget_gate_wiring(ok.layer_forward)


@pytest.mark.parametrize("which", ["no_dt_bias", "a_log_heads_reversed", "fa_fb_swapped_order"])
def test_forget_gate_wiring_mutants(which):
    real = ok.layer_forward

    def layer(L, U, S, Z, **kw):
        kv = dict(L.__dict__)
        if which == "no_dt_bias":
            kv["dt_bias"] = np.zeros_like(L.dt_bias)
        elif which == "a_log_heads_reversed":
            kv["a_log"] = L.a_log[::-1].copy()
        else:   # f = F_b (F_a u) with the low-rank vector reversed in between
            kv["fb"] = L.fb[:, ::-1].copy()
        return real(ok.OracleLayer(**kv), U, S, Z, **kw)
    assert not pin_forget_gate_wiring(layer)


def pin_beta_heads(layer_fn) -> bool:
    """One token from S0 = 0 and an empty window: S_h = beta_h k_h v_h^T with
    beta_h = sigmoid((W_beta u)_h) and k_h, v_h the head's slices of SiLU(w[:, 3] * p)
    (k L2-normalised); the betas of the heads differ, so a row mix-up of W_beta shows."""
    L, run = _tiny_layer(seed=14, norm_eps=0.0, l2_eps=0.0)
    H, dk, dv = L.n_heads, L.d_k, L.d_v
    K = H * dk
    u = run.x[0, 0, 0].astype(np.float64)
    # spread the logits so the heads' betas are far apart
    L.wbeta = L.wbeta * np.linspace(1.0, 8.0, H)[:, None]
    _, S, _ = layer_fn(L, u[None, :], np.zeros((H, dk, dv)), np.zeros((3, L.channels)))
    w3 = L.conv_w[:, 3]
    sl = lambda y: y / (1 + np.exp(-y))
    ka = sl(w3[K:2 * K] * (L.wk @ u)).reshape(H, dk)
    ka = ka / np.linalg.norm(ka, axis=1, keepdims=True)
    va = sl(w3[2 * K:] * (L.wv @ u)).reshape(H, dv)
    good = True
    for h in range(H):
        b = 1.0 / (1.0 + math.exp(-float(L.wbeta[h] @ u)))
        good &= np.allclose(S[h], b * np.outer(ka[h], va[h]), rtol=1e-12, atol=1e-15)
    return bool(good)


def test_beta_head_mapping():
    assert pin_beta_heads(ok.layer_forward)


def test_beta_head_mapping_mutant_reversed_rows():
    real = ok.layer_forward

    def layer(L, U, S, Z, **kw):
        return real(ok.OracleLayer(**{**L.__dict__, "wbeta": L.wbeta[::-1].copy()}), U, S, Z, **kw)
    assert not pin_beta_heads(layer)


# ----------------------------------------------------------------------------------------
# forget-gate variants: the lower-bounded ("safe") gate and the per-head scalar gate
# ----------------------------------------------------------------------------------------
def pin_safe_gate(gate_fn) -> bool:
    lb = -5.0
    # f = 0: sigmoid(0) = 1/2, alpha = exp(lb / 2)
    good = np.allclose(gate_fn(np.zeros((2, 3)), np.array([0.7, 2.0]), lb), math.exp(lb / 2), rtol=1e-15)
    # f a -> +inf: alpha -> 1; f a -> -inf: alpha -> e^lb
    good &= np.allclose(gate_fn(np.full((1, 2), 60.0), np.array([1.0]), lb), 1.0, rtol=1e-15)
    good &= np.allclose(gate_fn(np.full((1, 2), -60.0), np.array([1.0]), lb), math.exp(lb), rtol=1e-12)
    # per-head factor: head h at f = 1 gives exp(lb / (1 + e^{a_h})), libm scalars
    a = np.array([0.3, 1.5, -0.4])
    al = gate_fn(np.ones((3, 4)), a, lb)
    for h in range(3):
        good &= np.allclose(al[h], math.exp(lb / (1.0 + math.exp(a[h]))), rtol=1e-14)
    # bounds
    rng = RNG(21)
    al = gate_fn(rng.standard_normal((4, 16)) * 4, rng.uniform(0.1, 3, 4), lb)
    good &= bool(np.all((al > math.exp(lb)) & (al < 1)))
    return bool(good)


def test_safe_gate_pins():
    assert pin_safe_gate(ok.safe_gate)


def test_safe_gate_mutant_sign():
    def mutant(f, a, lb):
        return np.exp(lb * ok.sigmoid(f * a[:, None]))
    assert not pin_safe_gate(mutant)


def pin_scalar_gate(gate_fn) -> bool:
    dk = 5
    # softplus(0) = ln 2, exp(A_log = 0) = 1: alpha = 1/2 on every channel of the head
    good = np.allclose(gate_fn(np.zeros(2), np.zeros(2), dk), 0.5, rtol=1e-15)
    f = np.array([0.4, -1.2, 3.0])
    a_log = np.array([-0.5, 0.2, -1.0])
    al = gate_fn(f, a_log, dk)
    good &= al.shape == (3, dk)
    for h in range(3):
        sp = max(f[h], 0.0) + math.log1p(math.exp(-abs(f[h])))
        good &= np.allclose(al[h], math.exp(-math.exp(a_log[h]) * sp), rtol=1e-14)
    return bool(good)


def test_scalar_gate_pins():
    assert pin_scalar_gate(ok.scalar_gate)


def test_scalar_gate_mutant_head_order():
    def mutant(f, a_log, dk):
        return ok.scalar_gate(f, a_log[::-1].copy(), dk)
    assert not pin_scalar_gate(mutant)


def _gate_layer(gate, seed):
    d = synth.LayerDims(d_model=256, n_heads=2, d_k=64, d_v=64, rank_f=16, rank_g=16, gate=gate)
    w = synth.scaled(synth.WORKLOADS["tiny"], dims=d, steps=2, seed=seed)
    run = synth.draw_run(w)
    L = ok.prepare_layer(run.layers[0], "f32", 2, 64, 64, norm_eps=0.0, gate=gate, gate_lb=-5.0)
    return L, run


def pin_gate_variant_wiring(layer_fn, gate) -> bool:
    """As pin_forget_gate_wiring, for the other gate forms: with F_a = 0 the gate input is
    dt_bias exactly, and a beta = 1 token followed by a beta = 0 token gives
    S2 = diag(alpha) S1 with alpha from the gate's closed form (libm scalars): the safe gate
    per key channel exp(lb sigmoid(-dt_bias[h dk + i] a[h])), the scalar gate one value per
    head exp(-exp(A_log[h]) softplus(dt_bias[h]))."""
    L, run = _gate_layer(gate, 31)
    H, dk, dv = L.n_heads, L.d_k, L.d_v
    u1 = run.x[0, 0, 0].astype(np.float64)
    L.wbeta = np.tile(u1 / np.linalg.norm(u1), (H, 1)) * np.linspace(3e3, 5e3, H)[:, None]
    L.a_log = np.array([0.6, -0.8])
    L.fa = np.zeros_like(L.fa)
    U = np.stack([u1, -u1])
    _, S1, _ = layer_fn(L, U[:1], np.zeros((H, dk, dv)), np.zeros((3, L.channels)))
    _, S2, _ = layer_fn(L, U, np.zeros((H, dk, dv)), np.zeros((3, L.channels)))
    good = True
    for h in range(H):
        for i in range(dk):
            if gate == "safe":
                z = float(L.dt_bias[h * dk + i]) * float(L.a_log[h])
                a = math.exp(-5.0 / (1.0 + math.exp(z)))
            else:
                z = float(L.dt_bias[h])
                a = math.exp(-math.exp(float(L.a_log[h])) * (max(z, 0.0) + math.log1p(math.exp(-abs(z)))))
            good &= np.allclose(S2[h, i], a * S1[h, i], rtol=1e-12, atol=1e-15)
    return bool(good)


@pytest.mark.parametrize("gate", ["safe", "scalar"])
def test_gate_variant_wiring(gate):
    assert pin_gate_variant_wiring(ok.layer_forward, gate)


@pytest.mark.parametrize("gate", ["safe", "scalar"])
def test_gate_variant_wiring_mutant_kda_formula(gate):
    """Planted mistakes fail the pins: the KDA formula on the safe gate's input, and the
    scalar gate reading its heads' inputs in reverse order."""
    real = ok.layer_forward

    def layer(L, U, S, Z, **kw):
        if gate == "scalar":
            kv = dict(L.__dict__)
            kv.update(fb=L.fb[::-1].copy(), dt_bias=L.dt_bias[::-1].copy())
            return real(ok.OracleLayer(**kv), U, S, Z, **kw)
        return real(ok.OracleLayer(**{**L.__dict__, "gate": "kda"}), U, S, Z, **kw)
    assert not pin_gate_variant_wiring(layer, gate)


def test_scalar_gate_state_decays_uniformly():
    """With beta = 0 the scalar gate scales each head's whole state by one number: the
    ratio S2 / S1 is constant over the head (a per-channel gate would vary)."""
    L, run = _gate_layer("scalar", 32)
    H, dk, dv = L.n_heads, L.d_k, L.d_v
    L.wbeta = -1e4 * np.tile(np.sign(run.x[0, 0, 0]), (H, 1))     # beta logits << 0
    S0 = RNG(33).standard_normal((H, dk, dv))
    _, S1, _ = ok.layer_forward(L, run.x[:1, 0, 0].astype(np.float64), S0, np.zeros((3, L.channels)))
    for h in range(H):
        r = S1[h] / S0[h]
        assert np.allclose(r, r.flat[0], rtol=1e-12)
        assert 0 < r.flat[0] < 1
