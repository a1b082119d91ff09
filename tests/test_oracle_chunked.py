"""The sequential recurrence of the oracle equals the chunk_kda WY/UT form (float64).

The chunked form (oracle/chunked.py) is written from the chunk_kda commit of
torad-labs/llama.cpp PR #84; agreement to ~1e-12 at chunk sizes 16 and 64, with a
partial last chunk and with per-channel slow/fast gates (so state really crosses chunk
boundaries), pins the oracle's update order: decay, error against the decayed state,
rank-1 update, read-out after the update.
"""
import numpy as np
import pytest

import synth
from oracle import kda as ok
from oracle.chunked import chunked_delta_rule


def _sequential(q, k, v, log_alpha, beta, S0):
    S = S0[None].copy()
    outs = []
    for t in range(q.shape[0]):
        S, o = ok.delta_rule_step(S, q[t][None], k[t][None], v[t][None],
                                  np.exp(log_alpha[t])[None], np.array([beta[t]]))
        outs.append(o[0])
    return np.array(outs), S[0]


def _inputs(T, dk, dv, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True) * np.sqrt(dk)
    v = rng.standard_normal((T, dv))
    g = synth.kda_decay_gate_inputs(rng, T, 1, dk)[:, 0]
    beta = rng.uniform(0.05, 0.95, T)
    S0 = rng.standard_normal((dk, dv)) * 0.1
    return q, k, v, g, beta, S0


@pytest.mark.parametrize("chunk", [16, 64])
def test_chunked_equals_sequential(chunk):
    q, k, v, g, beta, S0 = _inputs(T=150, dk=32, dv=24, seed=chunk)
    o_seq, S_seq = _sequential(q, k, v, g, beta, S0)
    o_chk, S_chk = chunked_delta_rule(q, k, v, g, beta, S0, chunk)
    scale = np.abs(o_seq).max()
    assert np.abs(o_chk - o_seq).max() / scale < 1e-11
    assert np.abs(S_chk - S_seq).max() < 1e-11


def test_gate_generator_carries_state_across_chunks():
    """With per-channel rates some channels keep > 1e-3 of their state over 16 tokens."""
    g = synth.kda_decay_gate_inputs(np.random.default_rng(0), 16, 4, 128)
    carried = np.exp(g.sum(axis=0))
    assert (carried > 1e-3).mean() > 0.3


def test_chunk_mutant_neighbour_channel_decay_fails():
    """Decaying each state row by its neighbour channel's G_last at chunk ends must break
    the agreement (a planted mistake in the chunked form, on the CPU)."""
    q, k, v, g, beta, S0 = _inputs(T=96, dk=32, dv=24, seed=3)
    o_seq, S_seq = _sequential(q, k, v, g, beta, S0)
    import oracle.chunked as oc
    src_fn = oc.chunked_delta_rule

    def mutant(q, k, v, log_alpha, beta, S0, chunk):
        T = q.shape[0]
        S = S0.copy()
        o = np.empty((T, v.shape[1]))
        for c0 in range(0, T, chunk):
            c1 = min(T, c0 + chunk)
            o_c, S_next = src_fn(q[c0:c1], k[c0:c1], v[c0:c1], log_alpha[c0:c1], beta[c0:c1], S, c1 - c0)
            G_last = np.cumsum(log_alpha[c0:c1], axis=0)[-1]
            fix = np.exp(np.roll(G_last, 1) - G_last)[:, None]
            S = S_next + (fix - 1) * np.exp(G_last)[:, None] * S
            o[c0:c1] = o_c
        return o, S
    o_m, S_m = mutant(q, k, v, g, beta, S0, 16)
    assert np.abs(S_m - S_seq).max() > 1e-4
