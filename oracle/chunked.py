"""Float64 chunked (WY/UT) form of the gated delta rule with a per-key-channel gate.

TEST INFRASTRUCTURE ONLY.  This is not the oracle of the prefill path (that is the
sequential ``kda.layer_forward``); it exists so that a test can show that the
sequential recurrence the oracle uses is exactly the recurrence whose chunking the
chunk_kda commit of torad-labs/llama.cpp PR #84 describes:

  * G = the inclusive sum of each key channel's log-decay along the chunk;
  * L[t][s] = beta_t * sum_i k_t[i] k_s[i] exp(G_t[i] - G_s[i])      (s < t);
  * the masked A[t][s] = sum_i q_t[i] k_s[i] exp(G_t[i] - G_s[i])     (s <= t);
  * solve (I + L) x = b for b = beta exp(G) k and for b = beta v;
  * q scaled by exp(G_t), k by exp(G_last - G_t), each state row k decayed by
    exp(G_last[k]) at the chunk end.

Per chunk and head, with S the state at the chunk start ([dk][dv], row = key channel):
  W = (I+L)^-1 (beta exp(G) k),  U = (I+L)^-1 (beta v),  D = U - W S
  o_t = (exp(G_t) q_t) S + sum_{s<=t} A[t][s] D_s
  S_end = diag(exp(G_last)) S + sum_s (exp(G_last - G_s) k_s) D_s^T
"""
from __future__ import annotations

import numpy as np


def chunked_delta_rule(q, k, v, log_alpha, beta, S0, chunk: int):
    """q, k, log_alpha: [T][dk]; v: [T][dv]; beta: [T]; S0: [dk][dv].  One head.
    Returns (o [T][dv], S_end).  The last chunk may be partial."""
    T = q.shape[0]
    S = np.array(S0, np.float64, copy=True)
    o = np.empty((T, v.shape[1]))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        qc, kc, vc = q[c0:c1], k[c0:c1], v[c0:c1]
        bc = beta[c0:c1]
        G = np.cumsum(log_alpha[c0:c1], axis=0)                     # inclusive, <= 0
        n = c1 - c0
        decay = np.exp(G[:, None, :] - G[None, :, :])               # [t][s][i]
        KK = np.einsum("ti,si,tsi->ts", kc, kc, decay)
        QK = np.einsum("ti,si,tsi->ts", qc, kc, decay)
        Lm = np.tril(bc[:, None] * KK, -1)
        Am = np.tril(QK, 0)
        I = np.eye(n)
        W = np.linalg.solve(I + Lm, bc[:, None] * np.exp(G) * kc)
        U = np.linalg.solve(I + Lm, bc[:, None] * vc)
        Dm = U - W @ S
        o[c0:c1] = (np.exp(G) * qc) @ S + Am @ Dm
        g_last = G[-1]
        S = np.exp(g_last)[:, None] * S + (np.exp(g_last[None, :] - G) * kc).T @ Dm
    return o, S
