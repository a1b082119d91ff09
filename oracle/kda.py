"""Plain float64 oracle of one KDA layer and of a pre-norm residual stack of them.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources, cited by page title and section:
  [TTK]  "Thirty tiny kernels per layer: a 16% decode win for GLM-5.3-Flash on Apple
         Silicon" (frederic.ai): the bulleted list under "Where the time goes" (the order
         of the decode step) and the pure step ``_decode_step_pure`` under "Why mx.compile
         fits here and not elsewhere" (q|k|v concatenation, conv input = window + current
         token, new window = last K-1 rows, SiLU, head split, q = l2norm * head_dim^-1/2,
         k = l2norm, gated delta update, o_norm with the output gate, o_proj).
  [LCPP] torad-labs/llama.cpp PR #84: the commit that fuses KDA's output gate (per head:
         RMS_NORM, MUL by the o_norm weight, then MUL by SIGMOID(gate)); the chunk_kda
         commit (per-key-channel log-decay; the recurrence that the chunked form chunks).
  [DS4]  antirez/ds4 PR #964: the commit that requantises KDA's BF16 projections to Q8_0
         (blocks of 32 int8 values with one fp16 scale), and the KDA recurrence-kernel
         commit (one A_log value per head).
  Workload text: the tiny single-layer workload defines the forget gate
         g = -exp(A_log) * softplus(f_b(f_a(x)) + dt_bias), alpha = exp(g) applied on the
         key dimension, beta = sigmoid(W_b x), the output gate sigmoid(g_b(g_a(x))) and
         RMSNorm eps = 1e-6.

Readings where the pages are silent:
  * state S[h] is [dk][dv], row = key channel; the update order is
      S' = diag(alpha) S ; delta = beta (v - S'^T k) ; S = S' + k delta^T ; o = S^T q
    (the output is read after the update).  This is the recurrence whose chunking the
    chunk_kda commit describes; tests/test_oracle_chunked.py checks that algebra.
  * conv tap 3 multiplies the current token, taps 0..2 the window (oldest first); SiLU is
    applied to all of q|k|v; no conv bias.
  * L2 norm: x / sqrt(sum x^2 + l2_eps) with l2_eps = 1e-6; the head_dim^-1/2 scale is
    applied to q only, after the norm.
  * the gated RMSNorm is per head over dv with weight ones; gate = sigmoid(g_b(g_a(u))).
  * Q8_0 (see q8_0_quantize).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------------------
# Weight formats
# ---------------------------------------------------------------------------------------
def bf16_round(a32: np.ndarray) -> np.ndarray:
    """Nearest BF16 value of each fp32 input, ties to the even mantissa; float64 out.

    Written from the definition: the two BF16 neighbours of x are its truncation toward
    zero (low 16 bits cleared) and the next BF16 value away from zero; take the nearer,
    and on a tie the one whose last kept mantissa bit is 0.  (Finite inputs only.)
    Pin: tests/test_oracle_formats.py (hand-worked ties, and torch's BF16 conversion)."""
    a = np.ascontiguousarray(a32, dtype=np.float32)
    bits = a.view(np.uint32)
    trunc_bits = bits & np.uint32(0xFFFF0000)
    up_bits = trunc_bits + np.uint32(0x10000)
    lo = trunc_bits.view(np.float32).astype(np.float64)
    hi = up_bits.view(np.float32).astype(np.float64)
    x = a.astype(np.float64)
    d_lo = np.abs(x - lo)
    d_hi = np.abs(hi - x)
    lo_even = ((trunc_bits >> np.uint32(16)) & np.uint32(1)) == 0
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & lo_even)
    return np.where(pick_lo, lo, hi)


def q8_0_quantize(w32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Q8_0 quantisation of a [rows][cols] fp32 matrix, cols % 32 == 0 ([DS4], Q8_0
    requantisation commit: blocks of 32 weights, one fp16 scale each).

    Per block of 32 consecutive values along a row (the rounding rules are this
    library's reading; the pages give only the format):
      amax = max |x_i|                         (fp32, exact)
      d    = amax / 127                        (fp32, correctly rounded)
      d16  = fp16(d), round to nearest even
      q_i  = clamp(round_half_away(x_i / float(d16)), -127, 127), the division in fp32
             correctly rounded; if d16 == 0 every q_i = 0.
    Returns (d16 as float16 [rows][cols/32], q as int8 [rows][cols]).
    Pins: |x - d16 q| <= d16/2; the amax element maps to +-127; hand-worked block in
    tests/golden/q8_0_block.txt; d16 is the nearest fp16 of d."""
    x = np.ascontiguousarray(w32, dtype=np.float32)
    rows, cols = x.shape
    if cols % 32:
        raise ValueError("Q8_0 needs cols % 32 == 0")
    blocks = x.reshape(rows, cols // 32, 32)
    amax = np.max(np.abs(blocks), axis=-1)
    d = (amax / np.float32(127.0)).astype(np.float32)
    d16 = d.astype(np.float16)
    dq = d16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (blocks / dq[..., None]).astype(np.float32)
    v64 = v.astype(np.float64)
    r = np.sign(v64) * np.floor(np.abs(v64) + 0.5)       # exact in float64
    r = np.where((dq == 0)[..., None], 0.0, r)
    q = np.clip(r, -127, 127).astype(np.int8)
    return d16, q.reshape(rows, cols)


def q8_0_dequantize(d16: np.ndarray, q: np.ndarray) -> np.ndarray:
    rows, cols = q.shape
    d = d16.astype(np.float64).reshape(rows, cols // 32, 1)
    return (d * q.astype(np.float64).reshape(rows, cols // 32, 32)).reshape(rows, cols)


# The E2M1 element grid of MXFP4 (non-negative half; sign separate): exponent bits e and
# mantissa bit m give 0.5 m for e = 0 and 2^(e-1) (1 + m/2) otherwise.
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mxfp4_quantize(w32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP4 quantisation of a [rows][cols] fp32 matrix, cols % 32 == 0.

    MXFP4 is one of the block formats the quant-format commit of torad-labs/llama.cpp PR
    #84 ranks at the KDA projection shapes; its definition is the OCP Microscaling (MX)
    format specification v1.0: blocks of 32 consecutive values along a row share one
    E8M0 scale X = 2^s, s = floor(log2(max|x|)) - 2 (2 = the exponent of E2M1's largest
    normal), clamped to [-127, 127]; each element is the E2M1 value nearest to x / X, ties
    to the even mantissa bit, clamped to +-6 (the largest E2M1 value).  A block of zeros
    takes s = -127 and zero elements.
    Returns (e8m0 = s + 127 as uint8 [rows][cols/32], codes as uint8 [rows][cols] with
    code = sign << 3 | index into E2M1_GRID).
    Pins: values on the grid times X come back exactly; |x - q| <= X/4 below 4 X, <= X
    between 4 X and 6 X (the grid's spacing halves), and the saturation of (6 X, 8 X);
    hand-worked ties."""
    x = np.ascontiguousarray(w32, dtype=np.float32).astype(np.float64)
    rows, cols = x.shape
    if cols % 32:
        raise ValueError("MXFP4 needs cols % 32 == 0")
    blocks = x.reshape(rows, cols // 32, 32)
    amax = np.max(np.abs(blocks), axis=-1)
    _, ex = np.frexp(amax)                       # amax = m 2^ex, m in [0.5, 1)
    s = np.where(amax > 0, ex - 1 - 2, -127)
    s = np.clip(s, -127, 127)
    v = blocks / np.exp2(s)[..., None]           # exact: a power-of-two scale
    a = np.minimum(np.abs(v), 6.0)
    # nearest grid point; on a tie the even index (mantissa bit 0): E2M1_GRID index i has
    # mantissa bit i & 1
    d = np.abs(a[..., None] - E2M1_GRID)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    odd = (np.arange(8) & 1) == 1
    idx = np.where(cand & ~odd, np.arange(8), 99).min(axis=-1)
    idx = np.where(idx == 99, np.argmax(cand, axis=-1), idx)
    sign = (v < 0) & (idx > 0)
    codes = (sign.astype(np.uint8) << 3) | idx.astype(np.uint8)
    return (s + 127).astype(np.uint8), codes.reshape(rows, cols)


def mxfp4_dequantize(e8m0: np.ndarray, codes: np.ndarray) -> np.ndarray:
    rows, cols = codes.shape
    mag = E2M1_GRID[codes & 7]
    val = np.where(codes & 8, -mag, mag).reshape(rows, cols // 32, 32)
    return (val * np.exp2(e8m0.astype(np.float64) - 127.0)[..., None]).reshape(rows, cols)


PROJECTIONS = ("wq", "wk", "wv", "wo", "fa", "fb", "wbeta", "ga", "gb")


@dataclasses.dataclass
class OracleLayer:
    """One layer's parameters in float64, after the weight format was applied."""
    d_model: int
    n_heads: int
    d_k: int
    d_v: int
    conv_k: int
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    fa: np.ndarray
    fb: np.ndarray
    wbeta: np.ndarray
    ga: np.ndarray
    gb: np.ndarray
    conv_w: np.ndarray     # [C][conv_k]
    a_log: np.ndarray      # [H]
    dt_bias: np.ndarray    # [H*dk]
    o_norm_w: np.ndarray   # [dv]
    norm_eps: float = 1e-6
    l2_eps: float = 1e-6
    gate: str = "kda"      # forget-gate form: kda | safe | scalar (see forget_alpha)
    gate_lb: float = -5.0  # lower bound of log(alpha) of the safe gate

    @property
    def channels(self) -> int:
        return 2 * self.n_heads * self.d_k + self.n_heads * self.d_v


def prepare_layer(draws: Dict[str, np.ndarray], wtype: str, n_heads: int, d_k: int,
                  d_v: int, norm_eps: float = 1e-6, l2_eps: float = 1e-6, gate: str = "kda",
                  gate_lb: float = -5.0) -> OracleLayer:
    """Apply the projection weight format (f32 | bf16 | q8_0 | mxfp4) to fp32 draws."""
    def fmt(w):
        if wtype == "f32":
            return np.asarray(w, np.float32).astype(np.float64)
        if wtype == "bf16":
            return bf16_round(w)
        if wtype == "q8_0":
            return q8_0_dequantize(*q8_0_quantize(w))
        if wtype == "mxfp4":
            return mxfp4_dequantize(*mxfp4_quantize(w))
        raise ValueError(wtype)

    mats = {k: fmt(draws[k]) for k in PROJECTIONS}
    d_model = mats["wq"].shape[1]
    return OracleLayer(
        d_model=d_model, n_heads=n_heads, d_k=d_k, d_v=d_v,
        conv_k=draws["conv_w"].shape[1],
        conv_w=draws["conv_w"].astype(np.float64),
        a_log=draws["a_log"].astype(np.float64),
        dt_bias=draws["dt_bias"].astype(np.float64),
        o_norm_w=np.ones(d_v, np.float64),
        norm_eps=norm_eps, l2_eps=l2_eps, gate=gate, gate_lb=gate_lb, **mats)


# ---------------------------------------------------------------------------------------
# Elementwise functions (float64, libm)
# ---------------------------------------------------------------------------------------
def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(y):
    return y / (1.0 + np.exp(-y))


def softplus(z):
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def rms_norm(x, w, eps):
    """x / sqrt(mean(x^2) + eps) * w along the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def l2_normalize(x, eps):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


# ---------------------------------------------------------------------------------------
# The steps of one token, each a function of its own so each can be pinned
# ---------------------------------------------------------------------------------------
def conv_silu(Z: np.ndarray, p: np.ndarray, w: np.ndarray):
    """Causal depthwise conv over (window, current token), then SiLU; rolls the window.

    Z: [K-1][C] oldest first, p: [C] current token, w: [C][K] with tap K-1 on the
    current token.  Returns (a [C], Z' = Z[1:] + [p])  ([TTK] pure step: conv input =
    window || current, new window = its last K-1 rows).
    Pins: identity kernel [0,..,0,1] gives SiLU(p); an impulse walks back through the
    taps; the window is a pure copy."""
    y = np.sum(w[:, :-1].T * Z, axis=0) + w[:, -1] * p
    return silu(y), np.concatenate([Z[1:], p[None, :]], axis=0)


def split_heads(a: np.ndarray, H: int, dk: int, dv: int, l2_eps: float):
    """q | k | v channels (head-major inside each) -> per-head q, k (L2-normalised, q
    also scaled by dk^-1/2) and v  ([TTK] pure step).  Pin: ||k_h|| = 1, ||q_h|| = dk^-1/2."""
    K = H * dk
    q = l2_normalize(a[:K].reshape(H, dk), l2_eps) * (dk ** -0.5)
    k = l2_normalize(a[K:2 * K].reshape(H, dk), l2_eps)
    v = a[2 * K:2 * K + H * dv].reshape(H, dv)
    return q, k, v


def forget_gate(f: np.ndarray, a_log: np.ndarray) -> np.ndarray:
    """alpha = exp(-exp(A_log[h]) * softplus(f[h, i]))  (workload text).  f: [H][dk].
    Pins: softplus(0) = ln 2 closed form; alpha in (0, 1]; A_log -> -inf gives 1."""
    return np.exp(-np.exp(a_log)[:, None] * softplus(f))


def safe_gate(f: np.ndarray, a: np.ndarray, lb: float) -> np.ndarray:
    """The lower-bounded ("safe") forget gate: alpha = exp(lb * sigmoid(-f * a[h])) per key
    channel, with a per-head factor a used as given and lb < 0, so log(alpha) lies in
    (lb, 0)  (torad-labs/llama.cpp PR #84, the decay-precompute commit, which writes the KDA
    decay as exp(raw_lb * sigmoid(-(g * raw_a[h]))); "Thirty tiny kernels per layer" lists
    the "safe gate" transform among the step's parts).  f: [H][dk].
    Pins: f = 0 gives exp(lb / 2); the bounds e^lb < alpha < 1; a closed form per head."""
    return np.exp(lb * sigmoid(-f * a[:, None]))


def scalar_gate(f: np.ndarray, a_log: np.ndarray, dk: int) -> np.ndarray:
    """The gated delta rule's scalar gate: one alpha per head,
    alpha_h = exp(-exp(A_log[h]) * softplus(f_h)), applied to every key channel of the head
    (the chunk_kda commit of torad-labs/llama.cpp PR #84 contrasts it with KDA's gate "one
    per key channel").  f: [H].  Returns [H][dk].
    Pins: constant along a head's channels; softplus(0) = ln 2 closed form; layer wiring."""
    a = np.exp(-np.exp(a_log) * softplus(f))
    return np.repeat(a[:, None], dk, axis=1)


def forget_alpha(L: "OracleLayer", f: np.ndarray) -> np.ndarray:
    """alpha [H][dk] of one token from the forget-gate input f = F_b F_a u + dt_bias
    ([H*dk], or [H] for the scalar gate) in the layer's gate form."""
    H, dk = L.n_heads, L.d_k
    if L.gate == "kda":
        return forget_gate(f.reshape(H, dk), L.a_log)
    if L.gate == "safe":
        return safe_gate(f.reshape(H, dk), L.a_log, L.gate_lb)
    if L.gate == "scalar":
        return scalar_gate(f.reshape(H), L.a_log, dk)
    raise ValueError(L.gate)


def delta_rule_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    alpha: np.ndarray, beta: np.ndarray):
    """Gated delta rule for every head.  S: [H][dk][dv] (row = key channel), q, k, alpha:
    [H][dk], v: [H][dv], beta: [H].  Returns (S_new, o):
        S' = diag(alpha) S ; delta = beta (v - S'^T k) ; S_new = S' + k delta^T ;
        o = S_new^T q.
    Pins: brute force S_T = prod((I - b k k^T) diag(alpha)) S_0 + ...; beta = 1 with unit
    k maps k to v; alpha = 1, beta = 0 leaves S unchanged; fp64 chunked form agrees."""
    S1 = alpha[:, :, None] * S
    e = np.einsum("hij,hi->hj", S1, k)
    delta = beta[:, None] * (v - e)
    S_new = S1 + k[:, :, None] * delta[:, None, :]
    o = np.einsum("hij,hi->hj", S_new, q)
    return S_new, o


def gated_norm(o: np.ndarray, gate: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Per head: RMSNorm over dv with weight w, then times gate  ([LCPP] output-gate
    commit: RMS_NORM, MUL(o_norm), MUL(SIGMOID(gate)), per head).  Pin: with w = 1 and
    gate = 1 every head has RMS 1 (up to eps)."""
    return rms_norm(o, w, eps) * gate


# ---------------------------------------------------------------------------------------
# One layer over a block of tokens of one sequence
# ---------------------------------------------------------------------------------------
def layer_forward(L: OracleLayer, U: np.ndarray, S: np.ndarray, Z: np.ndarray,
                  keep_after: Optional[int] = None, trace: Optional[dict] = None):
    """Run tokens U [T][D] (layer inputs) of one sequence through one layer, in order.

    S: [H][dk][dv] state, Z: [conv_k-1][C] conv window (oldest first).  Returns
    (out [T][D], S_end, Z_end) where S_end/Z_end are the state after ``keep_after``
    tokens (default: all T).  Projections of all T tokens are computed first (they do
    not depend on the recurrence); the conv, gates and delta rule then run token by
    token ([TTK] step list and pure step)."""
    U = np.atleast_2d(np.asarray(U, np.float64))
    T = U.shape[0]
    H, dk, dv = L.n_heads, L.d_k, L.d_v
    keep = T if keep_after is None else int(keep_after)
    # q, k, v projections, concatenated q | k | v
    P = np.concatenate([U @ L.wq.T, U @ L.wk.T, U @ L.wv.T], axis=1)    # [T][C]
    # forget-gate input, beta, output gate
    F = (U @ L.fa.T) @ L.fb.T + L.dt_bias                   # [T][H*dk] (scalar gate: [T][H])
    Bt = sigmoid(U @ L.wbeta.T)                                         # [T][H]
    G = sigmoid((U @ L.ga.T) @ L.gb.T)                                  # [T][H*dv]

    S = np.array(S, np.float64, copy=True)
    Z = np.array(Z, np.float64, copy=True)
    S_keep, Z_keep = (S.copy(), Z.copy()) if keep == 0 else (None, None)
    N = np.empty((T, H * dv))
    for t in range(T):
        a, Z = conv_silu(Z, P[t], L.conv_w)
        q, k, v = split_heads(a, H, dk, dv, L.l2_eps)
        alpha = forget_alpha(L, F[t])
        S, o = delta_rule_step(S, q, k, v, alpha, Bt[t])
        n = gated_norm(o, G[t].reshape(H, dv), L.o_norm_w, L.norm_eps)
        N[t] = n.reshape(-1)
        if trace is not None:
            for name, val in (("p", P[t]), ("a", a), ("q", q), ("k", k), ("v", v),
                              ("alpha", alpha), ("beta", Bt[t]), ("o", o), ("n", n)):
                trace.setdefault(name, []).append(np.array(val))
        if t + 1 == keep:
            S_keep, Z_keep = S.copy(), Z.copy()
    out = N @ L.wo.T
    return out, S_keep, Z_keep


def layer_step(L: OracleLayer, u: np.ndarray, S: np.ndarray, Z: np.ndarray):
    """One token: (u [D], S, Z) -> (out [D], S', Z')  ([TTK] pure decode step)."""
    out, S2, Z2 = layer_forward(L, np.asarray(u)[None, :], S, Z)
    return out[0], S2, Z2


def stack_step(layers: Sequence[OracleLayer], X: np.ndarray, S: List[np.ndarray],
               Z: List[np.ndarray], keep_after: Optional[int] = None, eps: float = 1e-6):
    """Tokens X [T][D] of one sequence through the pre-norm residual stack
    x_{l+1} = x_l + layer_l(RMSNorm(x_l)) (RMSNorm weight ones).  Returns
    (x_final [T][D], S list, Z list) with the states after ``keep_after`` tokens."""
    X = np.array(np.atleast_2d(X), np.float64, copy=True)
    S_out, Z_out = [], []
    for l, L in enumerate(layers):
        h = rms_norm(X, 1.0, eps)
        out, s2, z2 = layer_forward(L, h, S[l], Z[l], keep_after=keep_after)
        X = X + out
        S_out.append(s2)
        Z_out.append(z2)
    return X, S_out, Z_out


# ---------------------------------------------------------------------------------------
# Runs over a whole workload
# ---------------------------------------------------------------------------------------
def decode_run(layers: Sequence[OracleLayer], x: np.ndarray, s0: np.ndarray,
               prenorm_residual: bool, steps: Optional[int] = None,
               check_every: int = 0):
    """Decode ``steps`` tokens for every sequence.  x: [steps][B][1][D]; s0:
    [n_layers][B][H][dk][dv].  Returns (y [steps][B][D], S [n_layers][B][H][dk][dv],
    Z [n_layers][B][conv_k-1][C], snapshots {step: S}) where y is the layer output
    (single layer) or the final residual stream (stack)."""
    n_l = len(layers)
    steps = x.shape[0] if steps is None else steps
    Bsz = x.shape[1]
    C = layers[0].channels
    kc = layers[0].conv_k - 1
    S = [[np.array(s0[l, b], np.float64) for b in range(Bsz)] for l in range(n_l)]
    Z = [[np.zeros((kc, C)) for _ in range(Bsz)] for _ in range(n_l)]
    ys = np.empty((steps, Bsz, layers[0].d_model))
    snaps = {}
    for t in range(steps):
        for b in range(Bsz):
            xt = x[t, b, 0].astype(np.float64)[None, :]
            if prenorm_residual:
                y, s_new, z_new = stack_step(layers, xt, [S[l][b] for l in range(n_l)],
                                             [Z[l][b] for l in range(n_l)])
            else:
                y, s1, z1 = layer_forward(layers[0], xt, S[0][b], Z[0][b])
                s_new, z_new = [s1], [z1]
            ys[t, b] = y[0]
            for l in range(n_l):
                S[l][b], Z[l][b] = s_new[l], z_new[l]
        if check_every and (t + 1) % check_every == 0:
            snaps[t + 1] = np.array([[S[l][b] for b in range(Bsz)] for l in range(n_l)])
    S_arr = np.array([[S[l][b] for b in range(Bsz)] for l in range(n_l)])
    Z_arr = np.array([[Z[l][b] for b in range(Bsz)] for l in range(n_l)])
    return ys, S_arr, Z_arr, snaps


def verify_run(layers: Sequence[OracleLayer], x: np.ndarray, s0: np.ndarray,
               accept: np.ndarray, steps: Optional[int] = None):
    """Multi-token verify with rollback.  x: [steps][B][T][D]; accept: [steps][B] in 1..T.

    Each step runs all T tokens of every sequence through the stack from the committed
    state (every output is recorded, accepted or not), then commits the state and conv
    window reached after accept[step][b] tokens (read-only verify followed by a commit
    after k tokens, as in the gdn_step verify/commit modes of the regolith GDN audit).
    Returns (y [steps][B][T][D], S, Z) with the final committed state."""
    n_l = len(layers)
    steps = x.shape[0] if steps is None else steps
    Bsz, T = x.shape[1], x.shape[2]
    C = layers[0].channels
    kc = layers[0].conv_k - 1
    S = [[np.array(s0[l, b], np.float64) for b in range(Bsz)] for l in range(n_l)]
    Z = [[np.zeros((kc, C)) for _ in range(Bsz)] for _ in range(n_l)]
    ys = np.empty((steps, Bsz, T, layers[0].d_model))
    for t in range(steps):
        for b in range(Bsz):
            y, s_new, z_new = stack_step(layers, x[t, b].astype(np.float64),
                                         [S[l][b] for l in range(n_l)],
                                         [Z[l][b] for l in range(n_l)],
                                         keep_after=int(accept[t, b]))
            ys[t, b] = y
            for l in range(n_l):
                S[l][b], Z[l][b] = s_new[l], z_new[l]
    S_arr = np.array([[S[l][b] for b in range(Bsz)] for l in range(n_l)])
    Z_arr = np.array([[Z[l][b] for b in range(Bsz)] for l in range(n_l)])
    return ys, S_arr, Z_arr


def prefill_run(layer: OracleLayer, x: np.ndarray, s0: np.ndarray, tokens: Optional[int] = None,
                seqs: Optional[Sequence[int]] = None):
    """Sequential token-by-token prefill of one layer.  x: [B][L][D]; s0: [B][H][dk][dv].
    Returns (y [nb][L][D], S [nb][H][dk][dv], Z [nb][conv_k-1][C]) for the selected
    sequences (default all) over the first ``tokens`` tokens (default all)."""
    seqs = range(x.shape[0]) if seqs is None else seqs
    Lt = x.shape[1] if tokens is None else tokens
    C = layer.channels
    kc = layer.conv_k - 1
    ys, Ss, Zs = [], [], []
    for b in seqs:
        y, s, z = layer_forward(layer, x[b, :Lt].astype(np.float64), s0[b], np.zeros((kc, C)))
        ys.append(y)
        Ss.append(s)
        Zs.append(z)
    return np.array(ys), np.array(Ss), np.array(Zs)
