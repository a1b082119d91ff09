"""Seeded synthetic inputs for the KDA decode / verify / prefill workloads.

This module is shared by the CPU oracle, the tests, the benchmark and the HIP
binding's callers.  It holds NO arithmetic of the method: it only draws random
numbers with numpy's PCG64 generator, scales them by the stated standard
deviation, and (for inputs that the workload defines as BF16) rounds them to
BF16 with round-to-nearest-even so that every consumer sees the same bytes.
Quantisation of weights to Q8_0 and conversion of weights to BF16 are steps of
the method; each side (oracle, GPU packer) does those itself from the fp32
draws produced here.

Workloads (sizes from the gated-delta-rule / Kimi Delta Attention decode
workloads this library targets; "N(0, s)" means standard deviation s):

  tiny     single layer, D=256, H=2, dk=dv=64, fp32 weights, 16 decode steps
  layer    single layer, D=2048, H=16, dk=dv=128, BF16 weights, 256 steps
  stack    34 layers as "layer" with Q8_0 weights, pre-RMSNorm + residual,
           B=1, 128 steps
  verify   the "stack" model, B=8 sequences, T=4 tokens a step, 64 steps,
           accept lengths uniform in 1..T
  prefill  one "layer" layer, B=4, L=8192, chunk 64, S0=0
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

F32, BF16, Q8_0 = "f32", "bf16", "q8_0"

# Fixed draw order per layer (one generator per run, see draw_run()).
WEIGHT_ORDER = ("wq", "wk", "wv", "wo", "fa", "fb", "wbeta", "ga", "gb",
                "conv_w", "a_log", "dt_bias")


@dataclasses.dataclass(frozen=True)
class LayerDims:
    d_model: int
    n_heads: int
    d_k: int
    d_v: int
    rank_f: int
    rank_g: int
    conv_k: int = 4
    # forget-gate form: "kda" (per key channel), "safe" (per key channel, lower-bounded),
    # "scalar" (one gate per head: F_b is [H][rank_f] and dt_bias [H])
    gate: str = "kda"

    @property
    def key_dim(self) -> int:
        return self.n_heads * self.d_k

    @property
    def value_dim(self) -> int:
        return self.n_heads * self.d_v

    @property
    def conv_channels(self) -> int:
        return 2 * self.key_dim + self.value_dim

    def shapes(self) -> Dict[str, tuple]:
        """[out][in] row-major shapes of every per-layer parameter."""
        D, K, V = self.d_model, self.key_dim, self.value_dim
        FR = self.n_heads if self.gate == "scalar" else K     # forget-gate rows
        return {
            "wq": (K, D), "wk": (K, D), "wv": (V, D), "wo": (D, V),
            "fa": (self.rank_f, D), "fb": (FR, self.rank_f),
            "wbeta": (self.n_heads, D),
            "ga": (self.rank_g, D), "gb": (V, self.rank_g),
            "conv_w": (self.conv_channels, self.conv_k),
            "a_log": (self.n_heads,), "dt_bias": (FR,),
        }


@dataclasses.dataclass(frozen=True)
class WeightStd:
    qkvo: float
    fa: float
    fb: float
    wbeta: float
    ga: float
    gb: float
    conv: float = 0.5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: LayerDims
    wtype: str            # f32 | bf16 | q8_0  (projection weight format)
    std: WeightStd
    n_layers: int
    prenorm_residual: bool
    batch: int
    steps: int            # decode / verify steps (prefill: 1)
    tokens: int           # tokens per step per sequence (T for verify, L for prefill)
    s0_std: float         # 0 => S0 = 0
    x_bf16: bool          # inputs rounded to BF16
    seed: int
    chunk: int = 0        # prefill chunk size
    norm_eps: float = 1e-6
    l2_eps: float = 1e-6
    gate_lb: float = -5.0  # lower bound of log(alpha) for the "safe" gate form


def _tiny() -> Workload:
    d = LayerDims(d_model=256, n_heads=2, d_k=64, d_v=64, rank_f=16, rank_g=16)
    s = 1.0 / np.sqrt(256.0)
    std = WeightStd(qkvo=s, fa=s, fb=1.0 / np.sqrt(16.0), wbeta=s, ga=s,
                    gb=1.0 / np.sqrt(16.0))
    return Workload("tiny", d, F32, std, n_layers=1, prenorm_residual=False,
                    batch=1, steps=16, tokens=1, s0_std=0.0, x_bf16=False, seed=0)


_BIG = LayerDims(d_model=2048, n_heads=16, d_k=128, d_v=128, rank_f=128, rank_g=128)
_STD02 = WeightStd(qkvo=0.02, fa=0.02, fb=0.02, wbeta=0.02, ga=0.02, gb=0.02)

WORKLOADS: Dict[str, Workload] = {
    "tiny": _tiny(),
    "layer": Workload("layer", _BIG, BF16, _STD02, n_layers=1, prenorm_residual=False,
                      batch=1, steps=256, tokens=1, s0_std=0.1, x_bf16=True, seed=1),
    "stack": Workload("stack", _BIG, Q8_0, _STD02, n_layers=34, prenorm_residual=True,
                      batch=1, steps=128, tokens=1, s0_std=0.1, x_bf16=True, seed=2),
    "verify": Workload("verify", _BIG, Q8_0, _STD02, n_layers=34, prenorm_residual=True,
                       batch=8, steps=64, tokens=4, s0_std=0.1, x_bf16=True, seed=3),
    "prefill": Workload("prefill", _BIG, BF16, _STD02, n_layers=1, prenorm_residual=False,
                        batch=4, steps=1, tokens=8192, s0_std=0.0, x_bf16=True, seed=4,
                        chunk=64),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller test sizes)."""
    return dataclasses.replace(w, **changes)


# ----------------------------------------------------------------------------------------
# BF16 input rounding (round-to-nearest-even), used only for inputs that the workload
# defines as BF16.  Returns (fp32 values that are exactly BF16, uint16 bit patterns).
# ----------------------------------------------------------------------------------------
def to_bf16(a: np.ndarray):
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded[nan] = 0x7FC0
    vals = (rounded.astype(np.uint32) << 16).view(np.float32)
    return vals, rounded


def _normal(rng, shape, std) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)


def draw_layer(rng: np.random.Generator, w: Workload) -> Dict[str, np.ndarray]:
    """fp32 draws of one layer's parameters, in WEIGHT_ORDER."""
    shp = w.dims.shapes()
    sd = w.std
    stds = {"wq": sd.qkvo, "wk": sd.qkvo, "wv": sd.qkvo, "wo": sd.qkvo,
            "fa": sd.fa, "fb": sd.fb, "wbeta": sd.wbeta, "ga": sd.ga, "gb": sd.gb,
            "conv_w": sd.conv}
    out: Dict[str, np.ndarray] = {}
    for name in WEIGHT_ORDER:
        if name == "a_log":
            out[name] = rng.uniform(-1.0, 0.0, size=shp[name]).astype(np.float32)
        elif name == "dt_bias":
            out[name] = rng.uniform(-1.0, 1.0, size=shp[name]).astype(np.float32)
        else:
            out[name] = _normal(rng, shp[name], stds[name])
    return out


@dataclasses.dataclass
class RunInputs:
    workload: Workload
    layers: List[Dict[str, np.ndarray]]   # fp32 draws per layer
    s0: np.ndarray                        # [n_layers][batch][H][dk][dv] fp32
    x: np.ndarray                         # [steps][batch][tokens][D] fp32 (BF16-exact if x_bf16)
    x_bits: Optional[np.ndarray]          # uint16 BF16 bits of x, or None
    accept: Optional[np.ndarray]          # [steps][batch] int32 in 1..tokens (verify only)


def draw_run(w: Workload) -> RunInputs:
    """Every input of a workload, drawn from one PCG64 stream seeded with w.seed, in the
    order: per layer the weights (WEIGHT_ORDER), then S0 for every layer, then the
    token inputs, then (verify) the accept lengths."""
    rng = np.random.default_rng(w.seed)
    d = w.dims
    layers = [draw_layer(rng, w) for _ in range(w.n_layers)]
    s_shape = (w.n_layers, w.batch, d.n_heads, d.d_k, d.d_v)
    if w.s0_std > 0:
        s0 = _normal(rng, s_shape, w.s0_std)
    else:
        s0 = np.zeros(s_shape, np.float32)
    x = rng.standard_normal(size=(w.steps, w.batch, w.tokens, d.d_model), dtype=np.float32)
    bits = None
    if w.x_bf16:
        x, bits = to_bf16(x)
    accept = None
    if w.name.startswith("verify") or (w.tokens > 1 and w.chunk == 0):
        accept = rng.integers(1, w.tokens + 1, size=(w.steps, w.batch)).astype(np.int32)
    return RunInputs(w, layers, s0, x, bits, accept)


def kda_decay_gate_inputs(rng: np.random.Generator, tokens: int, heads: int, dk: int,
                          lo: float = 0.02, hi: float = 2.0, jitter: float = 0.05) -> np.ndarray:
    """Per-(head, channel) log-decay rates with small per-token jitter, so a slow channel
    stays slow across a chunk (per-token i.i.d. gates almost never carry state across a
    chunk boundary).  Returns g <= 0 of shape [tokens][heads][dk] (fp64)."""
    rate = rng.uniform(np.log(lo), np.log(hi), size=(heads, dk))
    base = -np.exp(rate)
    jit = rng.uniform(1.0 - jitter, 1.0 + jitter, size=(tokens, heads, dk))
    return base[None] * jit
