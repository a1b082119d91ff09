"""MI355X (gfx950) KDA / gated-delta-rule decode library: thin Python binding.

The functions named ``kda_*`` mirror the C ABI of include/kda.h one to one and take
torch CUDA tensors (device memory) plus an optional torch stream; ``KdaModel`` packs a
layer stack's fp32 weights on the device with ``kda_pack_device`` and owns the packed
buffers.
PyTorch provides device memory and streams only; every step of the decode / verify /
prefill path runs in the library's HIP kernels (libkda.so).  Importing this package
does not load the library; the first call does, and fails loudly if it is missing.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, List, Optional, Sequence

from . import _lib
from ._lib import (KDA_BF16, KDA_F32, KDA_Q8_0, KDA_MXFP4, KDA_OP_DECODE, KDA_OP_PREFILL, KDA_OP_SCAN,  # noqa: F401
                   KDA_OP_VERIFY, KDA_OPT_GRAPH, KDA_OPT_TIMING, KDA_K_PROJ, KDA_K_HEAD,
                   KDA_K_OUT, KDA_K_COMMIT, KDA_K_PREFILL, KDA_K_GATES, KDA_K_STEP, KDA_K_GEMM, KDA_K_CHUNK,
                   KDA_OPT_PERSISTENT, KDA_OPT_WAIT_US, KDA_OPT_COOPERATIVE, KDA_Q_PERSISTENT, KDA_Q_OWNS_WEIGHTS, DTYPES, KdaError,
                   KDA_GATE_KDA, KDA_GATE_SAFE, KDA_GATE_SCALAR, GATES)

_PROJ_NAMES = ("wq", "wk", "wv", "wo", "fa", "fb", "wbeta", "ga", "gb")


def _torch():
    import torch
    return torch


def _p(t) -> C.c_void_p:
    return C.c_void_p(0 if t is None else t.data_ptr())


def _s(stream) -> C.c_void_p:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dev_f32(t):
    torch = _torch()
    assert t.is_cuda and t.dtype == torch.float32 and t.is_contiguous(), "need contiguous cuda fp32"
    return t


# ----------------------------------------------------------------------------------------
# Functions with the C names
# ----------------------------------------------------------------------------------------
def kda_abi_version() -> int:
    return _lib.lib().kda_abi_version()


def kda_packed_bytes(dtype: int, rows: int, cols: int) -> int:
    return _lib.lib().kda_packed_bytes(dtype, rows, cols)


def kda_pack(dtype: int, src, dst, stream=None) -> None:
    """src: host fp32 [rows][cols] (numpy array or CPU tensor); dst: cuda uint8 tensor of
    kda_packed_bytes bytes.  Synchronous."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(src, dtype=np.float32))
    rows, cols = a.shape
    assert dst.numel() * dst.element_size() >= kda_packed_bytes(dtype, rows, cols)
    _lib.call("kda_pack", dtype, a.ctypes.data_as(C.c_void_p), rows, cols, _p(dst), _s(stream))


def kda_pack_device(dtype: int, src, dst, stream=None) -> None:
    """src: cuda fp32 [rows][cols]; dst: cuda uint8 tensor of kda_packed_bytes bytes."""
    rows, cols = src.shape
    _dev_f32(src)
    assert dst.numel() * dst.element_size() >= kda_packed_bytes(dtype, rows, cols)
    _lib.call("kda_pack_device", dtype, _p(src), rows, cols, _p(dst), _s(stream))


def kda_unpack_q8_0(packed, rows: int, cols: int, stream=None):
    """Canonical view of a Q8_0-packed matrix in host memory: (d16 bits as uint16 numpy
    [rows][cols/32], q as int8 numpy [rows][cols]).  Synchronous."""
    import numpy as np
    d16 = np.empty((rows, cols // 32), dtype=np.uint16)
    qs = np.empty((rows, cols), dtype=np.int8)
    _lib.call("kda_unpack_q8_0", _p(packed), rows, cols, d16.ctypes.data_as(C.c_void_p),
              qs.ctypes.data_as(C.c_void_p), _s(stream))
    return d16, qs


def kda_unpack_mxfp4(packed, rows: int, cols: int, stream=None):
    """Canonical view of an MXFP4-packed matrix in host memory: (e8m0 uint8 numpy
    [rows][cols/32], codes uint8 numpy [rows][cols]).  Synchronous."""
    import numpy as np
    e = np.empty((rows, cols // 32), dtype=np.uint8)
    c = np.empty((rows, cols), dtype=np.uint8)
    _lib.call("kda_unpack_mxfp4", _p(packed), rows, cols, e.ctypes.data_as(C.c_void_p),
              c.ctypes.data_as(C.c_void_p), _s(stream))
    return e, c


def kda_unpack_q8_0_device(packed, rows: int, cols: int, stream=None):
    """The same view on the device: (d16 bits as int16 [rows][cols/32], q as int8
    [rows][cols]) cuda tensors, asynchronous on the stream."""
    torch = _torch()
    d16 = torch.empty((rows, cols // 32), dtype=torch.int16, device=packed.device)
    qs = torch.empty((rows, cols), dtype=torch.int8, device=packed.device)
    _lib.call("kda_unpack_q8_0_device", _p(packed), rows, cols, _p(d16), _p(qs), _s(stream))
    return d16, qs


def kda_model_create(dims: _lib.KdaDims, layers: Sequence[_lib.KdaLayer]) -> C.c_void_p:
    arr = (_lib.KdaLayer * len(layers))(*layers)
    out = C.c_void_p()
    _lib.call("kda_model_create", C.byref(dims), arr, C.byref(out))
    return out


def kda_model_destroy(handle) -> None:
    _lib.lib().kda_model_destroy(handle)


def kda_model_set_option(handle, option: int, value: int) -> None:
    _lib.call("kda_model_set_option", handle, option, value)


def kda_model_query(handle, what: int) -> int:
    return _lib.lib().kda_model_query(handle, what)


def kda_model_status(handle) -> None:
    _lib.call("kda_model_status", handle)


def kda_timing_query(handle, kind: int, reset: bool = False):
    ms = C.c_double()
    n = C.c_int64()
    _lib.call("kda_timing_query", handle, kind, C.byref(ms), C.byref(n), int(reset))
    return ms.value, n.value


def kda_workspace_bytes(handle, op: int, batch: int, tokens: int) -> int:
    return _lib.lib().kda_workspace_bytes(handle, op, batch, tokens)


def kda_verify_log_bytes(handle, batch: int, T: int) -> int:
    return _lib.lib().kda_verify_log_bytes(handle, batch, T)


def _state(st) -> _lib.KdaState:
    return _lib.KdaState(st.S.data_ptr(), st.conv.data_ptr(), st.batch)


def kda_decode_step(handle, x, y, st, ws, stream=None) -> None:
    s = _state(st)
    _lib.call("kda_decode_step", handle, _p(x), _p(y), C.byref(s), _p(ws), ws.numel(), _s(stream))


def kda_decode_step_static(handle, x, y, st, stream=None) -> None:
    """kda_decode_step with the library's static workspace (allocates nothing)."""
    s = _state(st)
    _lib.call("kda_decode_step_static", handle, _p(x), _p(y), C.byref(s), _s(stream))


def kda_decode_step_masked(handle, x, y, st, active, ws, stream=None) -> None:
    """active: cuda int32 [B]; 0 = this sequence takes no token (state and window kept)."""
    s = _state(st)
    _lib.call("kda_decode_step_masked", handle, _p(x), _p(y), C.byref(s), _p(active), _p(ws),
              ws.numel(), _s(stream))


def kda_verify_steps(handle, x, T: int, y, st, log, ws, stream=None) -> None:
    s = _state(st)
    _lib.call("kda_verify_steps", handle, _p(x), T, _p(y), C.byref(s), _p(log),
              log.numel() * log.element_size(), _p(ws), ws.numel(), _s(stream))


def kda_verify_commit(handle, st, log, T: int, accept, stream=None) -> None:
    s = _state(st)
    _lib.call("kda_verify_commit", handle, C.byref(s), _p(log), log.numel() * log.element_size(),
              T, _p(accept), _s(stream))


def kda_state_flush(handle, st, stream=None) -> None:
    """Apply a commit pending on st (before st's buffers are read, copied or freed)."""
    s = _state(st)
    _lib.call("kda_state_flush", handle, C.byref(s), _s(stream))


def kda_prefill_scan(handle, x, L: int, y, st, ws, stream=None) -> None:
    """x, y: cuda fp32 [B][L][D]; st advanced by L tokens."""
    s = _state(st)
    _lib.call("kda_prefill_scan", handle, _p(x), L, _p(y), C.byref(s), _p(ws), ws.numel(), _s(stream))


def kda_stream_read_probe(buf, reps: int = 10, stream=None) -> float:
    """Mean ms per sequential read of the cuda tensor `buf` (measurement utility)."""
    ms = C.c_float()
    _lib.call("kda_stream_read_probe", _p(buf), buf.numel() * buf.element_size(), reps,
              _s(stream), C.byref(ms))
    return ms.value


def kda_conv_window_canonical(handle, st, out, stream=None) -> None:
    """out: cuda fp32 [n_layers][B][conv_k - 1][C], oldest token first."""
    s = _state(st)
    _lib.call("kda_conv_window_canonical", handle, C.byref(s), _p(out), _s(stream))


def kda_prefill_chunked(handle, x, x_dtype: int, L: int, chunk: int, y, st, ws, stream=None) -> None:
    s = _state(st)
    _lib.call("kda_prefill_chunked", handle, _p(x), x_dtype, L, chunk, _p(y), C.byref(s),
              _p(ws), ws.numel(), _s(stream))


# ----------------------------------------------------------------------------------------
# Owning helpers
# ----------------------------------------------------------------------------------------
class KdaStateBuf:
    """Device state of every layer for `batch` sequences: S [L][B][H][dk][dv] fp32 and the
    conv window [L][B][3][C] fp32 (oldest token first)."""

    def __init__(self, n_layers: int, batch: int, n_heads: int, d_k: int, d_v: int,
                 channels: int, device="cuda"):
        torch = _torch()
        self.batch = batch
        self.S = torch.zeros((n_layers, batch, n_heads, d_k, d_v), dtype=torch.float32, device=device)
        self.conv = torch.zeros((n_layers, batch, 3, channels), dtype=torch.float32, device=device)

    def clone(self) -> "KdaStateBuf":
        c = object.__new__(KdaStateBuf)
        c.batch = self.batch
        c.S = self.S.clone()
        c.conv = self.conv.clone()
        return c


class KdaModel:
    """Packs fp32 per-layer parameter draws (dicts with the keys of include/kda.h's
    kda_layer) into device buffers with kda_pack_device and creates the library model."""

    def __init__(self, layers: Sequence[Dict], *, n_heads: int, d_k: int, d_v: int,
                 wtype: str, prenorm_residual: bool, norm_eps: float = 1e-6,
                 l2_eps: float = 1e-6, gate: str = "kda", gate_lb: float = -5.0,
                 device="cuda", stream=None):
        torch = _torch()
        self.device = torch.device(device)
        self.wtype = DTYPES[wtype]
        d0 = layers[0]
        self.d_model = int(d0["wq"].shape[1])
        self.n_heads, self.d_k, self.d_v = n_heads, d_k, d_v
        self.rank_f, self.rank_g = int(d0["fa"].shape[0]), int(d0["ga"].shape[0])
        self.n_layers = len(layers)
        self.channels = 2 * n_heads * d_k + n_heads * d_v
        self.dims = _lib.KdaDims(self.d_model, n_heads, d_k, d_v, 4, self.rank_f, self.rank_g,
                                 self.n_layers, int(prenorm_residual), norm_eps, l2_eps, self.wtype,
                                 GATES[gate], gate_lb)
        self._keep: List = []
        self._packed: Dict = {}
        c_layers = []
        for li, dr in enumerate(layers):
            ptrs = {}
            for name in _PROJ_NAMES:
                w = torch.as_tensor(dr[name], dtype=torch.float32).to(self.device).contiguous()
                nb = kda_packed_bytes(self.wtype, *w.shape)
                if nb == 0:
                    raise ValueError(f"{name}: shape {tuple(w.shape)} cannot be packed as {wtype}")
                buf = torch.empty(nb, dtype=torch.uint8, device=self.device)
                kda_pack_device(self.wtype, w, buf, stream)
                self._keep.append(buf)
                self._packed[(li, name)] = buf
                ptrs[name] = buf.data_ptr()
            for name in ("conv_w", "a_log", "dt_bias"):
                t = torch.as_tensor(dr[name], dtype=torch.float32).to(self.device).contiguous()
                self._keep.append(t)
                ptrs[name] = t.data_ptr()
            onw = dr.get("o_norm_w")
            if onw is not None:
                t = torch.as_tensor(onw, dtype=torch.float32).to(self.device).contiguous()
                self._keep.append(t)
                ptrs["o_norm_w"] = t.data_ptr()
            else:
                ptrs["o_norm_w"] = None
            c_layers.append(_lib.KdaLayer(**ptrs))
        torch.cuda.synchronize(self.device)
        self.handle = kda_model_create(self.dims, c_layers)

    def packed(self, l: int, name: str):
        """Packed device buffer of matrix `name` of layer `l`."""
        return self._packed[(l, name)]

    def owns_weights(self) -> bool:
        """True if the library reads only its own copy of the packed matrices."""
        return kda_model_query(self.handle, KDA_Q_OWNS_WEIGHTS) == 1

    def release_packed(self) -> bool:
        """Drop the packed buffers this binding made, if the model no longer reads them."""
        if not self.owns_weights():
            return False
        ids = {id(b) for b in self._packed.values()}
        self._keep = [t for t in self._keep if id(t) not in ids]
        self._packed = {}
        return True

    def new_state(self, batch: int) -> KdaStateBuf:
        return KdaStateBuf(self.n_layers, batch, self.n_heads, self.d_k, self.d_v,
                           self.channels, self.device)

    def workspace(self, op: int, batch: int, tokens: int = 1):
        torch = _torch()
        n = kda_workspace_bytes(self.handle, op, batch, tokens)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)

    def set_option(self, option: int, value: int) -> None:
        kda_model_set_option(self.handle, option, value)

    def timing(self, kind: int, reset: bool = False):
        return kda_timing_query(self.handle, kind, reset)

    def persistent_blocks(self) -> int:
        """Blocks of the one-launch batch-1 decode (0: the model uses per-layer kernels)."""
        return kda_model_query(self.handle, KDA_Q_PERSISTENT)

    def status(self) -> None:
        """Synchronise; raise if a one-launch decode hit its bounded inter-block wait."""
        kda_model_status(self.handle)

    def decode_step(self, x, y, st: KdaStateBuf, ws, stream=None) -> None:
        kda_decode_step(self.handle, x, y, st, ws, stream)

    def decode_step_masked(self, x, y, st: KdaStateBuf, active, ws, stream=None) -> None:
        kda_decode_step_masked(self.handle, x, y, st, active, ws, stream)

    def verify_steps(self, x, T: int, y, st: KdaStateBuf, log, ws, stream=None) -> None:
        kda_verify_steps(self.handle, x, T, y, st, log, ws, stream)

    def verify_commit(self, st: KdaStateBuf, log, T: int, accept, stream=None) -> None:
        kda_verify_commit(self.handle, st, log, T, accept, stream)

    def flush(self, st: KdaStateBuf, stream=None) -> None:
        kda_state_flush(self.handle, st, stream)

    def conv_window(self, st: KdaStateBuf, stream=None):
        """The canonical conv windows [n_layers][B][3][C] (oldest first) as a new tensor."""
        torch = _torch()
        out = torch.empty((self.n_layers, st.batch, 3, self.channels), dtype=torch.float32,
                          device=self.device)
        kda_conv_window_canonical(self.handle, st, out, stream)
        return out

    def verify_log(self, batch: int, T: int):
        torch = _torch()
        return torch.empty(kda_verify_log_bytes(self.handle, batch, T), dtype=torch.uint8,
                           device=self.device)

    def prefill_scan(self, x, L: int, y, st: KdaStateBuf, ws, stream=None) -> None:
        kda_prefill_scan(self.handle, x, L, y, st, ws, stream)

    def prefill_chunked(self, x, x_dtype: int, L: int, chunk: int, y, st: KdaStateBuf, ws,
                        stream=None) -> None:
        kda_prefill_chunked(self.handle, x, x_dtype, L, chunk, y, st, ws, stream)

    def close(self) -> None:
        if getattr(self, "handle", None):
            kda_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
