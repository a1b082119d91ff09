"""ctypes binding of libkda.so (include/kda.h).  Argument marshalling only: every step of
the KDA path runs in the library's HIP kernels.  Loading fails loudly when the library
has not been built; there is no fallback."""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK, KDA_E_ARG, KDA_E_SHAPE, KDA_E_ALIGN, KDA_E_DTYPE, KDA_E_WORKSPACE, KDA_E_HIP, \
    KDA_E_UNSUPPORTED = range(8)
KDA_F32, KDA_BF16, KDA_Q8_0, KDA_MXFP4 = 0, 1, 2, 3
KDA_OP_DECODE, KDA_OP_VERIFY, KDA_OP_PREFILL, KDA_OP_SCAN = 0, 1, 2, 3
KDA_OPT_GRAPH, KDA_OPT_TIMING, KDA_OPT_PERSISTENT, KDA_OPT_WAIT_US, KDA_OPT_COOPERATIVE = 0, 1, 2, 3, 4
KDA_Q_PERSISTENT = 0
KDA_Q_OWNS_WEIGHTS = 1
KDA_K_PROJ, KDA_K_HEAD, KDA_K_OUT, KDA_K_COMMIT, KDA_K_PREFILL, KDA_K_GATES, KDA_K_STEP, \
    KDA_K_GEMM, KDA_K_CHUNK = range(9)
DTYPES = {"f32": KDA_F32, "bf16": KDA_BF16, "q8_0": KDA_Q8_0, "mxfp4": KDA_MXFP4}
KDA_GATE_KDA, KDA_GATE_SAFE, KDA_GATE_SCALAR = 0, 1, 2
GATES = {"kda": KDA_GATE_KDA, "safe": KDA_GATE_SAFE, "scalar": KDA_GATE_SCALAR}

EXPORTS = (
    "kda_abi_version", "kda_status_string", "kda_last_error", "kda_packed_bytes", "kda_pack",
    "kda_pack_device", "kda_unpack_q8_0", "kda_unpack_q8_0_device", "kda_model_create", "kda_model_destroy", "kda_model_set_option",
    "kda_timing_query", "kda_workspace_bytes", "kda_decode_step", "kda_verify_log_bytes",
    "kda_verify_steps", "kda_verify_commit", "kda_prefill_chunked", "kda_model_query",
    "kda_model_status", "kda_conv_window_canonical", "kda_decode_step_masked",
    "kda_decode_step_static", "kda_prefill_scan", "kda_unpack_mxfp4", "kda_stream_read_probe",
    "kda_state_flush",
)


class KdaDims(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("n_heads", C.c_int32), ("d_k", C.c_int32),
                ("d_v", C.c_int32), ("conv_k", C.c_int32), ("rank_f", C.c_int32),
                ("rank_g", C.c_int32), ("n_layers", C.c_int32),
                ("prenorm_residual", C.c_int32), ("norm_eps", C.c_float),
                ("l2_eps", C.c_float), ("wtype", C.c_int32), ("gate", C.c_int32),
                ("gate_lb", C.c_float)]


class KdaLayer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("wq", "wk", "wv", "wo", "fa", "fb", "wbeta", "ga", "gb",
                                           "conv_w", "a_log", "dt_bias", "o_norm_w")]


class KdaState(C.Structure):
    _fields_ = [("S_dev", C.c_void_p), ("conv_dev", C.c_void_p), ("batch", C.c_int32)]


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} -> status {status}: {detail}")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "python -m linear_attention_decode_amd._build")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        sig = {
            "kda_abi_version": (C.c_int, []),
            "kda_status_string": (C.c_char_p, [C.c_int]),
            "kda_last_error": (C.c_char_p, []),
            "kda_packed_bytes": (sz, [C.c_int, i64, i64]),
            "kda_pack": (C.c_int, [C.c_int, vp, i64, i64, vp, vp]),
            "kda_pack_device": (C.c_int, [C.c_int, vp, i64, i64, vp, vp]),
            "kda_unpack_q8_0": (C.c_int, [vp, i64, i64, vp, vp, vp]),
            "kda_unpack_q8_0_device": (C.c_int, [vp, i64, i64, vp, vp, vp]),
            "kda_unpack_mxfp4": (C.c_int, [vp, i64, i64, vp, vp, vp]),
            "kda_stream_read_probe": (C.c_int, [vp, sz, C.c_int, vp, C.POINTER(C.c_float)]),
            "kda_model_create": (C.c_int, [C.POINTER(KdaDims), C.POINTER(KdaLayer), C.POINTER(vp)]),
            "kda_model_destroy": (None, [vp]),
            "kda_model_set_option": (C.c_int, [vp, C.c_int, i64]),
            "kda_model_query": (C.c_int, [vp, C.c_int]),
            "kda_model_status": (C.c_int, [vp]),
            "kda_timing_query": (C.c_int, [vp, C.c_int, C.POINTER(C.c_double), C.POINTER(i64), C.c_int]),
            "kda_workspace_bytes": (sz, [vp, C.c_int, i32, i64]),
            "kda_decode_step": (C.c_int, [vp, vp, vp, C.POINTER(KdaState), vp, sz, vp]),
            "kda_decode_step_masked": (C.c_int, [vp, vp, vp, C.POINTER(KdaState), vp, vp, sz, vp]),
            "kda_decode_step_static": (C.c_int, [vp, vp, vp, C.POINTER(KdaState), vp]),
            "kda_prefill_scan": (C.c_int, [vp, vp, i64, vp, C.POINTER(KdaState), vp, sz, vp]),
            "kda_verify_log_bytes": (sz, [vp, i32, i32]),
            "kda_verify_steps": (C.c_int, [vp, vp, i32, vp, C.POINTER(KdaState), vp, sz, vp, sz, vp]),
            "kda_verify_commit": (C.c_int, [vp, C.POINTER(KdaState), vp, sz, i32, vp, vp]),
            "kda_state_flush": (C.c_int, [vp, C.POINTER(KdaState), vp]),
            "kda_conv_window_canonical": (C.c_int, [vp, C.POINTER(KdaState), vp, vp]),
            "kda_prefill_chunked": (C.c_int, [vp, vp, C.c_int, i64, i32, vp, C.POINTER(KdaState), vp, sz, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(fn: str, status: int) -> None:
    if status != KDA_OK:
        detail = lib().kda_last_error().decode()
        raise KdaError(fn, status, detail)


def call(fn: str, *args) -> None:
    check(fn, getattr(lib(), fn)(*args))
