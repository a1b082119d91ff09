"""Host-side checks of the C ABI that need no GPU: the library loads, exports every
function include/kda.h declares, and validates arguments before touching the device."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    from linear_attention_decode_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libkda.so not built (run __graft_entry__.build())")
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n


def test_abi_version(L):
    assert L.kda_abi_version() == 3


def test_packed_bytes(L):
    from linear_attention_decode_amd import _lib
    assert L.kda_packed_bytes(_lib.KDA_F32, 3, 5) == 60
    assert L.kda_packed_bytes(_lib.KDA_BF16, 3, 5) == 30
    # Q8_0: byte plane rounded up to 256, then the fp16 scales
    assert L.kda_packed_bytes(_lib.KDA_Q8_0, 3, 64) == 256 + 3 * 2 * 2
    assert L.kda_packed_bytes(_lib.KDA_Q8_0, 64, 2048) == 64 * 2048 + 64 * 64 * 2
    assert L.kda_packed_bytes(_lib.KDA_Q8_0, 3, 40) == 0
    assert L.kda_packed_bytes(_lib.KDA_F32, 0, 5) == 0
    assert L.kda_packed_bytes(7, 3, 5) == 0


def test_pack_validates_before_launch(L):
    from linear_attention_decode_amd import _lib
    p = C.c_void_p(4096)
    for fn in (L.kda_pack, L.kda_pack_device):
        assert fn(9, p, 2, 32, p, None) == _lib.KDA_E_DTYPE
        assert fn(_lib.KDA_Q8_0, p, 2, 40, p, None) == _lib.KDA_E_SHAPE
        assert fn(_lib.KDA_F32, None, 2, 4, p, None) == _lib.KDA_E_ARG
        assert fn(_lib.KDA_F32, p, 2, 4, C.c_void_p(4100), None) == _lib.KDA_E_ALIGN
        assert b"aligned" in L.kda_last_error()
    # the device source must be aligned too; the host source need not be
    assert L.kda_pack_device(_lib.KDA_F32, C.c_void_p(4100), 2, 4, p, None) == _lib.KDA_E_ALIGN


def test_unpack_validates_before_copy(L):
    from linear_attention_decode_amd import _lib
    p = C.c_void_p(4096)
    for fn in (L.kda_unpack_q8_0, L.kda_unpack_q8_0_device):
        assert fn(None, 2, 32, p, p, None) == _lib.KDA_E_ARG
        assert fn(p, 2, 40, p, p, None) == _lib.KDA_E_SHAPE
        assert fn(p, 0, 32, p, p, None) == _lib.KDA_E_SHAPE


def _dims(**kw):
    from linear_attention_decode_amd import _lib
    base = dict(d_model=256, n_heads=2, d_k=64, d_v=64, conv_k=4, rank_f=32, rank_g=32,
                n_layers=1, prenorm_residual=0, norm_eps=1e-6, l2_eps=1e-6, wtype=_lib.KDA_Q8_0,
                gate=0, gate_lb=-5.0)
    base.update(kw)
    return _lib.KdaDims(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(d_k=96, d_v=96), 2), (dict(d_v=128), 2), (dict(conv_k=3), 2),
    (dict(rank_f=16), 2), (dict(d_model=250), 2), (dict(wtype=5), 4), (dict(n_layers=0), 2),
    (dict(gate=3), 1), (dict(gate=1, gate_lb=0.0), 1), (dict(gate=1, gate_lb=float("nan")), 1),
])
def test_model_create_rejects_bad_dims(L, kw, status):
    from linear_attention_decode_amd import _lib
    layer = _lib.KdaLayer(*([4096] * 12), None)
    out = C.c_void_p()
    assert L.kda_model_create(C.byref(_dims(**kw)), C.byref(layer), C.byref(out)) == status
    assert not out.value


def test_model_create_rejects_null_and_unaligned(L):
    from linear_attention_decode_amd import _lib
    out = C.c_void_p()
    layer = _lib.KdaLayer(*([4096] * 11), None, None)
    assert L.kda_model_create(C.byref(_dims()), C.byref(layer), C.byref(out)) == _lib.KDA_E_ARG
    layer = _lib.KdaLayer(*([4096] * 11), 4100, None)
    assert L.kda_model_create(C.byref(_dims()), C.byref(layer), C.byref(out)) == _lib.KDA_E_ALIGN


def test_status_strings(L):
    for s in range(8):
        assert L.kda_status_string(s)


def test_verify_calls_validate_before_launch(L):
    """Null model or state pointers are refused by the verify, commit and flush calls."""
    from linear_attention_decode_amd import _lib
    p = C.c_void_p(4096)
    st = _lib.KdaState(None, None, 1)
    assert L.kda_state_flush(None, C.byref(st), None) == _lib.KDA_E_ARG
    assert L.kda_verify_commit(None, C.byref(st), p, 1 << 20, 4, p, None) == _lib.KDA_E_ARG
    assert L.kda_verify_steps(None, p, 4, p, C.byref(st), p, 1 << 20, p, 1 << 20, None) == _lib.KDA_E_ARG
    assert L.kda_verify_log_bytes(None, 1, 4) == 0
