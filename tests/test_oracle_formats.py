"""Pins of the oracle's weight formats (BF16 rounding, Q8_0 quantisation)."""
import os

import numpy as np
import pytest

import oracle
from oracle import kda as ok

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q8_0_block.txt")


def _read_golden():
    blocks, cur = [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "block":
                cur = {"name": rest}
                blocks.append(cur)
            elif key == "x_expr":
                i = np.arange(32, dtype=np.float64)
                sign = -1.0 if rest.startswith("-") else 1.0
                cur["x"] = (sign * (i / 31.0)).astype(np.float32)
            elif key == "x":
                cur["x"] = np.array([float(v) for v in rest.split()], np.float32)
            elif key == "d16_bits":
                cur["d16_bits"] = int(rest, 16)
            elif key == "q":
                cur["q"] = np.array([int(v) for v in rest.split()], np.int8)
    return blocks


@pytest.mark.parametrize("blk", _read_golden(), ids=lambda b: b["name"])
def test_q8_0_golden_blocks(blk):
    d16, q = oracle.q8_0_quantize(blk["x"][None, :])
    assert int(d16.view(np.uint16)[0, 0]) == blk["d16_bits"]
    np.testing.assert_array_equal(q[0], blk["q"])


def test_q8_0_half_step_bound_and_amax():
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[3, 32:64] *= 1e3          # wide dynamic range between blocks
    w[5, :32] = 0.0             # an all-zero block
    d16, q = oracle.q8_0_quantize(w)
    deq = oracle.q8_0_dequantize(d16, q)
    step = np.repeat(d16.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(w.astype(np.float64) - deq) <= step / 2)
    blocks = np.abs(w.reshape(64, 8, 32))
    imax = np.argmax(blocks, axis=-1)
    qb = q.reshape(64, 8, 32)
    amax_q = np.take_along_axis(qb, imax[..., None], axis=-1)[..., 0]
    nz = blocks.max(-1) > 0
    assert np.all(np.abs(amax_q[nz]) == 127)
    assert np.all(q[5, :32] == 0) and d16[5, 0] == 0


def test_q8_0_scale_is_nearest_fp16():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((128, 64)) * rng.uniform(1e-3, 10, (128, 1))).astype(np.float32)
    d16, _ = oracle.q8_0_quantize(w)
    amax = np.abs(w.reshape(128, 2, 32)).max(-1)
    d = (amax / np.float32(127)).astype(np.float64)
    up = np.nextafter(d16, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(d16, np.float16(-np.inf)).astype(np.float64)
    err = np.abs(d - d16.astype(np.float64))
    assert np.all(err <= np.abs(d - up)) and np.all(err <= np.abs(d - dn))


def test_q8_0_rejects_ragged_cols():
    with pytest.raises(ValueError):
        oracle.q8_0_quantize(np.zeros((2, 40), np.float32))


def test_bf16_round_hand_worked():
    one = 1.0
    cases = [
        (one + 2.0 ** -8, one),                       # tie, even side is 1.0
        (one + 3 * 2.0 ** -8, one + 2.0 ** -6),       # tie, even side is up
        (one + 2.0 ** -8 + 2.0 ** -20, one + 2.0 ** -7),
        (-(one + 2.0 ** -8), -one),
        (-(one + 3 * 2.0 ** -8), -(one + 2.0 ** -6)),
        (3.0, 3.0),
        (0.0, 0.0),
    ]
    x = np.array([c[0] for c in cases], np.float32)
    np.testing.assert_array_equal(oracle.bf16_round(x), np.array([c[1] for c in cases]))


def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(100000) * rng.uniform(1e-3, 1e3, 100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x), ref)


def test_mutant_round_half_even_fails_golden():
    """A Q8_0 quantiser that rounds ties to even must fail the golden 'ties' block."""
    blk = [b for b in _read_golden() if b["name"] == "ties"][0]
    x = blk["x"][None, :]
    amax = np.abs(x).max()
    d16 = np.float16(np.float32(amax) / np.float32(127))
    q_mut = np.clip(np.rint(x / np.float32(d16)), -127, 127).astype(np.int8)[0]
    assert not np.array_equal(q_mut, blk["q"])


# ----------------------------------------------------------------------------------------
# MXFP4 (OCP Microscaling format specification v1.0)
# ----------------------------------------------------------------------------------------
MX_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_block.txt")


def _read_mx_golden():
    blocks, cur = [], None
    with open(MX_GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "block":
                cur = {"name": rest}
                blocks.append(cur)
            elif key == "x":
                v = [float(t) for t in rest.split()]
                cur["x"] = np.array(v + [0.0] * (32 - len(v)), np.float32)
            elif key == "e8m0":
                cur["e8m0"] = int(rest)
            elif key == "codes":
                v = [int(t) for t in rest.split()]
                cur["codes"] = np.array(v + [0] * (32 - len(v)), np.uint8)
    return blocks


@pytest.mark.parametrize("blk", _read_mx_golden(), ids=lambda b: b["name"])
def test_mxfp4_golden_blocks(blk):
    e, c = ok.mxfp4_quantize(blk["x"][None, :])
    assert int(e[0, 0]) == blk["e8m0"]
    np.testing.assert_array_equal(c[0], blk["codes"])


def test_mxfp4_grid_values_round_trip():
    """Values on the E2M1 grid times a block's scale come back exactly (the block's largest
    magnitude is 4 or 6 times the scale, so the scale is the one chosen)."""
    rng = np.random.default_rng(12)
    for s in (-20, -7, 0, 5):
        idx = rng.integers(0, 8, (4, 64))
        idx[:, 0] = 7
        idx[:, 32] = 6
        sign = rng.integers(0, 2, (4, 64))
        x = (np.where(sign, -1.0, 1.0) * ok.E2M1_GRID[idx] * 2.0 ** s).astype(np.float32)
        e, c = ok.mxfp4_quantize(x)
        assert np.all(e == s + 127)
        np.testing.assert_array_equal(ok.mxfp4_dequantize(e, c), x.astype(np.float64))


def test_mxfp4_error_bounds():
    """With X the block scale: |x - q| <= X/4 where |x| <= 2X (grid spacing X/2), <= X/2
    up to 4X, <= X up to 6X, and <= 2X in the clamped range (6X, 8X); max|x| / X in [4, 8)."""
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[3, 32:64] *= 1e3
    w[5, :32] = 0.0
    e, c = ok.mxfp4_quantize(w)
    q = ok.mxfp4_dequantize(e, c)
    X = np.repeat(np.exp2(e.astype(np.float64) - 127), 32, axis=1)
    a = np.abs(w.astype(np.float64)) / X
    err = np.abs(w - q) / X
    assert np.all(err[a <= 2] <= 0.25)
    assert np.all(err[(a > 2) & (a <= 4)] <= 0.5)
    assert np.all(err[(a > 4) & (a <= 6)] <= 1.0)
    assert np.all(err[a > 6] <= 2.0)
    am = np.abs(w.reshape(64, 8, 32)).max(-1) / np.exp2(e.astype(np.float64) - 127)
    nz = am > 0
    assert np.all((am[nz] >= 4) & (am[nz] < 8))
    assert np.all(c[5, :32] == 0) and e[5, 0] == 0
