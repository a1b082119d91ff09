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
