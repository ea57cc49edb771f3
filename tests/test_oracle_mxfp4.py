"""Pins for the oracle's mxfp4 mode (the OCP Microscaling FP4 format that
the mlx ``mode="mxfp4"`` of the ml-explore/mlx issue #3856 repro names:
E2M1 elements, one E8M0 scale byte per 32 elements, no bias).

Hand-worked element values (tests/golden/mxfp4_values.txt), the E2M1
magnitudes as the spec's formula written out per code, the scale as a power
of two, group boundaries at 32 columns, a hand-packed word, and the qmatvec
of one-hot rows reading single weights back.
"""

import numpy as np
import pytest

import oracle
from tests.conftest import golden_rows


def _pack4(codes):
    c = np.asarray(codes, dtype=np.uint64)
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // 8, 8))
    w = np.zeros(c.shape[:-1], dtype=np.uint64)
    for j in range(8):
        w += c[..., j] << np.uint64(4 * j)
    return w.astype(np.uint32)


def _qt(codes, scale_bytes):
    codes = np.asarray(codes)
    rows, cols = codes.shape
    return {"q": _pack4(codes), "scales": np.asarray(scale_bytes, np.uint8).reshape(rows, -1),
            "biases": None, "rows": rows, "cols": cols, "bits": 4, "group_size": 32,
            "mode": "mxfp4"}


@pytest.mark.parametrize("row", golden_rows("mxfp4_values.txt"))
def test_hand_worked_values(row):
    code, e, want = int(row[0]), int(row[1]), float(row[2])
    codes = np.zeros((1, 32), np.int64)
    codes[0, 5] = code
    w = oracle.dequantize(_qt(codes, [e]))
    assert w.dtype == np.float32
    assert w[0, 5] == np.float32(want)
    assert np.signbit(w[0, 5]) == np.signbit(want)


def test_magnitudes_follow_the_e2m1_formula():
    # code = s e1 e0 m: e = 0 -> m/2, else (1 + m/2) * 2^(e-1)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = oracle.fp4_e2m1(c)
        assert abs(v) == mags[c & 7]
        assert np.signbit(v) == (c >= 8)


def test_scale_is_a_power_of_two_and_255_is_nan():
    assert oracle.e8m0_scale(127) == 1.0
    assert oracle.e8m0_scale(128) == 2.0
    assert oracle.e8m0_scale(0) == 2.0 ** -127
    assert oracle.e8m0_scale(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_scale(255))


def test_groups_of_32_columns_take_their_own_scale():
    codes = np.full((2, 96), 2, np.int64)                  # every element 1.0 before scaling
    w = oracle.dequantize(_qt(codes, [[127, 128, 126], [130, 127, 124]]))
    assert np.array_equal(w[0], np.repeat([1.0, 2.0, 0.5], 32).astype(np.float32))
    assert np.array_equal(w[1], np.repeat([8.0, 1.0, 0.125], 32).astype(np.float32))


def test_hand_packed_word_low_nibble_first():
    # word 0xFEDCBA98 holds codes 8..15 in columns 0..7
    q = np.array([[0xFEDCBA98, 0x76543210, 0, 0]], np.uint32)
    qt = {"q": q, "scales": np.array([[127]], np.uint8), "biases": None, "rows": 1, "cols": 32,
          "bits": 4, "group_size": 32, "mode": "mxfp4"}
    w = oracle.dequantize(qt)[0]
    assert list(w[:16]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
                            0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.signbit(w[0]) and not np.signbit(w[8])


def test_qmatvec_one_hot_reads_weights_and_rejects_other_shapes():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, (3, 64))
    qt = _qt(codes, rng.integers(120, 134, (3, 2)))
    w = oracle.dequantize(qt)
    for k in (0, 31, 32, 63):
        x = np.zeros((1, 64), np.float32)
        x[0, k] = 1.0
        assert np.array_equal(oracle.qmatvec(qt, x)[0], w[:, k].astype(np.float64))
    with pytest.raises(ValueError):
        oracle.dequantize(dict(qt, group_size=64, scales=qt["scales"][:, :1]))
