"""Pins for the oracle's 2-bit requantization (flash-moe-inference skill
page: the 4-bit to 2-bit conversion step and ``repack_experts_2bit.py``;
reading: each group's exact minimum to maximum in three equal steps, nearest
grid point, ties to the even code, stored step and minimum rounded to bf16).

The pins: bf16 rounding against hand-worked values; groups worked by hand
(exactly representable grids, a negative scale, ties, constant groups, a
step that rounds); a brute-force nearest-grid-point check over all four
codes in exact arithmetic; the error bound of the stored grid; the packing of
the 2-bit words.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.conftest import golden_rows


def _pack(codes, bits):
    """Pack codes along the last axis, low bits first (test-local packer)."""
    c = np.asarray(codes, dtype=np.uint64)
    per = 32 // bits
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // per, per))
    w = np.zeros(c.shape[:-1], dtype=np.uint64)
    for j in range(per):
        w += c[..., j] << np.uint64(bits * j)
    return w.astype(np.uint32)


def _qt(codes, s_bits, b_bits, bits, gs):
    codes = np.asarray(codes)
    rows, cols = codes.shape
    return {"q": _pack(codes, bits), "scales": np.asarray(s_bits, np.uint16).reshape(rows, -1),
            "biases": np.asarray(b_bits, np.uint16).reshape(rows, -1), "batch": 1,
            "rows": rows, "cols": cols, "bits": bits, "group_size": gs}


def _codes2(r):
    return oracle.unpack_codes(r["q"], 2, r["cols"])


@pytest.mark.parametrize("row", golden_rows("bf16_round.txt"))
def test_bf16_round_hand_worked(row):
    num, den, bits = int(row[0]), int(row[1]), int(row[2], 16)
    assert oracle.bf16_round(Fraction(num, den)) == bits


def test_bf16_round_rejects_values_outside_the_normal_range():
    with pytest.raises(ValueError):
        oracle.bf16_round(Fraction(3, 2 ** 130))
    with pytest.raises(ValueError):
        oracle.bf16_round(Fraction(2) ** 128)


def test_exact_grid_round_trips():
    # 4-bit codes on {0, 5, 10, 15}, s = 2^-6 (0x3C80), b = -1/8 (0xBE00):
    # lo = b, step = 5 s exactly (0x3DA0), q2 = q / 5, and the 2-bit grid
    # reproduces every weight exactly
    rng = np.random.default_rng(0)
    codes = rng.choice([0, 5, 10, 15], size=(3, 128))
    codes[:, 0], codes[:, 64], codes[:, 1], codes[:, 65] = 0, 0, 15, 15
    r = oracle.requant_2bit(_qt(codes, [0x3C80] * 6, [0xBE00] * 6, 4, 64))
    assert np.array_equal(_codes2(r), codes // 5)
    assert (r["scales"] == 0x3DA0).all() and (r["biases"] == 0xBE00).all()
    src = oracle.dequantize(_qt(codes, [0x3C80] * 6, [0xBE00] * 6, 4, 64))
    assert np.array_equal(oracle.dequantize(r), src)


def test_negative_scale_reverses_the_codes():
    # s = -2^-6 (0xBC80), b = 1/8 (0x3E00): the minimum sits at code 15,
    # lo = 1/8 - 15/64 = -7/64 (0xBDE0), q2 = (15 - q) / 5
    codes = np.tile(np.array([0, 5, 10, 15]), 16)[None, :]
    r = oracle.requant_2bit(_qt(codes, [0xBC80], [0x3E00], 4, 64))
    assert np.array_equal(_codes2(r)[0], (15 - codes[0]) // 5)
    assert r["scales"][0, 0] == 0x3DA0 and r["biases"][0, 0] == 0xBDE0


def test_ties_go_to_the_even_code():
    # 8-bit, s = 2^-7 (0x3C00), b = -1 (0xBF80), codes spanning 0..30: the
    # step is 10 codes, so code 5 sits at 0.5 steps (-> 0), 15 at 1.5 (-> 2),
    # 25 at 2.5 (-> 2); 10, 20, 30 are exact
    base = [0, 30, 5, 15, 25, 10, 20, 30]
    codes = np.array((base * 8)[:64])[None, :]
    r = oracle.requant_2bit(_qt(codes, [0x3C00], [0xBF80], 8, 64))
    want = {0: 0, 30: 3, 5: 0, 15: 2, 25: 2, 10: 1, 20: 2}
    assert list(_codes2(r)[0]) == [want[int(c)] for c in codes[0]]
    assert r["scales"][0, 0] == 0x3DA0 and r["biases"][0, 0] == 0xBF80


def test_rounded_step_and_nearest_codes():
    # 4-bit, s = 2^-6, b = -1/8, codes 0..14: step = 14/(3*64) = 7/96, which
    # rounds to 0x3D95; q2 = round(3q/14): 7 -> 1.5 -> 2, 2 -> 0.43 -> 0,
    # 3 -> 0.64 -> 1, 11 -> 2.36 -> 2, 12 -> 2.57 -> 3, 14 -> 3
    codes = np.array([0, 14, 7, 2, 3, 11, 12, 14] * 8)[None, :]
    r = oracle.requant_2bit(_qt(codes, [0x3C80], [0xBE00], 4, 64))
    want = {0: 0, 14: 3, 7: 2, 2: 0, 3: 1, 11: 2, 12: 3}
    assert list(_codes2(r)[0]) == [want[int(c)] for c in codes[0]]
    assert r["scales"][0, 0] == 0x3D95 and r["biases"][0, 0] == 0xBE00


def test_constant_groups_and_zero_scale():
    # all codes 7 with s = 2^-6, b = -1/8: w = -1/64 everywhere (0xBC80),
    # step 0; a zero scale with b = 1/2 makes every weight 1/2 (0x3F00)
    codes = np.concatenate([np.full(64, 7), np.random.default_rng(1).integers(0, 16, 64)])[None, :]
    r = oracle.requant_2bit(_qt(codes, [0x3C80, 0x0000], [0xBE00, 0x3F00], 4, 64))
    assert (_codes2(r) == 0).all()
    assert list(r["scales"][0]) == [0, 0] and list(r["biases"][0]) == [0xBC80, 0x3F00]


def test_packing_low_bits_first():
    # codes 0,1,2,3 repeating pack into 0b11_10_01_00 per byte = 0xE4E4E4E4
    codes = np.tile(np.array([0, 5, 10, 15]), 32)[None, :]
    r = oracle.requant_2bit(_qt(codes, [0x3C80, 0x3C80], [0xBE00, 0xBE00], 4, 64))
    assert r["q"].shape == (1, 8) and (r["q"] == 0xE4E4E4E4).all()


def _random_source(bits, gs, rows, cols, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 1 << bits, (rows, cols))
    # scales of either sign, some groups narrow (few distinct codes)
    s = rng.uniform(0.005, 0.02, (rows, cols // gs)) * rng.choice([-1.0, 1.0], (rows, cols // gs))
    b = rng.normal(0.0, 0.1, (rows, cols // gs))
    narrow = rng.random((rows, cols // gs)) < 0.25
    for r, g in zip(*np.nonzero(narrow)):
        codes[r, g * gs:(g + 1) * gs] = rng.integers(3, 6, gs)
    sb = np.array([oracle.bf16_round(Fraction(float(v))) for v in s.ravel()]).reshape(s.shape)
    bb = np.array([oracle.bf16_round(Fraction(float(v))) for v in b.ravel()]).reshape(b.shape)
    return _qt(codes, sb, bb, bits, gs)


@pytest.mark.parametrize("bits,gs", [(4, 64), (4, 128), (8, 64), (8, 128)])
def test_codes_are_the_nearest_grid_points_by_brute_force(bits, gs):
    src = _random_source(bits, gs, 4, 256, seed=bits * gs)
    r = oracle.requant_2bit(src)
    codes = oracle.unpack_codes(src["q"], bits, 256)
    s = oracle.bf16_bits_to_f32(src["scales"])
    b = oracle.bf16_bits_to_f32(src["biases"])
    q2 = _codes2(r)
    for row in range(4):
        for g in range(256 // gs):
            cols = slice(g * gs, (g + 1) * gs)
            sg, bg = Fraction(float(s[row, g])), Fraction(float(b[row, g]))
            ws = [sg * int(c) + bg for c in codes[row, cols]]      # exact weights
            lo, hi = min(ws), max(ws)
            grid = [lo + k * (hi - lo) / 3 for k in range(4)]
            for wj, qj in zip(ws, q2[row, cols]):
                d = [abs(wj - p) for p in grid]
                best = min(d)
                ks = [k for k in range(4) if d[k] == best]
                # the nearest point; of two equally near, the even one
                assert int(qj) == (ks[0] if len(ks) == 1 else [k for k in ks if k % 2 == 0][0])
            if hi > lo:
                assert set(q2[row, cols]) >= {0, 3}    # the extremes map to the ends


@pytest.mark.parametrize("bits,gs", [(4, 64), (8, 128)])
def test_stored_grid_error_bound(bits, gs):
    src = _random_source(bits, gs, 8, 512, seed=7 + bits)
    r = oracle.requant_2bit(src)
    w = oracle.dequantize(src).astype(np.float64)
    w2 = oracle.dequantize(r).astype(np.float64)
    g = w.reshape(8, -1, gs)
    lo, hi = g.min(axis=2), g.max(axis=2)
    step = (hi - lo) / 3
    s2 = oracle.bf16_bits_to_f32(r["scales"]).astype(np.float64)
    b2 = oracle.bf16_bits_to_f32(r["biases"]).astype(np.float64)
    # |w - (b2 + s2 q2)| <= step/2 + |b2 - lo| + 3 |s2 - step| (+ fp32 rounding of w2)
    bound = step / 2 + np.abs(b2 - lo) + 3 * np.abs(s2 - step) + 1e-6
    err = np.abs(w2 - w).reshape(8, -1, gs).max(axis=2)
    assert (err <= bound).all()
    # and bf16 rounding keeps the stored values within 2^-9 relative
    assert (np.abs(s2 - step) <= np.abs(step) * 2.0 ** -8).all()
    assert (np.abs(b2 - lo) <= np.abs(lo) * 2.0 ** -8).all()


def test_stacks_keep_their_shape_and_reject_bad_sources():
    src = _random_source(4, 64, 6, 128, seed=3)
    st = dict(src, q=src["q"].reshape(2, 3, -1), scales=src["scales"].reshape(2, 3, -1),
              biases=src["biases"].reshape(2, 3, -1), batch=2, rows=3)
    r = oracle.requant_2bit(st)
    assert r["q"].shape == (2, 3, 8) and r["scales"].shape == (2, 3, 2)
    flat = oracle.requant_2bit(src)
    assert np.array_equal(r["q"].reshape(6, -1), flat["q"])
    with pytest.raises(ValueError):
        oracle.requant_2bit(dict(src, group_size=32, scales=np.zeros((6, 4), np.uint16)))
    with pytest.raises(ValueError):
        oracle.requant_2bit(dict(_random_source(4, 64, 1, 64, 1), bits=2))


# ---- the integer form used over whole expert stacks (requant_2bit_fast) ----

def _same(a, b):
    return (np.array_equal(a["q"], b["q"]) and np.array_equal(a["scales"], b["scales"])
            and np.array_equal(a["biases"], b["biases"]))


@pytest.mark.parametrize("bits,gs,seed", [(4, 64, 1), (4, 128, 2), (8, 64, 3), (8, 128, 4),
                                          (4, 64, 5), (8, 64, 6)])
def test_fast_form_equals_the_exact_definition(bits, gs, seed):
    # negative scales, narrow groups (grid ties), random biases
    src = _random_source(bits, gs, 8, 512, seed=100 + seed)
    assert _same(oracle.requant_2bit_fast(src), oracle.requant_2bit(src))


def test_fast_form_on_degenerate_and_far_apart_groups():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, (6, 256))
    codes[0, :64] = 7                               # one code only: no spread
    codes[1, 64:128] = rng.choice([3, 4], 64)       # two neighbouring codes
    codes[2, :64] = rng.choice([0, 15], 64)         # only the two extremes
    s = [0x3C80] * 24
    b = [0xBE00] * 24
    s[1], b[1] = 0x0000, 0x3F00                      # zero scale
    s[2], b[2] = 0x8000, 0x8000                      # -0 scale and -0 bias
    s[5], b[5] = 0xBC80, 0x3E00                      # negative scale
    s[8], b[8] = 0x21C0, 0x3F80                      # s = 1.5 * 2^-60, b = 1: s*q + b inexact in fp64
    s[9], b[9] = 0xA1C0, 0xBF80                      # the same with both signs flipped
    s[12], b[12] = 0x0D80, 0x3F80                    # s near 2^-100 against 1
    src = _qt(codes, s, b, 4, 64)
    fast, exact = oracle.requant_2bit_fast(src), oracle.requant_2bit(src)
    assert _same(fast, exact)
    assert (_codes2(fast)[0, :64] == 0).all() and fast["scales"][0, 0] == 0


def test_fast_form_on_stacks_and_rejections():
    src = _random_source(4, 64, 6, 128, seed=3)
    st = dict(src, q=src["q"].reshape(2, 3, -1), scales=src["scales"].reshape(2, 3, -1),
              biases=src["biases"].reshape(2, 3, -1), batch=2, rows=3)
    r = oracle.requant_2bit_fast(st)
    assert r["q"].shape == (2, 3, 8) and r["scales"].shape == (2, 3, 2)
    assert _same({k: v.reshape(6, -1) for k, v in r.items() if k in ("q", "scales", "biases")},
                 oracle.requant_2bit(src))
    with pytest.raises(ValueError):
        oracle.requant_2bit_fast(dict(src, group_size=32, scales=np.zeros((6, 4), np.uint16)))
    with pytest.raises(ValueError):
        oracle.requant_2bit_fast(dict(_random_source(4, 64, 1, 64, 1), bits=2))
