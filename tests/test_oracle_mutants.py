"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in the oracle (on the CPU, via monkeypatch), runs
the pins that should notice it, and requires at least one of them to fail.
This is what makes the pins worth trusting: a dropped term, a wrong sign or
index, a transposed operand or a wrong tie rule cannot slip through.
"""

import numpy as np
import pytest

import oracle
import oracle.moe_oracle as mo
from tests import test_oracle_format as tf
from tests import test_oracle_mxfp4 as tm
from tests import test_oracle_norm as tn
from tests import test_oracle_requant as tq
from tests import test_oracle_route_ffn as tr
from tests.conftest import golden_rows


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(mo, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(*checks):
    for chk in checks:
        try:
            chk()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


_unpack = mo.unpack_codes
_dequant = mo.dequantize
_route = mo.route
_top_k = mo.top_k
_silu = mo.silu
_moe_experts = mo.moe_experts
_bf16_round = mo.bf16_round
_rms_norm = mo.rms_norm
_fp4 = mo.fp4_e2m1
_e8m0 = mo.e8m0_scale
_moe_block = mo.moe_block
_requant = mo.requant_2bit


def _format_pins():
    for row in golden_rows("hand_packed_words.txt"):
        tf.test_unpack_hand_packed_words(row)
    tf.test_unpack_multiword_rows_keep_column_order()
    for row in golden_rows("dequant_values.txt"):
        tf.test_dequant_closed_form(row)
    tf.test_dequant_group_boundaries()
    tf.test_qmatvec_one_hot_x_reads_codes()
    tf.test_qmatvec_constant_codes_group_sums()


def _route_pins():
    tr.test_topk_matches_sort_based_brute_force(16, 4)
    tr.test_route_weights_sum_to_one_and_equal_topk_only_softmax()
    tr.test_route_special_cases()


def _layer_pins():
    tr.test_layer_matches_python_brute_force(True, 4)
    tr.test_silu_values()


def _requant_pins():
    for row in golden_rows("bf16_round.txt"):
        tq.test_bf16_round_hand_worked(row)
    tq.test_exact_grid_round_trips()
    tq.test_negative_scale_reverses_the_codes()
    tq.test_ties_go_to_the_even_code()
    tq.test_rounded_step_and_nearest_codes()
    tq.test_constant_groups_and_zero_scale()
    tq.test_packing_low_bits_first()
    tq.test_codes_are_the_nearest_grid_points_by_brute_force(4, 64)
    tq.test_stored_grid_error_bound(4, 64)


def _norm_pins():
    tn.test_three_four_row()
    for c, eps, want in [(2.0, 0.0, 1.0), (1e-3, 1e-6, 2 ** -0.5), (3.0, 7.0, 0.75)]:
        tn.test_constant_rows(c, eps, want)
    tn.test_invariants()
    tn.test_block_brute_force(True)
    tn.test_block_routes_and_runs_on_the_normalized_row()


def _mxfp4_pins():
    for row in golden_rows("mxfp4_values.txt"):
        tm.test_hand_worked_values(row)
    tm.test_magnitudes_follow_the_e2m1_formula()
    tm.test_scale_is_a_power_of_two_and_255_is_nan()
    tm.test_groups_of_32_columns_take_their_own_scale()
    tm.test_hand_packed_word_low_nibble_first()


def test_pins_pass_on_the_real_oracle():
    _format_pins()
    _route_pins()
    _layer_pins()
    _requant_pins()
    _norm_pins()
    _mxfp4_pins()


def test_fp4_exponent_bias_zero_is_caught(monkeypatch):
    _patch(monkeypatch, "fp4_e2m1", lambda c: 2.0 * _fp4(c))
    assert _fails(_mxfp4_pins)


def test_fp4_sign_ignored_is_caught(monkeypatch):
    _patch(monkeypatch, "fp4_e2m1", lambda c: np.abs(_fp4(c)))
    assert _fails(_mxfp4_pins)


def test_e8m0_bias_off_by_one_is_caught(monkeypatch):
    _patch(monkeypatch, "e8m0_scale", lambda b: _e8m0(b) / 2.0)
    assert _fails(_mxfp4_pins)


def test_norm_without_eps_is_caught(monkeypatch):
    _patch(monkeypatch, "rms_norm", lambda x, w, eps: _rms_norm(x, w, 0.0))
    assert _fails(_norm_pins)


def test_norm_by_sum_instead_of_mean_is_caught(monkeypatch):
    def bad(x, w, eps):
        x64 = np.atleast_2d(np.asarray(x, np.float64))
        return x64 / np.sqrt(np.sum(x64 * x64, axis=1, keepdims=True) + eps) * np.asarray(w)[None, :]
    _patch(monkeypatch, "rms_norm", bad)
    assert _fails(_norm_pins)


def test_block_with_the_normalized_row_as_residual_is_caught(monkeypatch):
    def bad(layer, x, g, eps, k, renorm=True):
        h = mo.rms_norm(x, g, eps)
        y, idx, w, _ = mo.moe_layer(layer, h, k, renorm, residual=h)
        return y, idx, w, h
    _patch(monkeypatch, "moe_block", bad)
    assert _fails(_norm_pins)


def test_block_routing_on_the_raw_row_is_caught(monkeypatch):
    def bad(layer, x, g, eps, k, renorm=True):
        x64 = np.atleast_2d(np.asarray(x, np.float64))
        h = mo.rms_norm(x64, g, eps)
        lg = mo.qmatvec(layer["router"], x64)
        y, idx, w, _ = mo.moe_layer(layer, h, k, renorm, residual=x64, logits=lg)
        return y, idx, w, h
    _patch(monkeypatch, "moe_block", bad)
    assert _fails(_norm_pins)


def test_high_bits_first_unpack_is_caught(monkeypatch):
    def bad(words, bits, cols):
        c = _unpack(words, bits, cols)
        per = 32 // bits
        return c.reshape(c.shape[:-1] + (cols // per, per))[..., ::-1].reshape(c.shape)
    _patch(monkeypatch, "unpack_codes", bad)
    assert _fails(_format_pins)


def test_bias_inside_the_product_is_caught(monkeypatch):
    def bad(qt):
        codes = mo.unpack_codes(qt["q"], qt["bits"], qt["cols"]).astype(np.float32)
        s = np.repeat(mo.bf16_bits_to_f32(qt["scales"]), qt["group_size"], axis=-1)
        b = np.repeat(mo.bf16_bits_to_f32(qt["biases"]), qt["group_size"], axis=-1)
        return (s * (codes + b)).astype(np.float32)
    _patch(monkeypatch, "dequantize", bad)
    assert _fails(_format_pins)


def test_dropped_bias_is_caught(monkeypatch):
    def bad(qt):
        q2 = dict(qt)
        q2["biases"] = np.zeros_like(np.asarray(qt["biases"]))
        return _dequant(q2)
    _patch(monkeypatch, "dequantize", bad)
    assert _fails(_format_pins)


def test_scales_tiled_instead_of_repeated_is_caught(monkeypatch):
    def bad(qt):
        codes = mo.unpack_codes(qt["q"], qt["bits"], qt["cols"]).astype(np.float32)
        s = np.tile(mo.bf16_bits_to_f32(qt["scales"]), qt["group_size"])
        b = np.tile(mo.bf16_bits_to_f32(qt["biases"]), qt["group_size"])
        return (s * codes + b).astype(np.float32)
    _patch(monkeypatch, "dequantize", bad)
    assert _fails(_format_pins)


def test_transposed_weight_in_matvec_is_caught(monkeypatch):
    def bad(qt, x):
        w = mo.dequantize(qt).astype(np.float64)
        x64 = np.asarray(x, np.float64)
        if w.shape[0] == w.shape[1]:
            return x64 @ w
        return x64[:, : w.shape[0]] @ w[:, : w.shape[0]]
    _patch(monkeypatch, "qmatvec", bad)
    assert _fails(_format_pins)


def test_ties_to_higher_index_are_caught(monkeypatch):
    def bad(scores, k):
        s = np.asarray(scores, np.float64)
        if s.ndim == 1:
            s = s[None, :]
        e = s.shape[1]
        idx, val = _top_k(s[:, ::-1], k)
        return (e - 1 - idx).astype(np.int32), val
    _patch(monkeypatch, "top_k", bad)
    assert _fails(_route_pins)


def test_missing_renormalization_is_caught(monkeypatch):
    _patch(monkeypatch, "route", lambda logits, k, renorm=True: _route(logits, k, False))
    assert _fails(_route_pins)


def test_silu_sign_error_is_caught(monkeypatch):
    def bad(g):
        g = np.asarray(g, np.float64)
        with np.errstate(over="ignore"):
            return g / (1.0 + np.exp(g))
    _patch(monkeypatch, "silu", bad)
    assert _fails(_layer_pins)


def test_swapped_slot_weights_are_caught(monkeypatch):
    def bad(layer, x, idx, w, residual=None):
        return _moe_experts(layer, x, idx, np.asarray(w)[:, ::-1], residual)
    _patch(monkeypatch, "moe_experts", bad)
    assert _fails(_layer_pins)


def test_shared_expert_without_sigmoid_is_caught(monkeypatch):
    def bad(layer, x, idx, w, residual=None):
        sh = layer.get("shared")
        if sh is None:
            return _moe_experts(layer, x, idx, w, residual)
        lay = dict(layer)
        lay["shared"] = None
        y = _moe_experts(lay, x, idx, w, residual)
        x64 = np.asarray(x, np.float64).reshape(-1, np.asarray(x).shape[-1])
        g = x64 @ mo._deq64(sh["gate"]).T
        u = x64 @ mo._deq64(sh["up"]).T
        return y + mo.swiglu(g, u) @ mo._deq64(sh["down"]).T     # gate scale dropped
    _patch(monkeypatch, "moe_experts", bad)
    assert _fails(_layer_pins)


def test_bf16_truncation_instead_of_rounding_is_caught(monkeypatch):
    def bad(v):
        from fractions import Fraction
        v = Fraction(v)
        if v == 0:
            return 0
        a = abs(v)
        e = a.numerator.bit_length() - a.denominator.bit_length()
        if a < Fraction(2) ** e:
            e -= 1
        m = int(a / Fraction(2) ** (e - 7))          # truncates
        return (0x8000 if v < 0 else 0) | ((e + 127) << 7) | (m - 128)
    _patch(monkeypatch, "bf16_round", bad)
    assert _fails(_requant_pins)


def _requant_with(monkeypatch, rounding=None, lo_from_codes=False):
    """The oracle's requantization with one step changed."""
    from fractions import Fraction

    def bad(qt):
        r = _requant(qt)
        if rounding is None and not lo_from_codes:
            return r
        bits, gs, cols = qt["bits"], qt["group_size"], qt["cols"]
        codes = mo.unpack_codes(qt["q"], bits, cols).reshape(-1, cols // gs, gs)
        s_in = mo.bf16_bits_to_f32(qt["scales"]).reshape(-1, cols // gs)
        b_in = mo.bf16_bits_to_f32(qt["biases"]).reshape(-1, cols // gs)
        q2 = np.zeros(codes.shape, np.uint8)
        for i in range(codes.shape[0]):
            for g in range(codes.shape[1]):
                s, b = Fraction(float(s_in[i, g])), Fraction(float(b_in[i, g]))
                q = [int(c) for c in codes[i, g]]
                lo = s * min(q) + b if lo_from_codes else min(s * c + b for c in q)
                hi = s * max(q) + b if lo_from_codes else max(s * c + b for c in q)
                step = (hi - lo) / 3
                if step != 0:
                    q2[i, g] = [rounding((s * c + b - lo) / step) if rounding else
                                min(3, max(0, round((s * c + b - lo) / step))) for c in q]
        r["q"] = mo._pack_2bit(q2.reshape(np.asarray(r["q"]).shape[:-1] + (cols,)))
        return r
    _patch(monkeypatch, "requant_2bit", bad)


def test_requant_ties_rounded_up_are_caught(monkeypatch):
    import math
    _requant_with(monkeypatch, rounding=lambda v: math.floor(v + 0.5))
    assert _fails(_requant_pins)


def test_requant_minimum_taken_at_the_smallest_code_is_caught(monkeypatch):
    # right only for positive scales: a negative scale puts the minimum at
    # the largest code
    _requant_with(monkeypatch, lo_from_codes=True)
    assert _fails(_requant_pins)


def test_requant_high_bits_first_packing_is_caught(monkeypatch):
    def bad(codes):
        c = np.asarray(codes, dtype=np.uint32)
        c = c.reshape(c.shape[:-1] + (c.shape[-1] // 16, 16))
        words = np.zeros(c.shape[:-1], dtype=np.uint32)
        for j in range(16):
            words |= c[..., j] << np.uint32(30 - 2 * j)
        return words
    monkeypatch.setattr(mo, "_pack_2bit", bad)
    assert _fails(_requant_pins)


@pytest.mark.parametrize("name", ["unpack_codes", "dequantize", "route", "moe_experts",
                                  "bf16_round", "requant_2bit", "rms_norm", "moe_block",
                                  "fp4_e2m1", "e8m0_scale"])
def test_each_patch_target_exists(name):
    assert callable(getattr(mo, name))
