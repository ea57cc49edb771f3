"""Pins for the oracle's RMSNorm and the MoE step with the norm before it and
the residual after it (flash-moe-inference skill page: the per-layer
pipeline, CMD2 o_proj + norm + routing, the two-pass ``rms_norm_pass1/2`` and
``moe_combine_residual``; danveloper/flash-moe issue thread, "Definitive
finding": o_proj -> residual_add -> rms_norm -> routing gate matvec).

Closed forms worked by hand (a 3-4 row, constant rows with and without
eps), invariants the definition implies (scale invariance without eps, unit
mean square, the weight applied elementwise), and for the block: routing
and experts see the normalized row (scale invariance of y - x), the residual
is the raw row, and the layer on the normalized row brute-forced with
exactly rounded sums.
"""

import math

import numpy as np
import pytest

import oracle
from quantized_moe_expert_unpack_amd import synth
from tests import test_oracle_route_ffn as tr


def test_three_four_row():
    # mean square (9 + 16)/2 = 12.5, sqrt = 5/sqrt(2): h = (3, 4) * sqrt(2)/5
    h = oracle.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert np.allclose(h[0], [3 * math.sqrt(2) / 5, 4 * math.sqrt(2) / 5], rtol=1e-15, atol=0)


@pytest.mark.parametrize("c,eps,want", [(2.0, 0.0, 1.0), (-0.5, 0.0, -1.0),
                                        (1e-3, 1e-6, 1 / math.sqrt(2)),
                                        (3.0, 7.0, 3.0 / 4.0)])
def test_constant_rows(c, eps, want):
    # every element c: h = c / sqrt(c^2 + eps)  (1e-3 with eps 1e-6: 1/sqrt 2;
    # 3 with eps 7: 3/4)
    h = oracle.rms_norm(np.full((2, 64), c), np.ones(64), eps)
    assert np.allclose(h, want, rtol=1e-14, atol=0)


def test_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 256))
    g = rng.uniform(0.5, 1.5, 256)
    h1 = oracle.rms_norm(x, np.ones(256), 0.0)
    assert np.allclose(np.mean(h1 * h1, axis=1), 1.0, rtol=1e-13)          # unit mean square
    assert np.allclose(oracle.rms_norm(37.5 * x, np.ones(256), 0.0), h1, rtol=1e-13)
    assert np.allclose(oracle.rms_norm(-2.0 * x, np.ones(256), 0.0), -h1, rtol=1e-13)
    assert np.allclose(oracle.rms_norm(x, g, 0.0), h1 * g[None, :], rtol=1e-14)
    # rows are independent
    assert np.allclose(oracle.rms_norm(x[2:3], g, 1e-6), oracle.rms_norm(x, g, 1e-6)[2:3], rtol=0)
    with pytest.raises(ValueError):
        oracle.rms_norm(x, np.ones(255), 0.0)


def _cfg(shared=False):
    return tr._tiny_cfg(shared=shared, seed=31)


@pytest.mark.parametrize("shared", [False, True])
def test_block_brute_force(shared):
    cfg = _cfg(shared)
    layer = synth.host_layer(cfg, 0, threads=1)
    x = synth.decode_x(cfg, 0, 0, m=2) * 3.0
    g = np.random.default_rng(6).uniform(0.5, 1.5, cfg.hidden)
    eps = 1e-5
    y, idx, w, h = oracle.moe_block(layer, x, g, eps, cfg.top_k)
    for t in range(2):
        xt = x[t].astype(np.float64).tolist()
        ms = math.fsum(v * v for v in xt) / len(xt)
        ht = [v / math.sqrt(ms + eps) * gv for v, gv in zip(xt, g.tolist())]
        assert np.allclose(h[t], ht, rtol=1e-14, atol=0)
        rw = tr._deq_py(layer["router"])
        lg = [tr._dot(r, ht) for r in rw]
        assert idx[t].tolist() == tr._brute_topk(lg, cfg.top_k)
        ref = tr._brute_layer(layer, ht, idx[t].tolist(), w[t].tolist())
        want = [a + b for a, b in zip(xt, ref)]                 # the raw row is the residual
        assert np.allclose(y[t], want, rtol=1e-11, atol=1e-11 * max(map(abs, want)))


def test_block_routes_and_runs_on_the_normalized_row():
    # without eps, h does not change when x is scaled, so y - x does not
    # either; routing or experts fed the raw row would break this
    cfg = _cfg(True)
    layer = synth.host_layer(cfg, 0, threads=1)
    x = synth.decode_x(cfg, 0, 1, m=3)
    g = np.random.default_rng(7).uniform(0.5, 1.5, cfg.hidden)
    y1, i1, w1, _ = oracle.moe_block(layer, x, g, 0.0, cfg.top_k)
    y2, i2, w2, _ = oracle.moe_block(layer, 4.0 * x, g, 0.0, cfg.top_k)   # exact scaling
    assert np.array_equal(i1, i2) and np.allclose(w1, w2, rtol=1e-13)
    assert np.allclose(y1 - x, y2 - 4.0 * x, rtol=1e-10, atol=1e-12)
    y0, _, _, _ = oracle.moe_layer(layer, x, cfg.top_k)
    assert not np.allclose(y1 - x, y0, rtol=1e-3)              # differs from the un-normalized step
