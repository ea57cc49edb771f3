"""GPU parity of the step with its neighbours fused: RMSNorm before the router
and the experts, the raw row added back in the combine (flash-moe-inference
skill page: the CMD2 chain o_proj -> norm -> routing and moe_combine_residual;
the oracle's ``rms_norm`` and ``moe_block``).

Acceptance: moe_rms_norm per-row relative L2 <= 1e-6 (fp32 arithmetic);
moe_forward_norm top-K indices bit-exact and per-row relative L2 <= 1e-4, in
the one-launch form (8-bit router, M <= 4), the per-token form and the
batched form, with and without a shared expert; reruns bitwise equal.  The
norm after the combine (rms_norm(y) * w2, the norm closing the page's CMD3):
y unchanged bit for bit, y_norm within 1e-6 of the oracle's norm of the
library's own y and within 1e-4 of the oracle's whole block.
"""

import functools

import numpy as np
import pytest
import torch

import oracle
from quantized_moe_expert_unpack_amd import moeq, synth
from tests.gpu_util import dev, rel_l2_rows, say, to_dev, topk_gaps_ok

pytestmark = pytest.mark.gpu

EPS = 1e-6
SCALE = 4.0          # the residual stream's rows are larger than N(0, 1); exact scaling


@pytest.mark.parametrize("m,h", [(1, 256), (5, 2048), (37, 4096), (3, 160)])
def test_rms_norm(m, h):
    rng = np.random.default_rng(m * 7 + h)
    x = (rng.standard_normal((m, h)) * rng.uniform(0.1, 10.0, (m, 1))).astype(np.float32)
    g = rng.uniform(0.5, 1.5, h).astype(np.float32)
    got = moeq.moe_rms_norm(to_dev(x), to_dev(g), EPS).cpu().numpy()
    ref = oracle.rms_norm(x, g, EPS)
    assert rel_l2_rows(got, ref).max() <= 1e-6


def _gapped_norm_tokens(cfg, host, g, layer_idx, slot, m):
    """Rows whose normalized router scores satisfy the top-K gap (redrawn
    from the next sub-seed otherwise)."""
    for sub in range(100):
        x = synth.decode_x(cfg, layer_idx, slot, sub=sub, m=m) * np.float32(SCALE)
        lg = oracle.qmatvec(host["router"], oracle.rms_norm(x, g, EPS))
        if topk_gaps_ok(lg, cfg.top_k).all():
            return x
    raise AssertionError("no gapped draw found")


VARIANTS = {
    "c1": synth.CONFIGS["c1"],
    "c1_shared": synth.scaled(synth.CONFIGS["c1"], shared_inter=128, shared_bits=4,
                              shared_gate_bits=8, seed=71),
    "c1_4bit_router": synth.scaled(synth.CONFIGS["c1"], router_bits=4, seed=72),
    "c2": synth.CONFIGS["c2"],
    "c3": synth.CONFIGS["c3"],
}


@functools.lru_cache(maxsize=3)
def _layer(name):
    cfg = VARIANTS[name]
    host = synth.host_layer(cfg, 0, threads=16)
    return cfg, host, moeq.MoELayer.from_host(host, dev()), synth.norm_weight(cfg, 0)


def _check(name, m, slot=1):
    cfg, host, L, g = _layer(name)
    say(f"moe_forward_norm {name} M={m}")
    x = _gapped_norm_tokens(cfg, host, g, 0, slot, m)
    y, idx, w = moeq.moe_forward_norm(L, to_dev(x), cfg.top_k, to_dev(g), EPS, cfg.renorm)
    torch.cuda.synchronize()
    ry, ridx, rw, _ = oracle.moe_block(host, x, g, EPS, cfg.top_k, cfg.renorm)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    err = rel_l2_rows(y.cpu().numpy(), ry).max()
    say(f"  max rel-L2 {err:.3e}")
    assert err <= 1e-4
    return x, y


@pytest.mark.parametrize("m", [1, 2, 4, 7, 24])
def test_c1_all_forms(m):
    # M <= 4: one launch; 7: per-token launches; 24: batched by expert
    _check("c1", m)


@pytest.mark.parametrize("m", [1, 3, 20])
def test_c1_shared_expert(m):
    _check("c1_shared", m)


def test_router_not_8bit_takes_the_separate_norm_launch():
    _check("c1_4bit_router", 2)


def test_c2_shaped_layer():
    _check("c2", 1)


def test_c3_shaped_layer_with_shared_expert():
    _check("c3", 1)


def test_reruns_are_bitwise_equal_and_workspace_is_reused():
    cfg, host, L, g = _layer("c1_shared")
    x = _gapped_norm_tokens(cfg, host, g, 0, 3, 2)
    xd, gd = to_dev(x), to_dev(g)
    ws = moeq.workspace(L, 24, cfg.top_k, moeq.PATH_FORWARD_NORM, dev())
    y1, _, _ = moeq.moe_forward_norm(L, xd, cfg.top_k, gd, EPS, ws=ws)
    x24 = _gapped_norm_tokens(cfg, host, g, 0, 4, 24)
    y24, _, _ = moeq.moe_forward_norm(L, to_dev(x24), cfg.top_k, gd, EPS, ws=ws)
    y2, _, _ = moeq.moe_forward_norm(L, xd, cfg.top_k, gd, EPS, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ry, _, _, _ = oracle.moe_block(host, x24, g, EPS, cfg.top_k)
    assert rel_l2_rows(y24.cpu().numpy(), ry).max() <= 1e-4


def test_norm_equals_rms_norm_then_moe_forward_with_residual():
    # the fused launch against the library's own two-call composition
    cfg, host, L, g = _layer("c1")
    x = _gapped_norm_tokens(cfg, host, g, 0, 5, 3)
    xd, gd = to_dev(x), to_dev(g)
    y, idx, _ = moeq.moe_forward_norm(L, xd, cfg.top_k, gd, EPS)
    h = moeq.moe_rms_norm(xd, gd, EPS)
    y2, idx2, _ = moeq.moe_forward(L, h, cfg.top_k, residual=xd)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert rel_l2_rows(y.cpu().numpy(), y2.cpu().numpy().astype(np.float64)).max() <= 1e-5


@pytest.mark.parametrize("name,m", [("c1", 2), ("c1_shared", 7), ("c1_4bit_router", 3), ("c2", 1)])
def test_norm_after_the_combine(name, m):
    # one-launch form (c1, c2), per-token form (7 tokens), separate-norm form
    cfg, host, L, g = _layer(name)
    say(f"moe_forward_norm + post norm {name} M={m}")
    x = _gapped_norm_tokens(cfg, host, g, 0, 6, m)
    g2 = np.random.default_rng(m).uniform(0.5, 1.5, cfg.hidden).astype(np.float32)
    xd, gd = to_dev(x), to_dev(g)
    y, idx, _ = moeq.moe_forward_norm(L, xd, cfg.top_k, gd, EPS, cfg.renorm)
    y2, idx2, _, yn = moeq.moe_forward_norm(L, xd, cfg.top_k, gd, EPS, cfg.renorm,
                                            post_norm_w=to_dev(g2))
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(idx, idx2)
    yh = y2.cpu().numpy()
    assert rel_l2_rows(yn.cpu().numpy(), oracle.rms_norm(yh, g2, EPS)).max() <= 1e-6
    ry, _, _, _ = oracle.moe_block(host, x, g, EPS, cfg.top_k, cfg.renorm)
    err = rel_l2_rows(yn.cpu().numpy(), oracle.rms_norm(ry, g2, EPS)).max()
    say(f"  y_norm max rel-L2 against the oracle's block {err:.3e}")
    assert err <= 1e-4
