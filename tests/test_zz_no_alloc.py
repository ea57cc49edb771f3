"""GPU: moe_forward_noalloc, the allocation-free form of moe_forward whose
workspace is the library's static per-device array, against moe_forward on
a caller-allocated workspace (and against the oracle).

Acceptance (as for moe_forward): top-K indices bit-exact, max per-row
relative L2 <= 1e-4 against the oracle; here, against moe_forward, the same
bits, since both run the same kernels on the same inputs.  Two calls in a
row with the second smaller, a change of layer shape (the array is cleared
for the new layout), the many-token form, and the size limit.
"""

import functools

import numpy as np
import pytest
import torch

import oracle
from quantized_moe_expert_unpack_amd import moeq, synth
from tests.gpu_util import dev, gapped_tokens, rel_l2_rows, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-4


@functools.lru_cache(maxsize=2)
def _layer(name):
    cfg = synth.CONFIGS[name]
    host = synth.host_layer(cfg, 0, threads=16)
    return cfg, host, moeq.MoELayer.from_host(host, dev())


def _both(cfg, host, L, x):
    xd = to_dev(x)
    y_ref, idx_ref, w_ref = moeq.moe_forward(L, xd, cfg.top_k, renorm=cfg.renorm)
    status = torch.full((4,), -99, dtype=torch.int32, device=dev())
    y, idx, w = moeq.moe_forward_noalloc(L, xd, cfg.top_k, renorm=cfg.renorm, status=status)
    torch.cuda.synchronize()
    assert status[:2].tolist() == [0, 0]
    assert torch.equal(idx, idx_ref)
    assert torch.equal(w, w_ref)
    assert torch.equal(y, y_ref)
    ry, ridx, _, _ = oracle.moe_layer(host, x, cfg.top_k, cfg.renorm)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    err = rel_l2_rows(y.cpu().numpy(), ry).max()
    say(f"  {cfg.name} M={x.shape[0]}: same bits as moe_forward, max rel-L2 {err:.2e}")
    assert err <= TOL


def test_two_calls_in_a_row_the_second_smaller():
    cfg, host, L = _layer("c2")
    x = gapped_tokens(cfg, host, 0, 1, m=4)[0]
    _both(cfg, host, L, x)          # one launch, four tokens
    _both(cfg, host, L, x[:1])      # then one token on the array as the first call left it


def test_layout_changes_and_the_many_token_form():
    cfg3, host3, L3 = _layer("c3")
    x3 = gapped_tokens(cfg3, host3, 0, 1, m=16)[0]
    _both(cfg3, host3, L3, x3)         # 397B-A17B shapes: route launch + batched experts
    _both(cfg3, host3, L3, x3[:3])     # one launch, three tokens
    cfg2, host2, L2 = _layer("c2")
    x2 = gapped_tokens(cfg2, host2, 0, 1, m=2)[0]
    _both(cfg2, host2, L2, x2)         # back to the 30B-A3B shapes: the array is cleared first


def test_sizes_beyond_the_array_are_refused():
    cfg, host, L = _layer("c3")
    x = torch.zeros((256, cfg.hidden), dtype=torch.float32, device=dev())
    assert moeq.workspace_size(L, 256, cfg.top_k, moeq.PATH_FORWARD) > 16 << 20
    with pytest.raises(moeq.MoeqError) as e:
        moeq.moe_forward_noalloc(L, x, cfg.top_k)
    assert e.value.status == -8                      # MOEQ_ERR_WORKSPACE, nothing launched
