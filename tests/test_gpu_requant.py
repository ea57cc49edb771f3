"""GPU parity of the 2-bit requantization against the oracle (flash-moe-inference
skill page: the 4-bit to 2-bit conversion of the experts).

Acceptance: bit-exact 2-bit words, scales and biases (the codes are integer
decisions and the stored values are exactly rounded on both sides), at small
sizes that span several blocks and end on a ragged block, and on sampled rows
of a full-size expert stack.
"""

import numpy as np
import pytest
import torch

import oracle
from quantized_moe_expert_unpack_amd import moeq, synth
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _host(t: torch.Tensor, dtype):
    return t.cpu().numpy().view(dtype)


def _check(host, got, rows=None):
    ref = oracle.requant_2bit(host)
    q = _host(got.q, np.uint32).reshape(-1, host["cols"] // 16)
    s = _host(got.scales, np.uint16).reshape(-1, host["cols"] // host["group_size"])
    b = _host(got.biases, np.uint16).reshape(s.shape)
    if rows is not None:
        q, s, b = q[rows], s[rows], b[rows]
    rq = ref["q"].reshape(q.shape)
    bad = np.nonzero((q != rq).any(axis=1))[0]
    assert bad.size == 0, f"code words differ in rows {bad[:8]}"
    assert np.array_equal(s, ref["scales"].reshape(s.shape)), "scales differ"
    assert np.array_equal(b, ref["biases"].reshape(b.shape)), "biases differ"


@pytest.mark.parametrize("bits,gs", [(4, 64), (4, 128), (8, 64), (8, 128)])
@pytest.mark.parametrize("batch,rows,cols", [(3, 37, 384), (1, 1, 128), (2, 129, 256)])
def test_requant_matches_the_oracle(bits, gs, batch, rows, cols):
    say(f"requant bits={bits} gs={gs} shape=({batch},{rows},{cols})")
    host = synth.requant_source((41, bits, gs, rows), batch, rows, cols, bits, gs)
    got = moeq.requant_2bit(moeq.QTensor.from_host(host, dev()))
    torch.cuda.synchronize()
    assert got.bits == 2 and got.group_size == gs
    _check(host, got)


def test_one_group_and_reruns_are_bitwise_equal():
    host = synth.requant_source((42,), 1, 1, 64, 4, 64, narrow=1.0)
    W = moeq.QTensor.from_host(host, dev())
    a = moeq.requant_2bit(W)
    b = moeq.requant_2bit(W)
    torch.cuda.synchronize()
    _check(host, a)
    assert torch.equal(a.q, b.q) and torch.equal(a.scales, b.scales)


def test_requantized_experts_run_through_the_decode_path():
    # a 4-bit layer requantized on the device computes what the oracle
    # computes with the oracle's requantized weights
    from tests.gpu_util import gapped_tokens, rel_l2_rows, to_dev
    cfg = synth.scaled(synth.CONFIGS["c1"], seed=43)
    host = synth.host_layer(cfg, 0, threads=4)
    L4 = moeq.MoELayer.from_host(host, dev())
    L2 = moeq.MoELayer(L4.router, moeq.requant_2bit(L4.gate), moeq.requant_2bit(L4.up),
                       moeq.requant_2bit(L4.down))
    host2 = dict(host, gate=oracle.requant_2bit(host["gate"]), up=oracle.requant_2bit(host["up"]),
                 down=oracle.requant_2bit(host["down"]))
    x = gapped_tokens(cfg, host2, 0, 1, m=3)[0]
    y, idx, w = moeq.moe_forward(L2, to_dev(x), cfg.top_k, cfg.renorm)
    torch.cuda.synchronize()
    ry, ridx, _, _ = oracle.moe_layer(host2, x, cfg.top_k, cfg.renorm)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert rel_l2_rows(y.cpu().numpy(), ry).max() <= 1e-4


@pytest.mark.parametrize("bits", [4, 8])
def test_full_size_expert_stack_sampled_rows(bits):
    # the 397B-A17B-shaped expert stack [512][1024][4096] (gate or up) at 4
    # bits, and a quarter of it at 8 bits; 24 sampled rows checked bit-exactly
    E = 512 if bits == 4 else 128
    I, H, gs = 1024, 4096, 64
    say(f"requant full stack bits={bits} [{E}][{I}][{H}]")
    q, s, b = synth.requant_source_device(44 + bits, E, I, H, bits, gs, dev())
    W = moeq.QTensor(q, s, b, E, I, H, bits, gs)
    got = moeq.requant_2bit(W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(bits)
    rows = np.sort(rng.choice(E * I, 24, replace=False))
    rows[0], rows[-1] = 0, E * I - 1
    qh = q.reshape(E * I, -1)[torch.from_numpy(rows).to(dev())]
    sh = s.reshape(E * I, -1)[torch.from_numpy(rows).to(dev())]
    bh = b.reshape(E * I, -1)[torch.from_numpy(rows).to(dev())]
    host = {"q": _host(qh, np.uint32), "scales": _host(sh, np.uint16), "biases": _host(bh, np.uint16),
            "batch": 1, "rows": len(rows), "cols": H, "bits": bits, "group_size": gs}
    _check(host, got, rows=rows)
