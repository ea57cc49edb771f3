"""GPU checks of host-resident experts streamed into device slots
(moe_stream_experts; flash-moe-inference skill page: K expert reads per layer
into expert buffers, the page cache as the LRU).

Acceptance: the step run on the slots equals the step on the fully resident
layer bit for bit (the same kernels on the same bytes), through hits, misses
and evictions; the copy counts follow the LRU; the oracle agrees within the
decode tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
from quantized_moe_expert_unpack_amd import moeq, synth
from tests.gpu_util import dev, gapped_tokens, rel_l2_rows, say, to_dev

pytestmark = pytest.mark.gpu


def _streamed_step(cache, L, cfg, x):
    xd = to_dev(x)
    idx, w = moeq.moe_route(L.router, xd, cfg.experts, cfg.top_k, renorm=cfg.renorm)
    slot_idx, n = cache.stream(idx.cpu().numpy())
    y = moeq.moe_expert_forward(cache.layer, xd, to_dev(slot_idx), w)
    y_res = moeq.moe_expert_forward(L, xd, idx, w)
    torch.cuda.synchronize()
    return y, y_res, idx.cpu().numpy(), slot_idx, n


@pytest.mark.parametrize("name,slots", [("c1", 3), ("c1_shared", 4), ("c1_32experts", 8)])
def test_streamed_equals_resident(name, slots):
    cfg = {"c1": synth.CONFIGS["c1"],
           "c1_shared": synth.scaled(synth.CONFIGS["c1"], shared_inter=128, shared_bits=4,
                                     shared_gate_bits=8, seed=91),
           "c1_32experts": synth.scaled(synth.CONFIGS["c1"], experts=32, top_k=4, seed=92)}[name]
    host = synth.host_layer(cfg, 0, threads=4)
    L = moeq.MoELayer.from_host(host, dev())
    cache = moeq.ExpertCache(host, slots, L, dev())
    xs = gapped_tokens(cfg, host, 0, 6, m=1)
    copied = 0
    for t in range(6):
        say(f"{name} token {t}")
        y, y_res, idx, slot_idx, n = _streamed_step(cache, L, cfg, xs[t])
        assert torch.equal(y, y_res)
        held = cache.slot_expert
        assert all(held[s] == e for s, e in zip(slot_idx.ravel(), idx.ravel()))
        copied += n
        ry, _, _, _ = oracle.moe_layer(host, xs[t], cfg.top_k, cfg.renorm)
        assert rel_l2_rows(y.cpu().numpy(), ry).max() <= 1e-4
    # the same token again: every expert is already in a slot
    _, _, _, _, n = _streamed_step(cache, L, cfg, xs[5])
    assert n == 0
    say(f"  {copied} experts copied over 6 tokens")


def test_lru_order_and_too_few_slots():
    cfg = synth.scaled(synth.CONFIGS["c1"], experts=8, top_k=2, seed=93)
    host = synth.host_layer(cfg, 0, threads=4)
    L = moeq.MoELayer.from_host(host, dev())
    cache = moeq.ExpertCache(host, 3, L, dev())
    _, n = cache.stream(np.array([[0, 1]]))
    assert n == 2 and sorted(cache.slot_expert.tolist()) == [-1, 0, 1]
    _, n = cache.stream(np.array([[2, 0]]))          # fills the empty slot, 0 is a hit
    assert n == 1
    _, n = cache.stream(np.array([[3, 0]]))          # evicts 1 (least recently used)
    assert n == 1 and 1 not in cache.slot_expert.tolist() and 2 in cache.slot_expert.tolist()
    with pytest.raises(moeq.MoeqError):
        cache.stream(np.array([[4, 5], [6, 7]]))     # 4 distinct experts, 3 slots
    # the copies went out; a forward on the slots matches the resident layer
    x = gapped_tokens(cfg, host, 0, 1, m=1)[0]            # at most 2 experts: they fit
    y, y_res, _, _, _ = _streamed_step(cache, L, cfg, x)
    assert torch.equal(y, y_res)


def test_397b_shaped_layer_streamed():
    # one 397B-A17B-shaped layer (512 experts of 3 x 4096 x 1024 at 4 bits)
    # with 8 slots: two tokens, top-4
    cfg = synth.CONFIGS["c3"]
    host = synth.host_layer(cfg, 0, threads=16)
    L = moeq.MoELayer.from_host(host, dev())
    cache = moeq.ExpertCache(host, 8, L, dev())
    xs = gapped_tokens(cfg, host, 0, 2, m=1)
    for t in range(2):
        y, y_res, _, _, n = _streamed_step(cache, L, cfg, xs[t])
        say(f"c3 token {t}: {n} experts copied")
        assert torch.equal(y, y_res)
