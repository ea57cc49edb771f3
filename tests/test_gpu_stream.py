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


# ---- the device-side form: slot choice and copies on the device ---------------

def _device_step(cache, L, cfg, xd, idx=None, w=None):
    if idx is None:
        idx, w = moeq.moe_route(L.router, xd, cfg.experts, cfg.top_k, renorm=cfg.renorm)
    slot_idx, n = cache.stream_device(idx)
    y = moeq.moe_expert_forward(cache.layer, xd, slot_idx, w)
    y_res = moeq.moe_expert_forward(L, xd, idx, w)
    torch.cuda.synchronize()
    return y, y_res, idx, slot_idx, int(n.item())


def test_device_lru_takes_the_host_lru_decisions():
    # the same index sequence through both caches: same slots, same copies,
    # same state; out-of-range indices map to slot S on both
    cfg = synth.scaled(synth.CONFIGS["c1"], experts=16, top_k=2, seed=94)
    host = synth.host_layer(cfg, 0, threads=4)
    L = moeq.MoELayer.from_host(host, dev())
    S = 5
    ch = moeq.ExpertCache(host, S, L, dev())
    cd = moeq.ExpertCache(host, S, L, dev(), device_lru=True)
    rng = np.random.default_rng(7)
    for call in range(40):
        m = int(rng.integers(1, 3))                   # up to 4 pairs <= 5 slots
        idx = rng.integers(0, 6 if call < 20 else 16, (m, 2)).astype(np.int32)
        if call % 9 == 4:
            idx[0, 1] = -1 if call % 2 else 99
        sh, nh = ch.stream(idx)
        sd, nd = cd.stream_device(to_dev(idx))
        torch.cuda.synchronize()
        assert np.array_equal(sd.cpu().numpy(), sh), (call, idx)
        assert int(nd.item()) == nh
        assert np.array_equal(cd.slot_expert_dev.cpu().numpy(), ch.slot_expert)
        assert np.array_equal(cd.slot_stamp_dev.cpu().numpy()[:S], ch.slot_stamp)
    say("  40 calls: same slots, copies and state")


@pytest.mark.parametrize("name,slots", [("c1", 3), ("c1_shared", 4), ("c1_32experts", 8),
                                        ("c1_gs32", 4)])
def test_device_streamed_equals_resident(name, slots):
    cfg = {"c1": synth.CONFIGS["c1"],
           "c1_shared": synth.scaled(synth.CONFIGS["c1"], shared_inter=128, shared_bits=4,
                                     shared_gate_bits=8, seed=91),
           "c1_32experts": synth.scaled(synth.CONFIGS["c1"], experts=32, top_k=4, seed=92),
           "c1_gs32": synth.scaled(synth.CONFIGS["c1"], group_size=32, seed=95)}[name]
    host = synth.host_layer(cfg, 0, threads=4)
    L = moeq.MoELayer.from_host(host, dev())
    cache = moeq.ExpertCache(host, slots, L, dev(), device_lru=True)
    m = 2 if slots >= 2 * cfg.top_k else 1
    xs = gapped_tokens(cfg, host, 0, 6, m=m)
    copied = 0
    for t in range(6):
        say(f"{name} device-streamed token {t}")
        y, y_res, idx, slot_idx, n = _device_step(cache, L, cfg, to_dev(xs[t]))
        assert torch.equal(y, y_res)
        held = cache.slot_expert_dev.cpu().numpy()
        si, ii = slot_idx.cpu().numpy().ravel(), idx.cpu().numpy().ravel()
        assert all(held[s] == e for s, e in zip(si, ii))
        copied += n
        ry, _, _, _ = oracle.moe_layer(host, xs[t], cfg.top_k, cfg.renorm)
        assert rel_l2_rows(y.cpu().numpy(), ry).max() <= 1e-4
    _, _, _, _, n = _device_step(cache, L, cfg, to_dev(xs[5]))
    assert n == 0
    say(f"  {copied} experts copied over 6 steps")


def test_device_streamed_397b_shaped_layer():
    cfg = synth.CONFIGS["c3"]
    host = synth.host_layer(cfg, 0, threads=16)
    L = moeq.MoELayer.from_host(host, dev())
    cache = moeq.ExpertCache(host, 8, L, dev(), device_lru=True)
    xs = gapped_tokens(cfg, host, 0, 3, m=1)
    for t in range(3):
        y, y_res, _, _, n = _device_step(cache, L, cfg, to_dev(xs[t]))
        say(f"c3 device-streamed token {t}: {n} experts copied")
        assert torch.equal(y, y_res)


def test_device_stream_chain_in_a_graph():
    # route -> slot choice + copies -> forward captured once, replayed over
    # tokens whose experts differ (evictions inside the replays); every
    # replay against the resident layer, with eager work between replays
    cfg = synth.scaled(synth.CONFIGS["c1"], experts=32, top_k=4, seed=96)
    host = synth.host_layer(cfg, 0, threads=4)
    L = moeq.MoELayer.from_host(host, dev())
    cache = moeq.ExpertCache(host, 6, L, dev(), device_lru=True)
    xs = gapped_tokens(cfg, host, 0, 6, m=1)
    xin = to_dev(xs[0])
    idx = torch.empty((1, cfg.top_k), dtype=torch.int32, device=dev())
    w = torch.empty((1, cfg.top_k), dtype=torch.float32, device=dev())
    sidx = torch.empty((1, cfg.top_k), dtype=torch.int32, device=dev())
    ncp = torch.zeros(4, dtype=torch.int32, device=dev())
    y = torch.empty((1, cfg.hidden), dtype=torch.float32, device=dev())
    ws_r = moeq.workspace(L, 1, cfg.top_k, moeq.PATH_ROUTE, dev())
    ws_d = moeq.workspace(L, 1, cfg.top_k, moeq.PATH_DECODE, dev())

    def chain():
        moeq.moe_route(L.router, xin, cfg.experts, cfg.top_k, renorm=cfg.renorm, ws=ws_r, idx=idx, w=w)
        cache.stream_device(idx, slot_idx=sidx, n_copied=ncp)
        moeq.moe_expert_forward(cache.layer, xin, sidx, w, ws=ws_d, y=y)

    chain()                                              # eager once (token 0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        chain()
    torch.cuda.synchronize()
    total = 0
    for t in range(1, 6):
        xin.copy_(to_dev(xs[t]))
        g.replay()
        torch.cuda.synchronize()
        ref, ridx, _ = moeq.moe_forward(L, to_dev(xs[t]), cfg.top_k, cfg.renorm)   # eager, between
        torch.cuda.synchronize()
        assert torch.equal(idx, ridx)
        assert torch.equal(y, moeq.moe_expert_forward(L, xin, idx, w))
        held = cache.slot_expert_dev.cpu().numpy()
        assert all(held[a] == b for a, b in zip(sidx.cpu().numpy().ravel(), idx.cpu().numpy().ravel()))
        total += int(ncp[0].item())
        say(f"  replay {t}: {int(ncp[0].item())} experts copied")
    assert total > 0
