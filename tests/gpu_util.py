"""Helpers shared by the GPU parity tests (no method arithmetic here: the
expected values always come from the oracle)."""

import sys

import numpy as np
import torch

import oracle
from quantized_moe_expert_unpack_amd import synth

GAP = 1e-4          # minimum gap between consecutive top-(K+1) router scores


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def rel_l2_rows(got, ref):
    """Per-row relative L2 error ||got_t - ref_t|| / ||ref_t||."""
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return num / np.maximum(den, 1e-300)


def topk_gaps_ok(logits, k, gap=GAP):
    """True per row when the top-(k+1) scores are pairwise >= gap apart."""
    s = -np.sort(-np.asarray(logits, np.float64), axis=-1)[..., : k + 1]
    return np.all(np.diff(-s, axis=-1) >= gap, axis=-1) if s.shape[-1] > 1 else np.ones(s.shape[0], bool)


def gapped_tokens(cfg, layer_host, layer_idx, n_tokens, m=1):
    """Decode activations for ``n_tokens`` token slots whose oracle router
    scores satisfy the top-K gap, redrawing a slot's x from the next sub-seed
    when they do not.  Returns ``[n_tokens, m, H]`` fp32."""
    out = []
    for t in range(n_tokens):
        for sub in range(100):
            x = synth.decode_x(cfg, layer_idx, t, sub=sub, m=m)
            lg = oracle.qmatvec(layer_host["router"], x)
            if topk_gaps_ok(lg, cfg.top_k).all():
                out.append(x)
                break
        else:
            raise AssertionError("no gapped draw found")
    return np.stack(out)


def to_dev(a, device=None):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device or dev())


def bf16_dev(bits_u16, device=None):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(device or dev())


def bf16_bits_to_f32(bits_u16):
    return (np.asarray(bits_u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def oracle_requantized_layer(src_host, experts, threads=16):
    """The oracle's 2-bit form of a 4-bit host layer, for the experts listed
    (oracle.requant_2bit_fast per expert matrix) and the shared expert's FFN;
    the router and the shared expert gate stay as they are.  Stacks are dicts
    indexed by expert."""
    from concurrent.futures import ThreadPoolExecutor

    experts = [int(e) for e in experts]
    out = dict(src_host)
    jobs = [(name, e) for name in ("gate", "up", "down") for e in experts]

    def one(job):
        name, e = job
        return job, oracle.requant_2bit_fast(oracle.expert_slice(src_host[name], e))

    with ThreadPoolExecutor(threads) as ex:
        done = dict(ex.map(one, jobs))
    for name in ("gate", "up", "down"):
        t = src_host[name]
        out[name] = {"q": {e: done[(name, e)]["q"] for e in experts},
                     "scales": {e: done[(name, e)]["scales"] for e in experts},
                     "biases": {e: done[(name, e)]["biases"] for e in experts},
                     "rows": t["rows"], "cols": t["cols"], "bits": 2,
                     "group_size": t["group_size"], "batch": t["batch"]}
    sh = src_host.get("shared")
    if sh is not None:
        out["shared"] = {k: (v if k == "expert_gate" else oracle.requant_2bit_fast(v))
                         for k, v in sh.items()}
    return out


def assert_same_2bit_experts(dev_layer, host2, experts):
    """The device's requantized words, scales and biases of the listed
    experts (and of the shared expert) equal the oracle's, bit for bit."""
    for name in ("gate", "up", "down"):
        t = getattr(dev_layer, name)
        for e in experts:
            e = int(e)
            assert np.array_equal(t.q[e].cpu().numpy().view(np.uint32), host2[name]["q"][e]), (name, e)
            assert np.array_equal(t.scales[e].cpu().numpy().view(np.uint16), host2[name]["scales"][e])
            assert np.array_equal(t.biases[e].cpu().numpy().view(np.uint16), host2[name]["biases"][e])
    if dev_layer.shared is not None:
        for name in ("gate", "up", "down"):
            t, h = dev_layer.shared[name], host2["shared"][name]
            assert np.array_equal(t.q.cpu().numpy().view(np.uint32).reshape(h["q"].shape), h["q"])
            assert np.array_equal(t.scales.cpu().numpy().view(np.uint16).reshape(h["scales"].shape),
                                  h["scales"])
            assert np.array_equal(t.biases.cpu().numpy().view(np.uint16).reshape(h["biases"].shape),
                                  h["biases"])
