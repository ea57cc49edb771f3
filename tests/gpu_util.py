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
