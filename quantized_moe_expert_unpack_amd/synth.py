"""Seeded synthetic inputs for the quantized MoE step.

This module only draws random data and encodes it in the storage format
(uint32 words, bf16 bit patterns).  It holds none of the step's arithmetic:
no unpacking, dequantization, matrix products, routing or activation.  Both
the HIP path (through the binding) and the CPU oracle consume exactly the
arrays made here.

Every weight matrix is drawn from its own ``numpy.random.SeedSequence([seed,
layer, expert, tensor])`` stream, so any single expert of any layer can be
regenerated on its own (the oracle never needs the whole multi-GB model in
host memory).

The recipes follow the workloads named for the method: uniform codes (random
words make every packed field uniform), scales ``U(0.005, 0.02)`` rounded to
bf16, and biases at the code midpoint ``-2**(bits-1) * scale`` plus
``N(0, 0.001)`` noise, rounded to bf16 (for 4-bit codes this is
``-8 * scale``).  The 2-bit experts of the 397B-A17B-shaped batched decode
are the 397B-A17B-shaped decode's own 4-bit layers requantized to 2 bits;
the requantization is a library op (and an oracle function) and is not done
here: this module draws the 4-bit source (``source_config``).  Activations
are fp32 ``N(0, 1)`` (decode) or bf16-rounded ``N(0, 1)`` (prefill).  Prefill
router logits are ``log p_rank(e) + Gumbel`` with Zipf(1.1) rank
probabilities over a seeded permutation of the experts.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

GROUP = 64

# tensor ids inside the seed tuple
T_GATE, T_UP, T_DOWN, T_ROUTER, T_SH_GATE, T_SH_UP, T_SH_DOWN, T_SH_EG = range(8)
T_X = 16          # decode activations
T_XB = 17         # prefill activations
T_LOGIT = 18      # prefill router logits
T_PERM = 19       # Zipf rank permutation


@dataclass(frozen=True)
class MoEConfig:
    """Shape and storage of one MoE layer (plus how many layers/tokens)."""
    name: str
    hidden: int
    experts: int
    top_k: int
    inter: int
    expert_bits: int
    router_bits: int = 8
    group_size: int = GROUP
    shared_inter: int = 0           # 0: no shared expert
    shared_bits: int = 0            # bits of the shared expert FFN
    shared_gate_bits: int = 8       # bits of the shared_expert_gate row
    layers: int = 1
    tokens: int = 1                 # M per call
    seed: int = 0
    renorm: bool = True
    requant_from: int = 0           # 4: the experts are this config's 4-bit draws requantized to 2 bits
    expert_mode: str = "affine"     # "mxfp4": E2M1 experts, E8M0 scale per 32 columns
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def has_shared(self) -> bool:
        return self.shared_inter > 0


CONFIGS = {
    # tiny single-token layer: 4-bit experts, 8-bit router
    "c1": MoEConfig("c1-tiny", hidden=256, experts=8, top_k=2, inter=128,
                    expert_bits=4, router_bits=8, layers=1, tokens=1, seed=1),
    # 30B-A3B-shaped decode: 8-bit router and experts, 48 independent layers
    "c2": MoEConfig("c2-30b-a3b-decode", hidden=2048, experts=128, top_k=8,
                    inter=768, expert_bits=8, router_bits=8, layers=48,
                    tokens=1, seed=2),
    # 397B-A17B-shaped decode: 4-bit experts + 4-bit shared expert, 8-bit gates
    "c3": MoEConfig("c3-397b-a17b-decode", hidden=4096, experts=512, top_k=4,
                    inter=1024, expert_bits=4, router_bits=8,
                    shared_inter=1024, shared_bits=4, shared_gate_bits=8,
                    layers=8, tokens=1, seed=3),
    # prefill gather_qmm on the 30B-A3B shapes (logits given, Zipf loads)
    "c4": MoEConfig("c4-30b-a3b-prefill", hidden=2048, experts=128, top_k=8,
                    inter=768, expert_bits=8, router_bits=8, layers=2,
                    tokens=16384, seed=4),
    # the prefill on the same shapes with mxfp4 experts (group size 32)
    "c4_mxfp4": MoEConfig("c4-30b-a3b-prefill-mxfp4", hidden=2048, experts=128, top_k=8,
                          inter=768, expert_bits=4, router_bits=8, group_size=32, layers=2,
                          tokens=16384, seed=4, expert_mode="mxfp4"),
    # the 397B-A17B-shaped decode's own layers (seed 3) with the routed and
    # shared experts requantized from 4 to 2 bits (router and shared expert
    # gate kept at 8 bits), batched decode M=64
    "c5": MoEConfig("c5-397b-a17b-2bit-m64", hidden=4096, experts=512, top_k=4,
                    inter=1024, expert_bits=2, router_bits=8,
                    shared_inter=1024, shared_bits=2, shared_gate_bits=8,
                    layers=8, tokens=64, seed=3, requant_from=4),
    # the same batched decode on the same layers kept at 4 bits
    "c5_4bit": MoEConfig("c5-397b-a17b-4bit-m64", hidden=4096, experts=512,
                         top_k=4, inter=1024, expert_bits=4, router_bits=8,
                         shared_inter=1024, shared_bits=4, shared_gate_bits=8,
                         layers=8, tokens=64, seed=3),
}


def scaled(cfg: MoEConfig, **kw) -> MoEConfig:
    return replace(cfg, **kw)


# --------------------------------------------------------------------------
# storage encodings
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and
    return the 16-bit patterns.  Inputs are finite."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_as_f32(bits) -> np.ndarray:
    """bf16 bit patterns as float32 values (a storage decode of generated
    data, used only to build further generated data)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def pack_codes(codes, bits: int) -> np.ndarray:
    """Encode integer codes ``[..., cols]`` into uint32 words, low bits
    first: code ``k`` goes to word ``k // (32/bits)`` at bit
    ``bits * (k % (32/bits))``."""
    c = np.asarray(codes)
    per = 32 // bits
    if c.shape[-1] % per:
        raise ValueError("cols must fill whole words")
    if int(c.max(initial=0)) >> bits:
        raise ValueError(f"code out of range for {bits} bits")
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // per, per))
    out = np.zeros(c.shape[:-1], dtype=np.uint32)
    for j in range(per):
        out |= c[..., j].astype(np.uint32) << np.uint32(bits * j)
    return out


# --------------------------------------------------------------------------
# weight draws
# --------------------------------------------------------------------------

def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _scales_biases(rng, rows, groups, bits):
    s = rng.uniform(0.005, 0.02, size=(rows, groups)).astype(np.float32)
    s_bits = f32_to_bf16_bits(s)
    s_r = bf16_bits_as_f32(s_bits)
    noise = rng.normal(0.0, 0.001, size=(rows, groups)).astype(np.float32)
    b = (np.float32(-(2 ** (bits - 1))) * s_r + noise).astype(np.float32)
    return s_bits, f32_to_bf16_bits(b)


def draw_matrix(key, rows: int, cols: int, bits: int, group_size: int = GROUP):
    """One quantized matrix ``[rows, cols]`` drawn from stream ``key``:
    uniform random words, bf16 scales and biases."""
    rng = _rng(*key)
    words = rng.integers(0, 2 ** 32, size=(rows, cols * bits // 32), dtype=np.uint32)
    s_bits, b_bits = _scales_biases(rng, rows, cols // group_size, bits)
    return words, s_bits, b_bits


def source_config(cfg: MoEConfig) -> MoEConfig:
    """The config whose layers a requantized config's experts come from: the
    same shapes and seed with the source bit width (the layers of
    ``CONFIGS["c3"]`` for ``CONFIGS["c5"]``, at that config's token count)."""
    if not cfg.requant_from:
        return cfg
    return replace(cfg, expert_bits=cfg.requant_from,
                   shared_bits=cfg.requant_from if cfg.has_shared else 0, requant_from=0)


def draw_weight(cfg: MoEConfig, layer: int, expert: int, tensor: int, rows: int,
                cols: int, bits: int):
    if cfg.requant_from and tensor in (T_GATE, T_UP, T_DOWN, T_SH_GATE, T_SH_UP, T_SH_DOWN):
        raise ValueError(f"{cfg.name}: its experts are requantized from the {cfg.requant_from}-bit "
                         "layer of source_config(cfg); draw that one")
    key = (cfg.seed, layer, expert, tensor)
    return draw_matrix(key, rows, cols, bits, cfg.group_size)


# --------------------------------------------------------------------------
# layers (in host memory)
# --------------------------------------------------------------------------

def _qt(q, s, b, rows, cols, bits, gs, batch):
    return {"q": q, "scales": s, "biases": b, "rows": rows, "cols": cols,
            "bits": bits, "group_size": gs, "batch": batch}


class LazyStack:
    """Per-expert arrays of a stacked tensor, drawn on demand: ``stack[e]``
    regenerates expert ``e`` from its own stream (``part`` 0/1/2 picks words,
    scales or biases).  Used to give the oracle single experts of full-size
    layers without holding the layer in host memory."""

    def __init__(self, cfg, layer, tensor, rows, cols, bits, part):
        self.cfg, self.layer, self.tensor = cfg, layer, tensor
        self.rows, self.cols, self.bits, self.part = rows, cols, bits, part

    def __getitem__(self, e):
        return draw_weight(self.cfg, self.layer, int(e), self.tensor, self.rows,
                           self.cols, self.bits)[self.part]


def _stack_spec(cfg: MoEConfig):
    H, I, E = cfg.hidden, cfg.inter, cfg.experts
    return {"gate": (T_GATE, I, H), "up": (T_UP, I, H), "down": (T_DOWN, H, I)}, E


def lazy_layer(cfg: MoEConfig, layer: int) -> dict:
    """A layer whose expert stacks are drawn per expert on access (oracle use)."""
    specs, E = _stack_spec(cfg)
    out = {}
    for name, (tid, rows, cols) in specs.items():
        out[name] = _qt(*(LazyStack(cfg, layer, tid, rows, cols, cfg.expert_bits, p)
                          for p in range(3)), rows, cols, cfg.expert_bits,
                        cfg.group_size, E)
    out.update(_small_tensors(cfg, layer))
    return out


def _small_tensors(cfg: MoEConfig, layer: int) -> dict:
    H = cfg.hidden
    out = {}
    q, s, b = draw_weight(cfg, layer, 0, T_ROUTER, cfg.experts, H, cfg.router_bits)
    out["router"] = _qt(q, s, b, cfg.experts, H, cfg.router_bits, cfg.group_size, 1)
    if cfg.has_shared:
        Is, sb = cfg.shared_inter, cfg.shared_bits
        sh = {}
        for name, tid, rows, cols in (("gate", T_SH_GATE, Is, H), ("up", T_SH_UP, Is, H),
                                      ("down", T_SH_DOWN, H, Is)):
            q, s, b = draw_weight(cfg, layer, 0, tid, rows, cols, sb)
            sh[name] = _qt(q, s, b, rows, cols, sb, cfg.group_size, 1)
        q, s, b = draw_weight(cfg, layer, 0, T_SH_EG, 1, H, cfg.shared_gate_bits)
        sh["expert_gate"] = _qt(q, s, b, 1, H, cfg.shared_gate_bits, cfg.group_size, 1)
        out["shared"] = sh
    else:
        out["shared"] = None
    return out


def host_layer(cfg: MoEConfig, layer: int, threads: int = 8) -> dict:
    """A whole layer in host memory as stacked numpy arrays ``[E, rows, ...]``
    (expert ``e`` of the stack equals the lazy draw of expert ``e``)."""
    specs, E = _stack_spec(cfg)
    out = {}
    bits, gs = cfg.expert_bits, cfg.group_size
    jobs = []
    for name, (tid, rows, cols) in specs.items():
        q = np.empty((E, rows, cols * bits // 32), np.uint32)
        s = np.empty((E, rows, cols // gs), np.uint16)
        b = np.empty((E, rows, cols // gs), np.uint16)
        out[name] = _qt(q, s, b, rows, cols, bits, gs, E)
        jobs += [(name, tid, rows, cols, e) for e in range(E)]

    def fill(job):
        name, tid, rows, cols, e = job
        qq, ss, bb = draw_weight(cfg, layer, e, tid, rows, cols, bits)
        t = out[name]
        t["q"][e], t["scales"][e], t["biases"][e] = qq, ss, bb

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, jobs))
    else:
        for j in jobs:
            fill(j)
    out.update(_small_tensors(cfg, layer))
    return out


# --------------------------------------------------------------------------
# mxfp4 experts
# --------------------------------------------------------------------------

def draw_mxfp4(key, batch: int, rows: int, cols: int, e_lo: int = 118, e_hi: int = 124) -> dict:
    """An mxfp4 tensor (stack) in host memory: uniform random words (every
    4-bit E2M1 field uniform) and E8M0 scale bytes uniform on [e_lo, e_hi]
    (2^-9 .. 2^-3 by default: weights up to 0.75 in magnitude), no biases."""
    rng = _rng(*key)
    q = rng.integers(0, 2 ** 32, size=(batch, rows, cols // 8), dtype=np.uint32)
    sc = rng.integers(e_lo, e_hi + 1, size=(batch, rows, cols // 32)).astype(np.uint8)
    return {"q": q, "scales": sc, "biases": None, "batch": batch, "rows": rows, "cols": cols,
            "bits": 4, "group_size": 32, "mode": "mxfp4"}


def mxfp4_experts(cfg: MoEConfig, layer: int) -> dict:
    """The expert stacks of a layer of ``cfg``'s shapes in mxfp4 (gate, up
    ``[E][I][H]``, down ``[E][H][I]``); no router and no shared expert (the
    prefill path takes routing logits)."""
    E, H, I = cfg.experts, cfg.hidden, cfg.inter
    return {"gate": draw_mxfp4((cfg.seed, layer, 0x4D58, T_GATE), E, I, H),
            "up": draw_mxfp4((cfg.seed, layer, 0x4D58, T_UP), E, I, H),
            "down": draw_mxfp4((cfg.seed, layer, 0x4D58, T_DOWN), E, H, I),
            "router": None, "shared": None}


# --------------------------------------------------------------------------
# sources for the 2-bit requantization
# --------------------------------------------------------------------------

def requant_source(key, batch: int, rows: int, cols: int, bits: int, group_size: int,
                   narrow: float = 0.25, negative: float = 0.3, zero: float = 0.03) -> dict:
    """A 4- or 8-bit tensor (stack) to requantize, in host memory: uniform
    codes, except that a ``narrow`` fraction of the groups draws its codes
    from three or four neighbouring values (small spans, so grid ties occur
    at 4 bits too); bf16 scales U(0.005, 0.02) with a ``negative`` fraction
    negated and a ``zero`` fraction set to zero; bf16 biases N(0, 0.1)."""
    rng = _rng(*key)
    n, ng = batch * rows, cols // group_size
    codes = rng.integers(0, 1 << bits, (n, ng, group_size))
    pick = rng.random((n, ng)) < narrow
    lo = rng.integers(0, (1 << bits) - 4, (n, ng))
    width = rng.integers(3, 5, (n, ng))
    near = lo[..., None] + rng.integers(0, 8, (n, ng, group_size)) % width[..., None]
    codes = np.where(pick[..., None], near, codes).reshape(n, cols)
    s = rng.uniform(0.005, 0.02, (n, ng)).astype(np.float32)
    s = np.where(rng.random((n, ng)) < negative, -s, s)
    s = np.where(rng.random((n, ng)) < zero, np.float32(0.0), s).astype(np.float32)
    b = rng.normal(0.0, 0.1, (n, ng)).astype(np.float32)
    return {"q": pack_codes(codes, bits).reshape(batch, rows, -1),
            "scales": f32_to_bf16_bits(s).reshape(batch, rows, ng),
            "biases": f32_to_bf16_bits(b).reshape(batch, rows, ng),
            "batch": batch, "rows": rows, "cols": cols, "bits": bits, "group_size": group_size}


def requant_source_device(seed: int, batch: int, rows: int, cols: int, bits: int,
                          group_size: int, device):
    """The same recipe without narrow groups, drawn on the device with torch's
    generator (for sizes that host generation would make slow): returns int32
    words and int16 bf16 bit patterns."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    n, ng = batch * rows, cols // group_size
    q = torch.randint(-(2 ** 31), 2 ** 31, (batch, rows, cols * bits // 32), dtype=torch.int64,
                      device=device, generator=g).to(torch.int32)
    s = torch.empty((n, ng), device=device).uniform_(0.005, 0.02, generator=g)
    sign = torch.where(torch.rand((n, ng), device=device, generator=g) < 0.3, -1.0, 1.0)
    s = s * sign
    b = torch.empty((n, ng), device=device).normal_(0.0, 0.1, generator=g)
    to16 = lambda t: t.to(torch.bfloat16).view(torch.int16).reshape(batch, rows, ng).contiguous()
    return q, to16(s), to16(b)


# --------------------------------------------------------------------------
# activations and router logits
# --------------------------------------------------------------------------

def norm_weight(cfg: MoEConfig, layer: int) -> np.ndarray:
    """The RMSNorm weight in front of a layer's MoE step: fp32 U(0.5, 1.5)."""
    rng = _rng(cfg.seed, layer, 0x4E4F524D)
    return rng.uniform(0.5, 1.5, cfg.hidden).astype(np.float32)


def decode_x(cfg: MoEConfig, layer: int, token: int, sub: int = 0, m: int = 1) -> np.ndarray:
    """fp32 ``N(0,1)`` activations ``[m, hidden]`` for (layer, token slot);
    ``sub`` selects a redraw."""
    rng = _rng(cfg.seed, layer, token, T_X, sub)
    return rng.standard_normal((m, cfg.hidden), dtype=np.float32)


def prefill_x_bf16(cfg: MoEConfig, m: int, layer: int = 0) -> np.ndarray:
    """bf16 bit patterns of ``N(0,1)`` activations ``[m, hidden]``."""
    rng = _rng(cfg.seed, layer, 0, T_XB)
    return f32_to_bf16_bits(rng.standard_normal((m, cfg.hidden), dtype=np.float32))


def zipf_logits(cfg: MoEConfig, m: int, layer: int = 0, alpha: float = 1.1) -> np.ndarray:
    """fp32 router logits ``[m, E]`` whose top-K loads are Zipf-skewed:
    expert ``perm[r]`` has rank ``r+1`` with probability ``~ (r+1)**-alpha``
    and its logit is ``log p + Gumbel(0, 1)``, so top-K of a row is a draw of
    K experts without replacement weighted by ``p``."""
    E = cfg.experts
    perm = _rng(cfg.seed, layer, 0, T_PERM).permutation(E)
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-alpha)
    p /= p.sum()
    logp = np.empty(E, np.float64)
    logp[perm] = np.log(p)
    g = _rng(cfg.seed, layer, 0, T_LOGIT).gumbel(size=(m, E))
    return (logp[None, :] + g).astype(np.float32)


def bytes_of(t: dict) -> int:
    return int(t["q"].nbytes + t["scales"].nbytes + t["biases"].nbytes)


def expected_touched(E: int, K: int, M: int) -> float:
    """Expected number of distinct experts touched by M tokens drawing K of E
    uniformly (a workload statistic for batched decode)."""
    return E * (1.0 - (1.0 - K / E) ** M)


def log2i(v: int) -> int:
    return int(math.log2(v))
