#!/usr/bin/env python3
"""Throughput of the quantized MoE step on one MI355X.

Default workload (``--config c2``): 30B-A3B-shaped decode at batch 1 -- hidden
2048, 128 experts, top-8, expert intermediate 768, router and experts 8-bit
affine group 64 -- through 48 independent resident layers.  One step is one
token through all 48 layers: per layer the router projection with softmax and
top-K (moe_route) and the expert forward (moe_expert_forward), strictly one
layer after the other on one stream.  The 48-layer sweep of each of 64 token
slots is captured once in a HIP graph and replayed; the token slots rotate
so the routed experts change from step to step.  All weights and activations
are resident in HBM before the timed region.

Other workloads: ``c3`` (397B-A17B-shaped decode, 4-bit experts + shared
expert, 8 layers), ``c5`` / ``c5_4bit`` (the same shapes at 2 / 4 bits, 64
tokens per step), ``c4`` (prefill gather_qmm, M=16384 tokens, one layer),
``c4_mxfp4`` (the same prefill with mxfp4 experts), ``requant`` (the 2-bit requantization of one 397B-A17B-shaped layer's three
4-bit expert stacks, gate and up [512][1024][4096], down [512][4096][1024]).

Prints one JSON line.  ``roofline`` rates the dominant launch against the HBM
(decode) or bf16 MFMA (prefill) peak, timed live with HIP events on the stream
it runs on; ``cpu_baseline`` times the CPU oracle on a bounded sample of the
same workload on this host.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill) vs peak"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
TOKEN_SLOTS = 64
BATCH_MIN_M = 16     # moe_expert_forward groups pairs by expert from this many tokens
NORM_EPS = 1e-6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(cfg, touched: float) -> float:
    """Algorithmic bytes of one layer: the router, every distinct touched
    expert (codes + bf16 scale/bias) and the shared expert."""
    def mat(rows, cols, bits):
        return rows * cols * bits // 8 + rows * (cols // cfg.group_size) * 4
    router = mat(cfg.experts, cfg.hidden, cfg.router_bits)
    expert = 2 * mat(cfg.inter, cfg.hidden, cfg.expert_bits) + mat(cfg.hidden, cfg.inter, cfg.expert_bits)
    shared = 0
    if cfg.has_shared:
        shared = (2 * mat(cfg.shared_inter, cfg.hidden, cfg.shared_bits)
                  + mat(cfg.hidden, cfg.shared_inter, cfg.shared_bits)
                  + mat(1, cfg.hidden, cfg.shared_gate_bits))
    acts = 2 * cfg.tokens * cfg.hidden * 4          # x in, y out (fp32)
    return router + touched * expert + shared + acts


def expert_launch_bytes(cfg, touched: float) -> float:
    """Bytes one moe_expert_forward launch must move: touched experts, the
    shared expert, x, y and the routing (the router is not part of it)."""
    def mat(rows, cols, bits):
        return rows * cols * bits // 8 + rows * (cols // cfg.group_size) * 4
    expert = 2 * mat(cfg.inter, cfg.hidden, cfg.expert_bits) + mat(cfg.hidden, cfg.inter, cfg.expert_bits)
    shared = 0
    if cfg.has_shared:
        shared = (2 * mat(cfg.shared_inter, cfg.hidden, cfg.shared_bits)
                  + mat(cfg.hidden, cfg.shared_inter, cfg.shared_bits)
                  + mat(1, cfg.hidden, cfg.shared_gate_bits))
    return touched * expert + shared + 2 * cfg.tokens * cfg.hidden * 4 + cfg.tokens * cfg.top_k * 8


# --------------------------------------------------------------------------
# HBM traffic measured with rocprofv3 counters
# --------------------------------------------------------------------------

KERNEL_SOURCES = {
    "k_moe_decode": ["k_decode.hip", "decode_common.h", "common.h", "topk.h", "launch.h"],
    "k_batch": ["k_batch.hip", "k_sort.hip", "decode_common.h", "common.h", "launch.h"],
    "k_gqmm": ["k_gemm.hip", "common.h", "launch.h"],
    "k_requant2": ["k_requant.hip", "common.h", "launch.h"],
}


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "quantized_moe_expert_unpack_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(args, kernel):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    calibration) from profiles/traffic_<kernel>_<workload>.md, or null when
    those counters were taken on a different version of the kernel's sources."""
    if args.traffic is not None:
        return args.traffic
    if getattr(args, "group_size", 0):
        return None                 # the stored counters are for the workload's own group size
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{args.config}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_hash") != kernel_source_hash(kernel):
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------------------
# CPU oracle baseline
# --------------------------------------------------------------------------

class _Picked:
    """Stack view holding only pre-drawn experts (draw time stays out of the
    timed oracle call)."""

    def __init__(self, arrays):
        self.arrays = arrays

    def __getitem__(self, e):
        return self.arrays[int(e)]


def cpu_baseline_decode(cfg, tokens_per_layer, n_layers):
    import oracle
    from quantized_moe_expert_unpack_amd import synth
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = min(16, len(os.sched_getaffinity(0)))
    lim = threadpool_limits(cores) if threadpool_limits else None
    total = 0.0
    ntok = 0
    try:
        for l in range(n_layers):
            small = synth._small_tensors(cfg, l)
            x = np.concatenate([synth.decode_x(cfg, l, t) for t in range(tokens_per_layer)])
            # pre-draw exactly the experts the oracle will route to (untimed)
            lg = oracle.qmatvec(small["router"], x)
            idx, _, _ = oracle.route(lg, cfg.top_k)
            need = sorted(set(int(e) for e in idx.reshape(-1)))
            layer = dict(small)
            for name, tid, rows, cols in (("gate", synth.T_GATE, cfg.inter, cfg.hidden),
                                          ("up", synth.T_UP, cfg.inter, cfg.hidden),
                                          ("down", synth.T_DOWN, cfg.hidden, cfg.inter)):
                drawn = {e: synth.draw_weight(cfg, l, e, tid, rows, cols, cfg.expert_bits) for e in need}
                layer[name] = {"q": _Picked({e: d[0] for e, d in drawn.items()}),
                               "scales": _Picked({e: d[1] for e, d in drawn.items()}),
                               "biases": _Picked({e: d[2] for e, d in drawn.items()}),
                               "rows": rows, "cols": cols, "bits": cfg.expert_bits,
                               "group_size": cfg.group_size, "batch": cfg.experts}
            t0 = time.perf_counter()
            oracle.moe_layer(layer, x, cfg.top_k, cfg.renorm)
            total += time.perf_counter() - t0
            ntok += tokens_per_layer
    finally:
        if lim is not None:
            lim.restore_original_limits()
    # a token passes through every layer: oracle tokens/s over the full stack
    per_token_layer = total / ntok
    value = 1.0 / (per_token_layer * cfg.layers)
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{tokens_per_layer} token(s) x {n_layers} of {cfg.layers} layers "
                      f"(router + top-K + {cfg.top_k} experts{' + shared' if cfg.has_shared else ''}, "
                      f"fp64 numpy); {total:.1f} s of oracle time, scaled to {cfg.layers} layers/token"}


def cpu_baseline_prefill(cfg, host, m_sample):
    import oracle
    from quantized_moe_expert_unpack_amd import synth
    cores = min(16, len(os.sched_getaffinity(0)))
    try:
        from threadpoolctl import threadpool_limits
        lim = threadpool_limits(cores)
    except ImportError:  # pragma: no cover
        lim = None
    xb = synth.prefill_x_bf16(cfg, m_sample)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    lg = synth.zipf_logits(cfg, m_sample)
    t0 = time.perf_counter()
    idx, w, _ = oracle.route(lg.astype(np.float64), cfg.top_k)
    oracle.moe_experts(host, xf, idx, w)
    dt = time.perf_counter() - t0
    if lim is not None:
        lim.restore_original_limits()
    return {"value": m_sample / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{m_sample} of {cfg.tokens} prefill tokens, one layer (fp64 numpy); {dt:.1f} s"}


# --------------------------------------------------------------------------
# decode workloads
# --------------------------------------------------------------------------

def run_decode(args, cfg):
    import torch
    from quantized_moe_expert_unpack_amd import moeq, synth

    dev = torch.device("cuda:0")
    n_layers = args.layers or cfg.layers
    m, K, H = cfg.tokens, cfg.top_k, cfg.hidden
    t0 = time.time()
    layers = []
    for l in range(n_layers):
        host = synth.host_layer(cfg, l, threads=16)
        layers.append(moeq.MoELayer.from_host(host, dev))
        del host
    log(f"[bench] {n_layers} layers resident ({sum(L.gate.nbytes + L.up.nbytes + L.down.nbytes for L in layers) / 1e9:.1f} GB experts) in {time.time() - t0:.0f}s")
    slots = args.slots
    x = torch.empty((n_layers, slots, m, H), dtype=torch.float32, device=dev)
    for l in range(n_layers):
        for t in range(slots):
            x[l, t] = torch.from_numpy(synth.decode_x(cfg, l, t, m=m))
    idx = torch.zeros((n_layers, m, K), dtype=torch.int32, device=dev)
    w = torch.zeros((n_layers, m, K), dtype=torch.float32, device=dev)
    y = torch.zeros((n_layers, m, H), dtype=torch.float32, device=dev)
    # one launch per layer (router + top-K + experts) when the library can
    # route inside the launch (8-bit router, M <= 4); else route, then experts
    one_launch = cfg.router_bits == 8 and m <= 4
    ws_fwd = moeq.workspace(layers[0], m, K, moeq.PATH_FORWARD_NORM if args.norm else moeq.PATH_FORWARD,
                            dev)
    # --norm: RMSNorm in front of every layer's step, x added back in the combine
    gam = [torch.from_numpy(synth.norm_weight(cfg, l)).to(dev) for l in range(n_layers)] if args.norm else None
    # --post-norm: also the norm after the combine (the next layer's weight)
    gam2 = ([torch.from_numpy(synth.norm_weight(cfg, l + 1)).to(dev) for l in range(n_layers)]
            if args.post_norm else [None] * n_layers)
    yn = torch.zeros((n_layers, m, H), dtype=torch.float32, device=dev) if args.post_norm else None
    ws_route = moeq.workspace(layers[0], m, K, moeq.PATH_ROUTE, dev)
    ws_dec = moeq.workspace(layers[0], m, K, moeq.PATH_DECODE, dev)

    def layer_call(l, t):
        L = layers[l]
        if args.norm:
            moeq.moe_forward_norm(L, x[l, t], K, gam[l], NORM_EPS, cfg.renorm, ws=ws_fwd, y=y[l],
                                  idx=idx[l], w=w[l], post_norm_w=gam2[l],
                                  y_norm=yn[l] if args.post_norm else None)
        elif one_launch:
            moeq.moe_forward(L, x[l, t], K, cfg.renorm, ws=ws_fwd, y=y[l], idx=idx[l], w=w[l])
        else:
            moeq.moe_route(L.router, x[l, t], cfg.experts, K, cfg.renorm, ws=ws_route,
                           idx=idx[l], w=w[l])
            moeq.moe_expert_forward(L, x[l, t], idx[l], w[l], ws=ws_dec, y=y[l])

    def step(t):
        for l in range(n_layers):
            layer_call(l, t)

    # eager warm-up (also checks the path runs), then capture one graph per slot
    for t in range(min(2, slots)):
        step(t)
    torch.cuda.synchronize()
    capture_stream = torch.cuda.Stream()
    graphs = []
    for t in range(slots):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=capture_stream):
            step(t)
        graphs.append(g)
    torch.cuda.synchronize()

    # touched experts per layer (distinct experts over the step's tokens)
    touched = []
    for t in range(slots):
        graphs[t].replay()
        torch.cuda.synchronize()
        ii = idx.cpu().numpy()
        touched.append(np.mean([len(np.unique(ii[l])) for l in range(n_layers)]))
    touched = float(np.mean(touched))

    for s in range(args.warmup):
        graphs[s % slots].replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(args.steps):
        graphs[s % slots].replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms * 1e3:.1f} us/step")

    bytes_step = n_layers * layer_bytes(cfg, touched)
    gbps = bytes_step / (ms * 1e-3) / 1e9

    # dominant launch, timed live with HIP events recorded on the stream it is
    # launched on (eager launches, same buffers): the one-launch layer
    # (moe_forward), or the expert launch (moe_expert_forward) of the
    # two-launch form
    s_ = torch.cuda.current_stream()
    reps = max(1, args.launch_reps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps * n_layers)]
    k = 0
    for r in range(reps):
        t = r % slots
        for l, L in enumerate(layers):
            if args.norm:
                evs[k][0].record(s_)
                moeq.moe_forward_norm(L, x[l, t], K, gam[l], NORM_EPS, cfg.renorm, ws=ws_fwd, y=y[l],
                                      idx=idx[l], w=w[l], post_norm_w=gam2[l],
                                      y_norm=yn[l] if args.post_norm else None)
                evs[k][1].record(s_)
            elif one_launch:
                evs[k][0].record(s_)
                moeq.moe_forward(L, x[l, t], K, cfg.renorm, ws=ws_fwd, y=y[l], idx=idx[l], w=w[l])
                evs[k][1].record(s_)
            else:
                moeq.moe_route(L.router, x[l, t], cfg.experts, K, cfg.renorm, ws=ws_route,
                               idx=idx[l], w=w[l])
                evs[k][0].record(s_)
                moeq.moe_expert_forward(L, x[l, t], idx[l], w[l], ws=ws_dec, y=y[l])
                evs[k][1].record(s_)
            k += 1
    torch.cuda.synchronize()
    eager_us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    # one launch per layer: every node of the timed graphs is the kernel, so
    # its average duration is the timed region over (steps x layers); else
    # the eager, event-bracketed expert launches
    launch_us = ms * 1e3 / n_layers if one_launch else eager_us
    lbytes = (layer_bytes(cfg, touched) + m * K * 8) if one_launch else expert_launch_bytes(cfg, touched)
    if args.norm:
        lbytes += cfg.hidden * 4                      # the norm weight
        if not one_launch:                            # norm + route + experts, bracketed together
            lbytes = layer_bytes(cfg, touched) + m * K * 8 + cfg.hidden * 4 + 2 * m * cfg.hidden * 4
    if args.post_norm:                                # its weight, y read, y_norm written
        lbytes += cfg.hidden * 4 + 2 * m * cfg.hidden * 4
    achieved = lbytes / (launch_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": None if args.norm else traffic_for(
                    args, "k_batch" if not one_launch and m >= BATCH_MIN_M else "k_moe_decode"),
                "kernel": ("k_moe_decode + k_rmsnorm (moe_forward_norm with the norm after the "
                           "combine: two launches per layer)" if args.post_norm and one_launch else
                           "k_moe_decode (moe_forward_norm: RMSNorm + router + top-K + experts)"
                           if args.norm and one_launch else
                           "moe_forward_norm (norm, route, experts)" if args.norm else
                           "k_moe_decode (moe_forward: router + top-K + experts)") if one_launch or args.norm
                          else ("moe_expert_forward batched by expert (sort, k_bgate, k_bdown, "
                                "k_bcombine)" if m >= BATCH_MIN_M else "k_moe_decode (moe_expert_forward)"),
                "launch_us": round(launch_us, 2), "eager_launch_us": round(eager_us, 2),
                "bytes_per_launch": int(lbytes)}

    out = {
        "metric": METRIC, "value": round(m * 1e3 / ms, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "layers": n_layers, "tokens_per_step": m,
                   "hidden": H, "experts": cfg.experts, "top_k": K, "inter": cfg.inter,
                   "expert_bits": cfg.expert_bits, "router_bits": cfg.router_bits,
                   "shared_expert": cfg.has_shared, "group_size": cfg.group_size,
                   "token_slots": slots, "graph": True, "rmsnorm_fused": bool(args.norm),
                   "post_norm": bool(args.post_norm),
                   "launches_per_layer": (1 if one_launch else 2) + int(args.post_norm)},
        "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_step": int(bytes_step), "touched_experts_per_layer": round(touched, 2),
        "roofline": roofline,
    }
    return out


# --------------------------------------------------------------------------
# prefill workload
# --------------------------------------------------------------------------

def run_prefill(args, cfg):
    import torch
    from quantized_moe_expert_unpack_amd import moeq, synth

    dev = torch.device("cuda:0")
    m = args.tokens or cfg.tokens
    host = (synth.mxfp4_experts(cfg, 0) if cfg.expert_mode == "mxfp4"
            else synth.host_layer(cfg, 0, threads=16))
    L = moeq.MoELayer.from_host(host, dev)
    xb = torch.from_numpy(synth.prefill_x_bf16(cfg, m).view(np.int16)).to(dev)
    lg = torch.from_numpy(synth.zipf_logits(cfg, m)).to(dev)
    K = cfg.top_k
    idx = torch.empty((m, K), dtype=torch.int32, device=dev)
    w = torch.empty((m, K), dtype=torch.float32, device=dev)
    y = torch.empty((m, cfg.hidden), dtype=torch.float32, device=dev)
    ws = moeq.workspace(L, m, K, moeq.PATH_GATHER, dev)

    def step():
        moeq.moe_route(None, lg, cfg.experts, K, cfg.renorm, idx=idx, w=w)
        moeq.moe_gather_qmm(L, xb, idx, w, ws=ws, y=y)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    flops = 2.0 * m * K * 3 * cfg.inter * cfg.hidden
    tflops = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(m * 1e3 / ms, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": m, "hidden": cfg.hidden,
                   "experts": cfg.experts, "top_k": K, "inter": cfg.inter,
                   "expert_bits": cfg.expert_bits, "expert_mode": cfg.expert_mode,
                   "group_size": cfg.group_size, "logits": "zipf(1.1)+gumbel"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_for(args, "k_gqmm"), "kernel": "moe_route + moe_gather_qmm",
                     "flops_per_launch": flops},
    }
    out["_host"] = host
    return out


# --------------------------------------------------------------------------
# host-resident experts streamed into HBM slots
# --------------------------------------------------------------------------

PCIE_PEAK_GBPS = 64.0     # PCIe 5.0 x16, one direction


def run_stream(args, cfg):
    """Decode with the experts in pinned host memory only: per layer, route on
    the device, bring the selected experts into the layer's HBM slots
    (moe_stream_experts: LRU, async copies on the stream), run the expert
    forward on the slots.  The router and the shared expert stay resident."""
    import torch
    from quantized_moe_expert_unpack_amd import moeq, synth

    dev = torch.device("cuda:0")
    n_layers = args.layers or cfg.layers
    K = cfg.top_k
    caches, routers = [], []
    t0 = time.time()
    for l in range(n_layers):
        host = synth.host_layer(cfg, l, threads=16)
        sh = None
        if host.get("shared") is not None:
            sh = {k: moeq.QTensor.from_host(v, dev) for k, v in host["shared"].items()}
        resident = moeq.MoELayer(moeq.QTensor.from_host(host["router"], dev), None, None, None, sh)
        caches.append(moeq.ExpertCache(host, args.stream_slots, resident, dev,
                                       device_lru=args.stream_device))
        routers.append(resident.router)
        del host
    log(f"[bench] {n_layers} layers in pinned host memory, {args.stream_slots} HBM slots each "
        f"({time.time() - t0:.0f}s)")
    slots_n = args.slots
    x = torch.stack([torch.stack([torch.from_numpy(synth.decode_x(cfg, l, t)[0]) for t in range(slots_n)])
                     for l in range(n_layers)]).to(dev)
    y = torch.empty((1, cfg.hidden), dtype=torch.float32, device=dev)
    ws_dec = moeq.workspace(caches[0].layer, 1, K, moeq.PATH_DECODE, dev)
    ws_route = moeq.workspace(caches[0].layer, 1, K, moeq.PATH_ROUTE, dev)
    copied = [0]
    n_warm = max(1, args.warmup)
    # device form: one copy counter per (step, layer), summed after the run
    ncp = (torch.zeros((n_warm + args.steps, n_layers, 4), dtype=torch.int32, device=dev)
           if args.stream_device else None)
    idx_b = torch.empty((1, K), dtype=torch.int32, device=dev)
    w_b = torch.empty((1, K), dtype=torch.float32, device=dev)
    sidx_b = torch.empty((1, K), dtype=torch.int32, device=dev)

    def step(t):
        for l in range(n_layers):
            xt = x[l, t % slots_n][None, :]
            moeq.moe_route(routers[l], xt, cfg.experts, K, cfg.renorm, ws=ws_route, idx=idx_b, w=w_b)
            if args.stream_device:
                caches[l].stream_device(idx_b, slot_idx=sidx_b, n_copied=ncp[t, l])
                moeq.moe_expert_forward(caches[l].layer, xt, sidx_b, w_b, ws=ws_dec, y=y)
            else:
                slot_idx, n = caches[l].stream(idx_b.cpu().numpy())
                copied[0] += n
                moeq.moe_expert_forward(caches[l].layer, xt, torch.from_numpy(slot_idx).to(dev), w_b,
                                        ws=ws_dec, y=y)

    for s_ in range(n_warm):
        step(s_)
    torch.cuda.synchronize()
    copied[0] = 0
    t1 = time.perf_counter()
    for s_ in range(args.steps):
        step(n_warm + s_)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t1
    if args.stream_device:
        copied[0] = int(ncp[n_warm:, :, 0].sum().item())
    ms = dt * 1e3 / args.steps
    per_expert = 3 * cfg.hidden * cfg.inter * cfg.expert_bits // 8 + 3 * cfg.hidden * cfg.inter // cfg.group_size * 4
    gbps = copied[0] * per_expert / dt / 1e9
    log(f"[bench] stream: {ms:.3f} ms/token, {copied[0] / (args.steps * n_layers):.2f} experts copied per layer")
    return {
        "metric": "MoE-layer tokens/s with experts streamed from host memory (PCIe GB/s vs peak)",
        "value": round(1e3 / ms, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name + "-streamed", "layers": n_layers, "tokens_per_step": 1,
                   "hidden": cfg.hidden, "experts": cfg.experts, "top_k": K, "inter": cfg.inter,
                   "expert_bits": cfg.expert_bits, "hbm_slots_per_layer": args.stream_slots,
                   "expert_bytes": per_expert,
                   "slot_choice": "device" if args.stream_device else "host"},
        "experts_copied_per_layer": round(copied[0] / (args.steps * n_layers), 3),
        "roofline": {"bound": "pcie", "achieved": round(gbps, 2), "peak": PCIE_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PCIE_PEAK_GBPS, 4), "traffic": None,
                     "kernel": ("moe_stream_experts_device: k_slot_lru + k_slot_copy reading pinned host "
                                "memory (route, slot choice, copy, expert forward per layer, no host sync)"
                                if args.stream_device else
                                "moe_stream_experts host->device copies (route, copy, expert forward per layer)")},
    }


# --------------------------------------------------------------------------
# 2-bit requantization workload
# --------------------------------------------------------------------------

REQUANT_METRIC = "2-bit requantization throughput (algorithmic bytes read + written per s)"


def requant_bytes(E, rows, cols, bits, gs):
    """Algorithmic bytes of one requantization: the source codes and bf16
    scale/bias, the 2-bit codes and their bf16 scale/bias."""
    n = E * rows * cols
    return n * bits // 8 + n // gs * 4 + n // 4 + n // gs * 4


def cpu_baseline_requant(rows, cols, bits, gs):
    import oracle
    from quantized_moe_expert_unpack_amd import synth
    host = synth.requant_source((7, rows), 1, rows, cols, bits, gs, narrow=0.0)
    t0 = time.perf_counter()
    oracle.requant_2bit(host)
    dt = time.perf_counter() - t0
    return {"value": round(requant_bytes(1, rows, cols, bits, gs) / dt / 1e9, 6), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{rows} rows x {cols} columns of a {bits}-bit expert matrix (exact rational "
                      f"arithmetic, pure Python); {dt:.1f} s"}


def run_requant(args):
    import torch
    from quantized_moe_expert_unpack_amd import moeq, synth

    dev = torch.device("cuda:0")
    E, I, H, bits, gs = 512, 1024, 4096, 4, 64
    shapes = [(I, H), (I, H), (H, I)]                 # gate, up, down
    srcs = []
    for i, (r, c) in enumerate(shapes):
        q, sc, bi = synth.requant_source_device(100 + i, E, r, c, bits, gs, dev)
        srcs.append(moeq.QTensor(q, sc, bi, E, r, c, bits, gs))
    outs = [moeq.requant_2bit(W) for W in srcs]      # allocates the outputs once
    torch.cuda.synchronize()
    lib, s_ = moeq.lib(), torch.cuda.current_stream()
    import ctypes
    args_ = [(ctypes.byref(W.struct()), o.q.data_ptr(), o.scales.data_ptr(), o.biases.data_ptr())
             for W, o in zip(srcs, outs)]

    def launch(i):
        a = args_[i]
        st = lib.requant_2bit(a[0], a[1], a[2], a[3], s_.cuda_stream)
        if st:
            raise RuntimeError(f"requant_2bit failed: {st}")

    for _ in range(max(1, args.warmup)):
        for i in range(3):
            launch(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(3 * args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(s_)
    for k in range(args.steps):
        for i in range(3):
            evs[3 * k + i][0].record(s_)
            launch(i)
            evs[3 * k + i][1].record(s_)
    end.record(s_)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    launch_us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    per_launch = requant_bytes(E, I, H, bits, gs)     # the three stacks hold equal counts
    step_bytes = 3 * per_launch
    achieved = per_launch / (launch_us * 1e-6) / 1e9
    log(f"[bench] requant: {ms * 1e3:.1f} us/step, {launch_us:.1f} us/launch")
    return {
        "metric": REQUANT_METRIC, "value": round(step_bytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": "requant-397b-a17b-layer-4to2bit", "experts": E, "hidden": H,
                   "inter": I, "source_bits": bits, "group_size": gs,
                   "matrices": "gate, up [E][I][H]; down [E][H][I]"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_for(args, "k_requant2"), "kernel": "k_requant2<4>",
                     "launch_us": round(launch_us, 2), "bytes_per_launch": int(per_launch)},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2", choices=["c2", "c3", "c4", "c4_mxfp4", "c5", "c5_4bit", "requant"])
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (decode)")
    ap.add_argument("--group-size", type=int, default=0, choices=[0, 32, 64, 128],
                    help="override the quantization group size of every matrix")
    ap.add_argument("--tokens", type=int, default=0, help="override M (prefill)")
    ap.add_argument("--slots", type=int, default=TOKEN_SLOTS)
    ap.add_argument("--launch-reps", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stream-slots", type=int, default=0, metavar="S",
                    help="decode with the experts in pinned host memory, S HBM slots per layer")
    ap.add_argument("--stream-device", action="store_true",
                    help="with --stream-slots: slot choice and copies on the device (no host sync)")
    ap.add_argument("--norm", action="store_true",
                    help="decode: RMSNorm fused in front of the step (moe_forward_norm), x added back")
    ap.add_argument("--post-norm", action="store_true",
                    help="decode: --norm plus the norm after the combine (the next layer's input)")
    ap.add_argument("--cpu-layers", type=int, default=0)
    ap.add_argument("--traffic", type=float, default=None,
                    help="HBM bytes per launch from rocprofv3 counters, if taken")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device copies of MIB MiB (the reference kernel that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes) and exit")
    args = ap.parse_args()
    if args.post_norm:
        args.norm = True

    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "copies": 5}), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    from quantized_moe_expert_unpack_amd import synth
    if args.config == "requant":
        out = run_requant(args)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_requant(384, 4096, 4, 64)
        print(json.dumps(out), flush=True)
        return
    cfg = synth.CONFIGS[args.config]
    if args.group_size:
        if args.config == "c4_mxfp4":
            raise SystemExit("--group-size: mxfp4 groups are 32 columns by definition")
        cfg = synth.scaled(cfg, group_size=args.group_size, name=f"{cfg.name}-gs{args.group_size}")
    if args.config in ("c4", "c4_mxfp4"):
        out = run_prefill(args, cfg)
        host = out.pop("_host")
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_prefill(cfg, host, 1024)
    elif args.stream_slots:
        out = run_stream(args, cfg)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_decode(cfg, 2, args.cpu_layers or min(8, cfg.layers))
    else:
        out = run_decode(args, cfg)
        if not args.no_cpu_baseline:
            # bounded samples of ~10-30 s of oracle time: two tokens of the
            # 48-layer stack, two tokens of the 8-layer stack, one 64-token layer
            n, tok = {"c2": (48, 2), "c3": (8, 2), "c5": (1, 64), "c5_4bit": (1, 64)}[args.config]
            out["cpu_baseline"] = cpu_baseline_decode(cfg, tok, args.cpu_layers or n)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
