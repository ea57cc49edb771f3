"""Per-phase device timeline of the one-launch decode layer (moe_forward).

Runs the instrumented build (``python -m quantized_moe_expert_unpack_amd.build
--timeline`` makes lib/timeline/libmoeq.so, where every work unit of the
decode kernel records the 100 MHz device clock at each step of its protocol)
on a decode workload's layers, and prints a Markdown table: for each kind of
unit and each step, the time since the launch's first unit started
(minimum, median, 90th percentile and maximum over the units, averaged over
the recorded launches).

    python -m quantized_moe_expert_unpack_amd.timeline --config c2 --layers 16 --launches 8

Layers are visited round robin, so each recorded launch reads weights that the
previous launches did not bring into the caches (as in the benchmark's
48-layer sweep).
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from quantized_moe_expert_unpack_amd import build as _build  # noqa: E402

EVENTS = {
    "R": ["start", "fp64 dots done", "logits published", "-", "-", "router rows and x in"],
    "G": ["start", "x staged", "expert known (own top-K of the logits)", "weights in, partial dots done",
          "h written", "every logit seen (wave 0)", "#logit polling rounds", "logits in LDS (block barrier)"],
    "D": ["start", "experts and weights known (pairs from the gate/up units)", "every h segment in LDS",
          "h staged (after the unit's barrier)", "y written", "#h segments re-read from memory",
          "#polling rounds"],
}
KT_BLOCKS, KT_EVENTS = 4096, 12


def d_rows(cfg, m, routed=True):
    """Output rows per D unit, as the library chooses them: 16 for 2- and
    4-bit layers whose units at 8 rows would outnumber two resident units per
    CU (256 CUs), when the unit's scale/bias words fit one 16-byte word per
    thread and a D row spans at most 4 chunks per lane; 8 otherwise."""
    bits, gs = cfg.expert_bits, cfg.group_size
    if bits == 8 or cfg.hidden % 16:
        return 8
    groups = cfg.top_k * (cfg.inter // gs) + (cfg.shared_inter // gs if cfg.has_shared else 0)
    if 2 * 16 * groups * 2 // 16 > 512:
        return 8
    cpc = 128 // bits
    if cfg.top_k * (cfg.inter // cpc) + (cfg.shared_inter // cpc if cfg.has_shared else 0) > 4 * 64:
        return 8
    ng = (cfg.inter + 15) // 16
    ngs = (cfg.shared_inter + 15) // 16 if cfg.has_shared else 0
    units8 = ((cfg.experts + 3) // 4 if routed else 0) + m * (cfg.top_k * ng + ngs) + m * (cfg.hidden // 8)
    return 16 if units8 > 2 * 256 else 8


def plan(cfg, m=1):
    """Unit counts of the one-launch kernel (4 router rows per R unit, 16
    gate/up rows per G unit, d_rows() output rows per D unit) and the kind of
    every block: up to 32 R units (an even count) take the first blocks of
    XCDs 0 and 1 (block b runs on XCD b % 8), more are the first blocks in
    order; then G units, then D units, in block order."""
    r_units = (cfg.experts + 3) // 4
    ng = (cfg.inter + 15) // 16
    ngs = (cfg.shared_inter + 15) // 16 if cfg.has_shared else 0
    g_units = m * (cfg.top_k * ng + ngs)
    dr = d_rows(cfg, m)
    d_units = m * ((cfg.hidden + dr - 1) // dr)
    r2 = (r_units + 1) & ~1
    half = 0
    if r2 <= 32 and 8 * (r2 // 2 - 1) + 1 < r2 + g_units + d_units:
        r_units, half = r2, r2 // 2
    kinds = []
    for b in range(r_units + g_units + d_units):
        q, x = b >> 3, b & 7
        if half and x < 2 and q < half:
            kinds.append("R")
            continue
        o = b - (2 * min(q, half) + (min(x, 2) if q < half else 0)) if half else b - r_units
        if not half and b < r_units:
            kinds.append("R")
        else:
            kinds.append("G" if o < g_units else "D")
    return r_units, g_units, d_units, kinds


def read_ceiling(lib, sizes_mb, reps=8):
    """Device time of one cold read of each size (a fresh window of a large
    buffer every time, so neither L2 nor the MALL holds it), by k_read_probe
    at several grid sizes: a Markdown table of GB/s."""
    import torch
    dev = torch.device("cuda:0")
    lib.moeq_read_probe.restype = ctypes.c_int
    lib.moeq_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    pool = torch.ones((8 << 30) // 4, dtype=torch.float32, device=dev)     # 8 GiB of windows
    out = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    print("| bytes read | blocks of 256 | us (median of %d) | GB/s |" % reps)
    print("|---|---|---|---|")
    base = 0
    for mb in sizes_mb:
        n = mb << 20
        for blocks in (1024, 2048, 4096):
            ts = []
            for _ in range(reps):
                if base + n > pool.numel() * 4:
                    base = 0
                ptr = pool.data_ptr() + base
                base += n + (1 << 20)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                a.record(s)
                assert lib.moeq_read_probe(ptr, n, blocks, out.data_ptr(), s.cuda_stream) == 0
                b.record(s)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3)
            us = float(np.median(ts))
            print(f"| {n:,} | {blocks} | {us:.2f} | {n / us / 1e3:.0f} |")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3"])
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure cold one-shot reads of 10 MB to 420 MB (k_read_probe)")
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--launches", type=int, default=8)
    ap.add_argument("--build", action="store_true", help="build the instrumented library first")
    ap.add_argument("--pipelined", action="store_true",
                    help="record the last of each run of back-to-back launches over all layers "
                         "(as the benchmark's graph replays them) instead of a launch on an idle GPU")
    args = ap.parse_args()
    if args.build or not os.path.exists(_build.TIMELINE_LIB):
        _build.build(timeline=True)

    import torch
    from quantized_moe_expert_unpack_amd import moeq, synth
    moeq.use_library(_build.TIMELINE_LIB)
    lib = moeq.lib()
    lib.moeq_timeline_copy.restype = ctypes.c_int
    lib.moeq_timeline_copy.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.moeq_timeline_clear.restype = ctypes.c_int
    if args.read_ceiling:
        print("# Cold one-shot read ceiling (k_read_probe, 16-byte loads, four in flight per thread)\n")
        read_ceiling(lib, [10, 20, 40, 80, 420])
        return

    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    n_layers = min(args.layers, cfg.layers)
    layers = [moeq.MoELayer.from_host(synth.host_layer(cfg, l, threads=16), dev) for l in range(n_layers)]
    xs = [torch.from_numpy(synth.decode_x(cfg, l, 0)).to(dev) for l in range(n_layers)]
    ws = moeq.workspace(layers[0], 1, cfg.top_k, moeq.PATH_FORWARD, dev)
    y = torch.empty((1, cfg.hidden), dtype=torch.float32, device=dev)
    idx = torch.empty((1, cfg.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((1, cfg.top_k), dtype=torch.float32, device=dev)
    r_units, g_units, d_units, kinds = plan(cfg)
    n_units = r_units + g_units + d_units
    buf = np.zeros(KT_BLOCKS * KT_EVENTS, np.uint64)
    per = {k: [] for k in EVENTS}
    totals, xcd_start, rr_ok = [], [], []
    for rep in range(n_layers + args.launches):
        l = rep % n_layers
        record = rep >= n_layers
        if record:
            torch.cuda.synchronize()
            assert lib.moeq_timeline_clear() == 0
        if args.pipelined and record:
            # a run of back-to-back launches; the timestamps are the last one's
            for j in range(n_layers):
                ll = (l + 1 + j) % n_layers
                moeq.moe_forward(layers[ll], xs[ll], cfg.top_k, cfg.renorm, ws=ws, y=y, idx=idx, w=w)
        else:
            moeq.moe_forward(layers[l], xs[l], cfg.top_k, cfg.renorm, ws=ws, y=y, idx=idx, w=w)
        if not record:
            continue
        torch.cuda.synchronize()
        assert lib.moeq_timeline_copy(buf.ctypes.data, buf.size) == 0
        t = buf.reshape(KT_BLOCKS, KT_EVENTS)[:n_units].astype(np.int64)
        t0 = t[:, 0].min()
        rel = (t - t0) / 100.0                      # 100 MHz ticks -> microseconds
        rel[t == 0] = np.nan                        # a step the unit does not take (a shared-expert unit's poll)
        timed = np.zeros(rel.shape, bool)
        for kind, names in EVENTS.items():          # counters are counts, not times
            sel = [i for i, k in enumerate(kinds) if k == kind]
            for e, name in enumerate(names):
                if name.startswith("#"):               # summed over the run's launches
                    rel[sel, e] = t[sel, e] / (n_layers if args.pipelined else 1)
                elif name != "-":
                    timed[sel, e] = True
        totals.append(np.nanmax(rel[timed]))
        for kind in EVENTS:
            sel = [i for i, k in enumerate(kinds) if k == kind]
            per[kind].append(rel[sel][:, :len(EVENTS[kind])])
        xcd = buf.reshape(KT_BLOCKS, KT_EVENTS)[:n_units, KT_EVENTS - 1].astype(np.int64)
        xcd_start.append([rel[xcd == j, 0].min() if (xcd == j).any() else np.nan for j in range(8)])
        rr_ok.append(bool(np.array_equal(xcd, np.arange(n_units) % 8)))
    st, bits = moeq.workspace_status(ws)
    if st != 0:
        raise SystemExit(f"a bounded wait gave up during the timeline run (0x{bits:x})")

    print(f"# Device timeline of the one-launch decode layer: {cfg.name}"
          f"{' (back-to-back launches)' if args.pipelined else ''}\n")
    print(f"Units per launch: {r_units} R (router rows), "
          f"{g_units} G (gate/up rows of one expert), {d_units} D (output rows of the token).  "
          f"Times in us since the launch's first unit started, over {args.launches} launches "
          f"({n_layers} layers visited round robin); the launch's last mark averages "
          f"{np.mean(totals):.2f} us.\n")
    xs_ = np.nanmean(np.array(xcd_start), axis=0)
    print("First unit to start on each XCD (us; hardware XCC_ID of each block): " +
          ", ".join(f"XCD {j}: {v:.2f}" for j, v in enumerate(xs_)) +
          f".  Block b ran on XCD b % 8 in {sum(rr_ok)} of {len(rr_ok)} launches.\n")
    print("| unit | step | min | median | p90 | max |")
    print("|---|---|---|---|---|---|")
    for kind, names in EVENTS.items():
        a = np.stack(per[kind])                    # [launch][unit][event]
        for e, name in enumerate(names):
            if name == "-":
                continue
            v = a[:, :, e]
            if name.startswith("#"):
                v = np.nan_to_num(v)
            q = [np.mean(np.nanmin(v, axis=1)), np.mean(np.nanmedian(v, axis=1)),
                 np.mean(np.nanpercentile(v, 90, axis=1)), np.mean(np.nanmax(v, axis=1))]
            print(f"| {kind} | {name} | " + " | ".join(f"{x:.2f}" for x in q) + " |")


if __name__ == "__main__":
    main()
