"""GPU parity: the bf16-MFMA gather path (moe_gather_qmm, gather_qmm).

Acceptance: max per-row relative L2 <= 2e-2 against the fp64 oracle; one-shot
equals 2048-token chunks; no row left unwritten under two poison patterns;
reruns bitwise identical; zero bad rows at the row counts of the pages'
seam list.
"""

import functools

import numpy as np
import pytest
import torch

import oracle
from quantized_moe_expert_unpack_amd import moeq, synth
from tests.gpu_util import bf16_bits_to_f32, bf16_dev, dev, rel_l2_rows, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-2
POISON = (float("nan"), 3.0e38)


@functools.lru_cache(maxsize=1)
def _c4_layer():
    cfg = synth.CONFIGS["c4"]
    host = synth.host_layer(cfg, 0, threads=16)
    return cfg, host, moeq.MoELayer.from_host(host, dev())


def _prefill(cfg, L, xb, lg, chunk=None, poison=None):
    m = xb.shape[0]
    x = bf16_dev(xb)
    idx, w = moeq.moe_route(None, to_dev(lg), cfg.experts, cfg.top_k)
    y = torch.empty((m, cfg.hidden), dtype=torch.float32, device=dev())
    if poison is not None:
        y.fill_(poison)
    step = chunk or m
    for s in range(0, m, step):
        e = min(m, s + step)
        moeq.moe_gather_qmm(L, x[s:e], idx[s:e], w[s:e], y=y[s:e])
    torch.cuda.synchronize()
    return y, idx, w


@pytest.mark.parametrize("m", [1, 7, 300, 1000])
def test_moe_gather_small_m_vs_oracle(m):
    cfg, host, L = _c4_layer()
    say(f"moe_gather_qmm M={m}")
    xb = synth.prefill_x_bf16(cfg, m)
    lg = synth.zipf_logits(cfg, m)
    y, idx, w = _prefill(cfg, L, xb, lg, poison=POISON[0])
    ridx, rw, _ = oracle.route(lg.astype(np.float64), cfg.top_k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    ref = oracle.moe_experts(host, bf16_bits_to_f32(xb), ridx, rw)
    err = rel_l2_rows(y.cpu().numpy(), ref)
    say(f"  max rel-L2 {err.max():.3e}")
    assert np.isfinite(y.cpu().numpy()).all()
    assert err.max() <= TOL


# With at most 4 (token, slot) pairs per expert on average (M * K <= 4 E:
# M <= 64 here) moe_gather_qmm streams every touched expert once per tile of
# two pairs through the batched decode kernels (fp32 activations widened
# from bf16) instead of staging 256-row MFMA tiles; M = 65 is the first
# count that takes the MFMA form.
@pytest.mark.parametrize("m", [16, 64, 65])
def test_moe_gather_light_form_both_sides_of_the_switch(m):
    cfg, host, L = _c4_layer()
    say(f"moe_gather_qmm M={m} (pairs {m * cfg.top_k}, experts {cfg.experts})")
    xb = synth.prefill_x_bf16(cfg, m)
    lg = synth.zipf_logits(cfg, m)
    y, idx, w = _prefill(cfg, L, xb, lg, poison=POISON[0])
    y2, _, _ = _prefill(cfg, L, xb, lg, poison=POISON[1])
    assert torch.equal(y, y2)                   # nothing unwritten, bitwise rerun
    ridx, rw, _ = oracle.route(lg.astype(np.float64), cfg.top_k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    ref = oracle.moe_experts(host, bf16_bits_to_f32(xb), ridx, rw)
    err = rel_l2_rows(y.cpu().numpy(), ref)
    say(f"  max rel-L2 {err.max():.3e}")
    assert err.max() <= (1e-4 if m <= 64 else TOL)   # the light form accumulates in fp32


def test_moe_gather_light_and_gemm_forms_share_one_workspace():
    # one workspace sized for the largest call serves both forms in any
    # order: the GEMM form's per-expert counts (2000 tokens: 16000 pairs, the
    # multi-block sort) must still be zero after light calls, and each
    # result equals the same call on a fresh workspace bit for bit
    cfg, host, L = _c4_layer()
    seq = [2000, 16, 2000, 64, 1, 2000]
    ws = moeq.workspace(L, max(seq), cfg.top_k, moeq.PATH_GATHER, dev())
    for i, m in enumerate(seq):
        say(f"shared workspace call {i}: M={m}")
        xb = synth.prefill_x_bf16(cfg, m)
        lg = to_dev(synth.zipf_logits(cfg, m))
        idx, w = moeq.moe_route(None, lg, cfg.experts, cfg.top_k)
        y = moeq.moe_gather_qmm(L, bf16_dev(xb), idx, w, ws=ws)
        yf = moeq.moe_gather_qmm(L, bf16_dev(xb), idx, w)
        torch.cuda.synchronize()
        assert torch.equal(y, yf)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_moe_gather_widths_off_the_tile_grid(bits):
    # H = 320 (not a multiple of the 256-column down tile) and I = 192 (not a
    # multiple of the 128 gate/up rows of a tile): ragged column tiles in
    # both GEMMs, and rows past the last expert's 256-row tile
    cfg = synth.scaled(synth.CONFIGS["c4"], hidden=320, inter=192, experts=8, top_k=2,
                       expert_bits=bits, router_bits=8, tokens=600, seed=40 + bits)
    host = synth.host_layer(cfg, 0, threads=16)
    L = moeq.MoELayer.from_host(host, dev())
    m = 600
    say(f"moe_gather_qmm H=320 I=192 bits={bits} M={m}")
    xb = synth.prefill_x_bf16(cfg, m)
    lg = synth.zipf_logits(cfg, m)
    y, idx, w = _prefill(cfg, L, xb, lg, poison=POISON[0])
    ridx, rw, _ = oracle.route(lg.astype(np.float64), cfg.top_k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    ref = oracle.moe_experts(host, bf16_bits_to_f32(xb), ridx, rw)
    err = rel_l2_rows(y.cpu().numpy(), ref)
    say(f"  max rel-L2 {err.max():.3e}")
    assert np.isfinite(y.cpu().numpy()).all()
    assert err.max() <= TOL


@pytest.mark.parametrize("m", [16068, 16384])
def test_c4_full_size_every_row_chunks_poison(m):
    cfg, host, L = _c4_layer()
    say(f"c4 prefill M={m}")
    xb = synth.prefill_x_bf16(cfg, m)
    lg = synth.zipf_logits(cfg, m)
    y1, idx, w = _prefill(cfg, L, xb, lg, poison=POISON[0])
    y2, _, _ = _prefill(cfg, L, xb, lg, poison=POISON[1])
    assert torch.equal(y1, y2)                  # nothing unwritten, bitwise rerun
    yc, _, _ = _prefill(cfg, L, xb, lg, chunk=2048, poison=POISON[0])
    assert torch.equal(y1, yc)                  # one-shot == 2048-token chunks
    # every token row against the oracle (the middle tiles of the heavy
    # Zipf experts included)
    ridx, rw, _ = oracle.route(lg.astype(np.float64), cfg.top_k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    loads = np.bincount(ridx.reshape(-1), minlength=cfg.experts)
    ref = oracle.moe_experts(host, bf16_bits_to_f32(xb), ridx, rw)
    err = rel_l2_rows(y1.cpu().numpy(), ref)
    say(f"  all {m} rows: max rel-L2 {err.max():.3e} (expert loads {loads.max()} .. {loads.min()} rows)")
    assert err.max() <= TOL


def _gqmm_case(n, bits=4, E=8, N=64, Kd=64, seed=0):
    q, s, b = synth.draw_matrix((77, bits, E, N), E * N, Kd, bits)
    host = {"q": q.reshape(E, N, -1), "scales": s.reshape(E, N, -1), "biases": b.reshape(E, N, -1),
            "batch": E, "rows": N, "cols": Kd, "bits": bits, "group_size": 64}
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits((rng.standard_normal((n, Kd)) * 0.5).astype(np.float32))
    ridx = np.sort(rng.integers(0, E, n)).astype(np.int32)
    return host, x, ridx


# the seam list: the row counts the pages print (clean and corrupt ones)
SEAMS = [32768, 32769, 32802, 32833, 32896, 40000, 40002]


@pytest.mark.parametrize("n", SEAMS)
@pytest.mark.parametrize("bits", [4, 8])
def test_gather_qmm_seams_have_no_bad_rows(n, bits):
    say(f"gather_qmm seam n={n} bits={bits}")
    host, xb, ridx = _gqmm_case(n, bits)
    W = moeq.QTensor.from_host(host, dev())
    x, r = bf16_dev(xb), to_dev(ridx)
    outs = []
    for p in POISON:
        out = torch.full((n, 64), p, dtype=torch.float32, device=dev())
        moeq.gather_qmm(W, x, r, sorted_indices=True, out=out)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    ref = oracle.gather_qmm(host, bf16_bits_to_f32(xb), ridx)
    got = outs[0].cpu().numpy()
    abs_err = np.abs(got - ref).max(axis=1)
    rel = rel_l2_rows(got, ref)
    # a row is bad when it is not finite or off by more than the bf16 tolerance;
    # the issue's unwritten rows are ~1e3x above the noise floor, so a relative
    # per-row criterion separates them from rounding at any weight scale
    bad = int((~np.isfinite(rel) | (rel > TOL)).sum())
    say(f"  max|err| {np.nanmax(abs_err):.4f} max rel-L2 {np.nanmax(rel):.2e} bad rows {bad}/{n}")
    assert bad == 0


def test_gather_qmm_unsorted_equals_sorted_and_invalid_rows_are_nan():
    host, xb, ridx = _gqmm_case(1000, 8, E=16, N=192, Kd=256, seed=3)
    W = moeq.QTensor.from_host(host, dev())
    perm = np.random.default_rng(0).permutation(1000)
    out_s = moeq.gather_qmm(W, bf16_dev(xb), to_dev(ridx), sorted_indices=True)
    out_u = moeq.gather_qmm(W, bf16_dev(xb[perm]), to_dev(ridx[perm]), sorted_indices=False)
    assert torch.equal(out_s[perm], out_u)
    bad = ridx.copy()
    bad[5] = 99
    out_b = moeq.gather_qmm(W, bf16_dev(xb), to_dev(bad)).cpu().numpy()
    assert np.isnan(out_b[5]).all() and np.isfinite(np.delete(out_b, 5, axis=0)).all()


def test_gather_qmm_sorted_indices_are_used_in_place():
    # sorted_indices=True takes each expert's run of rows as its tiles with no
    # sort; a row's result depends only on its own row and expert, so both
    # modes give the same bits
    E = 16
    host, xb, ridx = _gqmm_case(5000, 4, E=E, N=192, Kd=256, seed=5)
    W = moeq.QTensor.from_host(host, dev())
    x = bf16_dev(xb)
    out_s = moeq.gather_qmm(W, x, to_dev(ridx), sorted_indices=True)
    out_u = moeq.gather_qmm(W, x, to_dev(ridx), sorted_indices=False)
    assert torch.equal(out_s, out_u)
    ref = oracle.gather_qmm(host, bf16_bits_to_f32(xb), ridx)
    assert rel_l2_rows(out_s.cpu().numpy(), ref).max() <= TOL
    # out-of-range indices at the ends keep the order: those rows are NaN,
    # every other row is unchanged
    ends = ridx.copy()
    ends[:3] = -1
    ends[-5:] = E + 3
    out_e = moeq.gather_qmm(W, x, to_dev(ends), sorted_indices=True).cpu().numpy()
    bad = np.zeros(5000, bool)
    bad[:3] = bad[-5:] = True
    assert np.isnan(out_e[bad]).all()
    assert np.array_equal(out_e[~bad], out_u.cpu().numpy()[~bad])
    # indices claimed sorted that are not: the runs of two experts overlap,
    # so some rows fall outside the run of their own index and come out NaN;
    # every row that is not NaN was computed with its own expert
    un = ridx.copy()
    i, j = 100, 4000
    assert un[i] != un[j]
    un[i], un[j] = un[j], un[i]
    out_x = moeq.gather_qmm(W, x, to_dev(un), sorted_indices=True).cpu().numpy()
    ok = moeq.gather_qmm(W, x, to_dev(un), sorted_indices=False).cpu().numpy()
    nan = np.isnan(out_x).all(axis=1)
    say(f"  two rows swapped: {int(nan.sum())} of 5000 rows NaN")
    assert nan.any()
    assert np.array_equal(out_x[~nan], ok[~nan])
    assert not np.isnan(out_x[~nan]).any()
